// Fused small-batch decode-and-multiply (qdec_gemv), one launch.
//
// Work decomposition.  A workgroup (4 waves) owns one panel of 128 output
// rows and one chunk of Kc input columns; the four waves split the chunk's
// tile columns.  Per workgroup:
//   1. issue the loads of its code words (they stay in flight during 2-3);
//   2. input RHT restricted to the chunk: with Sylvester ordering
//      H_B = H_a (x) H_Kc, so the chunk's slice of H_B (s .* x) is H_Kc applied
//      to a +/- combination of the a = B/Kc strided sub-vectors -- B adds
//      plus a Kc-point FWHT instead of a full B-point transform;
//   3. build the LDS lookup table (HYB / VQ / NUQ);
//   4. stream the tiles: each 8-lane group decodes one 16x16 tile per step,
//      each lane 32 weights of two rows, accumulating with v_dot2_f32_f16;
//   5. reduce the four waves in LDS and add the panel's partial sums into
//      the fp32 accumulator z with device-scope atomic adds.
// A second, small kernel (gemv_finish_kernel) then applies the output RHT,
// the scale and the signs to z, writes fp16 y and re-zeroes z.  Splitting
// there keeps every cross-workgroup dependency at a kernel boundary: an
// in-kernel "last workgroup finishes" scheme needs an agent-scope release
// (an L2 write-back) in every workgroup, which measured far more expensive
// than the second launch.  With a precomputed x' (args.xr, written by the
// RHT kernel) step 2 is replaced by a plain load of the chunk's slice.
// Small-batch inference is memory bound ("QTIP: Quantization with Trellises
// and Incoherence Processing", "QTIP's contribution (W1)"), so the codes are
// read from HBM exactly once and every other operand stays on chip.
#pragma once

#include "qdec_device.hpp"
#include "qdec_internal.hpp"

namespace qdec {

constexpr int GEMV_THREADS = 256;
constexpr int GEMV_MAX_TPW = 8;   // tile columns per wave (Kc <= 512)

template <int CODE>
struct GemvTable {
  // LDS table copies (HYB, VQ); NUQ levels use one copy.
  static constexpr int COPIES = (CODE == HYB || CODE == VQ) ? 8 : 1;
};

template <int CODE, int K>
__host__ __device__ constexpr int gemv_table_words(int Q) {
  return CODE == HYB ? (2 << Q) * GemvTable<CODE>::COPIES
       : CODE == VQ ? (1 << (2 * K)) * GemvTable<CODE>::COPIES
       : CODE == NUQ ? (1 << K) : 0;
}

// LDS of one workgroup: region A (lookup table; also the scratch of the
// input RHT, the wave reduction and the output RHT), then x' as fp16 pairs,
// then (3INST) x' duplicated into (x, x) pairs.
template <int CODE, int K, int NB>
__host__ __device__ inline size_t gemv_regA_bytes(int Q, int Kc, int U) {
  size_t tab = (size_t)gemv_table_words<CODE, K>(Q) * 4;
  size_t rht = (size_t)(GEMV_THREADS * 8 + NB * padded_words(Kc)) * 4;
  size_t red = ((size_t)4 * 128 * NB + padded_words(128 * NB)) * 4;
  (void)U;
  size_t r = tab;
  if (rht > r) r = rht;
  if (red > r) r = red;
  return (r + 15) & ~(size_t)15;
}

template <int CODE, int K, int NB>
__host__ __device__ inline size_t gemv_lds_bytes(int Q, int Kc, int U) {
  return gemv_regA_bytes<CODE, K, NB>(Q, Kc, U) + (size_t)NB * Kc * 2 +
         (CODE == INST3 ? (size_t)NB * Kc * 4 : 0);
}

// K consecutive code words of one lane (16-byte aligned tile blocks).
template <int K>
__device__ __forceinline__ void load_words(const uint32_t* __restrict__ p, uint32_t* w) {
  if constexpr (K == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x; w[1] = v.y;
  } else if constexpr (K == 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else {
#pragma unroll
    for (int i = 0; i < K; ++i) w[i] = p[i];
  }
}

template <int CODE, int K, int NB>
__global__ __launch_bounds__(GEMV_THREADS) void gemv_kernel(GemvArgs a) {
  constexpr int V = code_V(CODE);
  constexpr int L = code_L(CODE, K);
  constexpr int KV = K * V;
  constexpr int COPIES = GemvTable<CODE>::COPIES;
  extern __shared__ __align__(16) uint32_t smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar math
  const int64_t m = a.L.m, n = a.L.n;
  const int npanels = (int)(m / 128);
  const int panel = blockIdx.x % npanels;
  const int chunk = blockIdx.x / npanels;
  const int Kc = a.Kc;
  const int64_t c0 = (int64_t)chunk * Kc;
  const int kcols = (int)((n - c0) < Kc ? (n - c0) : Kc);   // multiple of 16
  const int ntc = kcols >> 4;                                  // tile columns in chunk
  const int tpw = (ntc + 3) >> 2;
  const int tc_begin = wave * tpw;
  int tc_count = ntc - tc_begin;
  tc_count = tc_count < 0 ? 0 : (tc_count > tpw ? tpw : tc_count);

  // LDS carve-up
  const size_t regA_words = gemv_regA_bytes<CODE, K, NB>(a.L.Q, Kc, a.U) / 4;
  uint32_t* regA = smem;
  float* fA = reinterpret_cast<float*>(smem);
  uint32_t* xh = smem + regA_words;                 // [NB][Kc/2] fp16 pairs
  uint32_t* xd = xh + (size_t)NB * Kc / 2;           // [NB][Kc] duplicated (3INST)
  __shared__ float sx_sum[NB];

  // ---- 0. activations of the first batch column for the input RHT: issued
  // first, so the RHT's wait on them does not also wait on the (older,
  // slower) code loads -- vector-memory counters drain in issue order.
  const int Bi = a.L.had_in;
  const int arows = Kc < Bi ? Bi / Kc : 1;
  const int64_t rbase = Kc < Bi ? (c0 / Bi) * Bi : c0;
  const int jhi = Kc < Bi ? (int)((c0 - rbase) / Kc) : 0;
  const int CG = kcols >> 3;                       // groups of 8 columns
  const int RG = CG >= GEMV_THREADS ? 1 : GEMV_THREADS / CG;
  constexpr int MAXR = 8;   // arows / RG <= 8 (B_in <= 16384, RG = 2048 / kcols)
  const uint32_t* __restrict__ sgn = a.L.sign_in;
  uint4 xraw[MAXR];
  uint32_t xsb[MAXR];
  auto load_x_rows = [&](int c, int idx) {
    const int cg = idx % CG, rg = idx / CG;
    const uint16_t* __restrict__ xc = a.x + (int64_t)c * n;
#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
      const int ih = rg + r * RG;
      const int ihc = ih < arows ? ih : 0;   // row 0 is always in bounds
      const int64_t col = rbase + (int64_t)ihc * Kc + cg * 8;
      xraw[r] = *reinterpret_cast<const uint4*>(xc + col);
      xsb[r] = sgn ? (sgn[col >> 5] >> (col & 31)) : 0u;
    }
  };
  const bool x_hoisted = !a.xr && tid < CG * RG;
  if (x_hoisted) load_x_rows(0, tid);

  // ---- 1. issue the code loads ------------------------------------------
  const int64_t tiles_row = n >> 4;
  const uint32_t* __restrict__ codes = a.L.codes;
  uint32_t buf[GEMV_MAX_TPW][K];
#pragma unroll
  for (int j = 0; j < GEMV_MAX_TPW; ++j) {
    if (j < tc_count) {
      const int64_t tcg = (c0 >> 4) + tc_begin + j;
      const uint32_t* src = codes + ((panel * tiles_row + tcg) * 8) * (8 * K) + lane * K;
      load_words<K>(src, buf[j]);
    }
  }

  // ---- 2. input RHT of the chunk (or load the precomputed x') -------------
  if (a.xr) {
    for (int idx = tid; idx < NB * (Kc / 2); idx += GEMV_THREADS) {
      const int c = idx / (Kc / 2), p = idx % (Kc / 2);
      uint32_t v = 0;
      if (2 * p < kcols && c < a.b)
        v = *reinterpret_cast<const uint32_t*>(a.xr + (int64_t)c * n + c0 + 2 * p);
      xh[idx] = v;
      if constexpr (CODE == INST3) {
        xd[c * Kc + 2 * p] = (v & 0xFFFFu) * 0x10001u;
        xd[c * Kc + 2 * p + 1] = (v >> 16) * 0x10001u;
      }
    }
    __syncthreads();
  } else {
    float* red = fA;                                 // [RG][kcols]
    float* u = fA + GEMV_THREADS * 8;                // [NB][padded Kc]
    const int ustride = padded_words(Kc);
    for (int c = 0; c < NB; ++c) {
      if (c < a.b) {
        for (int idx = tid; idx < CG * RG; idx += GEMV_THREADS) {
          if (!(c == 0 && idx == tid && x_hoisted)) load_x_rows(c, idx);
          const int rg = idx / CG, cg = idx % CG;
          float part[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) part[e] = 0.f;
#pragma unroll
          for (int r = 0; r < MAXR; ++r) {
            const int ih = rg + r * RG;
            if (ih < arows) {
              const uint32_t chi = (uint32_t)__builtin_popcount((unsigned)(jhi & ih)) & 1u;
              const uint32_t rw[4] = {xraw[r].x, xraw[r].y, xraw[r].z, xraw[r].w};
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const float v = h2f((uint16_t)(rw[e >> 1] >> (16 * (e & 1))));
                const uint32_t neg = ((xsb[r] >> e) & 1u) ^ chi;
                part[e] += neg ? -v : v;
              }
            }
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) red[rg * kcols + cg * 8 + e] = part[e];
        }
        __syncthreads();
        for (int col = tid; col < kcols; col += GEMV_THREADS) {
          float s = 0.f;
          for (int rg = 0; rg < RG; ++rg) s += red[rg * kcols + col];
          u[c * ustride + pad_index(col)] = s;
        }
        __syncthreads();
      } else {
        for (int col = tid; col < Kc; col += GEMV_THREADS) u[c * ustride + pad_index(col)] = 0.f;
      }
    }
    __syncthreads();
    const int S = Kc < Bi ? Kc : Bi;
    // transform each batch column's slice: segments of S within [0, kcols)
    for (int c = 0; c < NB; ++c) {
      if (c < a.b) fwht_segments(u + c * ustride, kcols, S, tid, GEMV_THREADS);
    }
    const float rs = 1.0f / sqrtf((float)Bi);
    for (int idx = tid; idx < NB * (Kc / 2); idx += GEMV_THREADS) {
      const int c = idx / (Kc / 2), p = idx % (Kc / 2);
      uint32_t v = 0;
      if (2 * p < kcols && c < a.b) {
        const uint32_t lo = f2h_bits(u[c * ustride + pad_index(2 * p)] * rs);
        const uint32_t hi = f2h_bits(u[c * ustride + pad_index(2 * p + 1)] * rs);
        v = lo | (hi << 16);
      }
      xh[idx] = v;
      if constexpr (CODE == INST3) {
        xd[c * Kc + 2 * p] = (v & 0xFFFFu) * 0x10001u;
        xd[c * Kc + 2 * p + 1] = (v >> 16) * 0x10001u;
      }
    }
    __syncthreads();
  }
  if constexpr (CODE == MAD1) {
    // sum of the fp16 x' of the chunk, per batch column (bias removal)
    for (int c = wave; c < NB; c += 4) {
      float s = 0.f;
      for (int p = lane; p < Kc / 2; p += 64) {
        const uint32_t v = xh[c * (Kc / 2) + p];
        s += h2f((uint16_t)(v & 0xFFFFu)) + h2f((uint16_t)(v >> 16));
      }
      for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
      if (lane == 0) sx_sum[c] = s;
    }
  }

  // ---- 3. lookup table --------------------------------------------------
  if constexpr (CODE == HYB) fill_signed_table<COPIES>(regA, a.L.lut, a.L.Q, tid, GEMV_THREADS);
  if constexpr (CODE == VQ) fill_plain_table<COPIES>(regA, a.L.lut, 1 << (2 * K), tid, GEMV_THREADS);
  if constexpr (CODE == NUQ) fill_plain_table<1>(regA, a.L.lut, 1 << K, tid, GEMV_THREADS);
  __syncthreads();

  // ---- 4. stream the tiles ------------------------------------------------
  const int q = lane & 7, tl = lane >> 3;
  const uint32_t* tabc = regA + (lane & (COPIES - 1));
  const int qshift = a.L.qshift;
  float acc[2][NB];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int c = 0; c < NB; ++c) acc[r][c] = 0.f;

#pragma unroll
  for (int j = 0; j < GEMV_MAX_TPW; ++j) {
    if (j < tc_count) {
      const int tcl = tc_begin + j;   // tile column within the chunk
      uint32_t w[K + 1];
#pragma unroll
      for (int i = 0; i < K; ++i) w[i] = buf[j][i];
      w[K] = next_lane_word(w[0], lane);
      if constexpr (CODE == INST3) {
#pragma unroll
        for (int t = 0; t < 32; ++t) {
          const uint32_t s = window_at<L>(w, t * KV);
          const half2v val = as_h2(inst3_bits(s));
#pragma unroll
          for (int c = 0; c < NB; ++c)
            acc[t >> 4][c] = __builtin_amdgcn_fdot2(val, as_h2(xd[c * Kc + tcl * 16 + (t & 15)]),
                                                    acc[t >> 4][c], false);
        }
      } else {
        uint32_t xp[NB][8];
#pragma unroll
        for (int c = 0; c < NB; ++c) {
          const uint4* px = reinterpret_cast<const uint4*>(xh + c * (Kc / 2) + tcl * 8);
          const uint4 p0 = px[0], p1 = px[1];
          xp[c][0] = p0.x; xp[c][1] = p0.y; xp[c][2] = p0.z; xp[c][3] = p0.w;
          xp[c][4] = p1.x; xp[c][5] = p1.y; xp[c][6] = p1.z; xp[c][7] = p1.w;
        }
        if constexpr (V == 2) {
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            const uint32_t s = window_at<L>(w, t * KV);
            uint32_t pair;
            if constexpr (CODE == HYB) pair = tabc[hyb_signed_index(s, qshift) * COPIES];
            else pair = tabc[s * COPIES];
#pragma unroll
            for (int c = 0; c < NB; ++c)
              acc[t >> 3][c] = __builtin_amdgcn_fdot2(as_h2(pair), as_h2(xp[c][t & 7]),
                                                      acc[t >> 3][c], false);
          }
        } else if constexpr (CODE == MAD1) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const uint32_t s0 = window_at<L>(w, (2 * i) * KV);
            const uint32_t s1 = window_at<L>(w, (2 * i + 1) * KV);
            const uint32_t v0 = __builtin_amdgcn_sad_u8(mad1_lcg(s0), 0u, 0x6400u);
            const uint32_t v1 = __builtin_amdgcn_sad_u8(mad1_lcg(s1), 0u, 0x6400u);
            const uint32_t pv = v0 | (v1 << 16);
#pragma unroll
            for (int c = 0; c < NB; ++c)
              acc[i >> 3][c] = __builtin_amdgcn_fdot2(as_h2(pv), as_h2(xp[c][i & 7]),
                                                      acc[i >> 3][c], false);
          }
        } else {  // NUQ
          const int64_t row0 = (int64_t)panel * 128 + tl * 16 + 2 * q;
          const int64_t gcol = (c0 + tcl * 16) / a.L.group;
          const int64_t gstride = n / a.L.group;
          const float gs0 = h2f(a.L.gscale[row0 * gstride + gcol]);
          const float gs1 = h2f(a.L.gscale[(row0 + 1) * gstride + gcol]);
          float part[2][NB];
#pragma unroll
          for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int c = 0; c < NB; ++c) part[r][c] = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const uint32_t s0 = window_at<L>(w, (2 * i) * KV);
            const uint32_t s1 = window_at<L>(w, (2 * i + 1) * KV);
            const uint32_t pv = (regA[s0] & 0xFFFFu) | (regA[s1] << 16);
#pragma unroll
            for (int c = 0; c < NB; ++c)
              part[i >> 3][c] = __builtin_amdgcn_fdot2(as_h2(pv), as_h2(xp[c][i & 7]),
                                                       part[i >> 3][c], false);
          }
#pragma unroll
          for (int c = 0; c < NB; ++c) {
            acc[0][c] += gs0 * part[0][c];
            acc[1][c] += gs1 * part[1][c];
          }
        }
      }
    }
  }

  // ---- 5. reduce the waves, add into the fp32 accumulator -----------------
  __syncthreads();   // table region becomes the reduction buffer
  float* red = fA;   // [4 waves][128 rows][NB]
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int c = 0; c < NB; ++c) red[(wave * 128 + tl * 16 + 2 * q + r) * NB + c] = acc[r][c];
  __syncthreads();
  // the panel's sums, scaled, then the output Hadamard stages that stay
  // inside the panel (H_min(Bo,128) on 128 rows); the rest is the finisher's
  float* pv = fA + 4 * 128 * NB;   // entry (c, row) at pad_index(c * 128 + row)
  for (int idx = tid; idx < 128 * NB; idx += GEMV_THREADS) {
    const int row = idx / NB, c = idx % NB;
    float s = red[(0 * 128 + row) * NB + c] + red[(1 * 128 + row) * NB + c] +
              red[(2 * 128 + row) * NB + c] + red[(3 * 128 + row) * NB + c];
    if constexpr (CODE == MAD1) s -= MAD1_BIAS * sx_sum[c];
    pv[pad_index(c * 128 + row)] = s * a.out_mult;
  }
  __syncthreads();
  const int Bo = a.L.had_out;
  if (Bo > 1) fwht_bits(pv, 128 * NB, 0, Bo >= 128 ? 7 : 31 - __builtin_clz((unsigned)Bo), tid, GEMV_THREADS);
  for (int idx = tid; idx < 128 * NB; idx += GEMV_THREADS) {
    const int c = idx >> 7, row = idx & 127;
    if (c < a.b)
      __hip_atomic_fetch_add(a.z + (int64_t)c * m + (int64_t)panel * 128 + row, pv[pad_index(c * 128 + row)],
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int CODE, int K, int NB>
hipError_t launch_gemv_t(const GemvArgs& a, hipStream_t stream) {
  const size_t lds = gemv_lds_bytes<CODE, K, NB>(a.L.Q, a.Kc, a.U);
  static size_t have = 0;
  const hipError_t e =
      ensure_dynamic_lds(reinterpret_cast<const void*>(&gemv_kernel<CODE, K, NB>), lds, &have);
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)((a.L.m / 128) * a.nchunks);
  hipLaunchKernelGGL((gemv_kernel<CODE, K, NB>), dim3(grid), dim3(GEMV_THREADS), lds, stream, a);
  const hipError_t e1 = hipGetLastError();
  if (e1 != hipSuccess) return e1;
  return launch_gemv_finish(a, stream);
}

template <int CODE, int K>
hipError_t launch_gemv_k(const GemvArgs& a, hipStream_t stream) {
  if (a.b <= 1) return launch_gemv_t<CODE, K, 1>(a, stream);
  if (a.b <= 2) return launch_gemv_t<CODE, K, 2>(a, stream);
  if (a.b <= 4) return launch_gemv_t<CODE, K, 4>(a, stream);
  return launch_gemv_t<CODE, K, 8>(a, stream);
}

template <int CODE>
hipError_t launch_gemv_code(const GemvArgs& a, hipStream_t stream) {
  switch (a.L.k) {
    case 2: return launch_gemv_k<CODE, 2>(a, stream);
    case 3: return launch_gemv_k<CODE, 3>(a, stream);
    case 4: return launch_gemv_k<CODE, 4>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qdec
