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
//   5. reduce the four waves in LDS and store the panel's partial sums (after
//      the output-Hadamard stages inside the panel) into the chunk's own fp32
//      slice of the workspace: plain stores, no atomics.
// A second, small kernel (gemv_finish_kernel) then adds the slices in chunk
// order -- a fixed summation order, so the output is reproducible bit for
// bit -- applies the rest of the output RHT, the scale and the signs, and
// writes fp16 y.  Splitting there keeps every cross-workgroup dependency at
// a kernel boundary: an in-kernel "last workgroup finishes" scheme needs an
// agent-scope release (an L2 write-back) in every workgroup, which measured
// far more expensive than the second launch.  With more than one batch column the input RHT
// runs once, in the RHT kernel, and step 2 is a plain load of the chunk's
// slice of x' (args.xr): the chunk transform costs b x B_in loads and adds
// in every workgroup, which at b = 8 outweighs the extra launch.  All
// global loads go through buffer resources and are issued unconditionally
// (switched off by their offsets), so they stay in flight together.
// Small-batch inference is memory bound ("QTIP: Quantization with Trellises
// and Incoherence Processing", "QTIP's contribution (W1)"), so the codes are
// read from HBM exactly once and every other operand stays on chip.
#pragma once

#include <type_traits>

#include "qdec_device.hpp"
#include "qdec_internal.hpp"

namespace qdec {

constexpr int GEMV_THREADS = 256;
// Every load slot costs address-unit issue time even when switched off, so
// the kernel comes in variants sized to the layer: PF is the depth of the
// code ring (tile columns in flight per wave: 2, 4 and 8 for chunks of at
// most 128, 256 and more columns); SL ("small loads") sizes the activation
// rows (2 per thread, enough for B_in <= 4096) and the table words (2 per
// thread, 2^Q <= 512) instead of 8 and 8.

template <int CODE>
struct GemvTable {
  // LDS table copies (HYB, VQ); NUQ levels use one copy.
  static constexpr int COPIES = (CODE == HYB || CODE == HYB1 || CODE == VQ) ? 8 : 1;
};

template <int CODE, int KV>
__host__ __device__ constexpr int gemv_table_words(int Q) {
  return (CODE == HYB || CODE == HYB1) ? (2 << Q) * GemvTable<CODE>::COPIES
       : CODE == VQ ? (1 << KV) * GemvTable<CODE>::COPIES
       : CODE == NUQ ? (1 << KV)
       : CODE == LUT ? (1 << 15) : 0;   // LUT: 2^16 fp16 values, two per word
}

// The GEMV's NUQ table holds level pairs: with no trellis overlap (L = kV)
// the indices of weights 2i and 2i + 1 are one 2k-bit field of the stream,
// so entry e = (s0 << k) | s1 is (level s0, level s1), one lookup per pair,
// in NUQ_PAIR_COPIES copies; the 2^k levels are staged after it.  (The group
// scales multiply the pair sums afterwards, so the pairs stay plain levels.)
constexpr int NUQ_PAIR_COPIES = 8;
template <int CODE, int KV>
__host__ __device__ constexpr int gemv_lut_words(int Q) {
  return CODE == NUQ ? (1 << (2 * KV)) * NUQ_PAIR_COPIES + (1 << KV) : gemv_table_words<CODE, KV>(Q);
}

// LDS of one workgroup: region A (lookup table; also the scratch of the
// input RHT, the wave reduction and the output RHT), then x' as fp16 pairs,
// then (3INST) x' duplicated into (x, x) pairs.
template <int CODE, int KV, int NB>
__host__ __device__ inline size_t gemv_regA_bytes(int Q, int Kc, int U) {
  size_t tab = (size_t)gemv_lut_words<CODE, KV>(Q) * 4;
  size_t rht = (size_t)(GEMV_THREADS * 8 + NB * padded_words(Kc)) * 4;
  size_t red = (size_t)4 * 128 * NB * 4;
  (void)U;
  size_t r = tab;
  if (rht > r) r = rht;
  if (red > r) r = red;
  return (r + 15) & ~(size_t)15;
}

// Full chunks of at most GEMV_WAVE_RHT_MAX columns (one batch column) take
// the wave-level input RHT, whose exchange area holds 4 x Kc fp32.  Up to
// GEMV_WRED_SEP_MAX columns that area has LDS of its own and the table is
// filled before the transform; wider chunks borrow the table region and
// fill the table after it.
constexpr int GEMV_WAVE_RHT_MAX = 512;
constexpr int GEMV_WRED_SEP_MAX = 256;
template <int NB>
__host__ __device__ inline size_t gemv_wred_bytes(int Kc) {
  return (NB == 1 && Kc <= GEMV_WRED_SEP_MAX) ? (size_t)4 * Kc * 4 : 0;
}
template <int CODE, int KV, int NB>
__host__ __device__ inline size_t gemv_lds_bytes(int Q, int Kc, int U) {
  return gemv_regA_bytes<CODE, KV, NB>(Q, Kc, U) + (size_t)NB * Kc * 2 +
         (CODE == INST3 ? (size_t)NB * Kc * 4 : 0) + gemv_wred_bytes<NB>(Kc);
}

// KVB > 0: a half-TCQ layer in one launch.  Workgroups [0, grid_a) take the
// first row part (width KV, codes a.L.codes, a.L.m rows), the others the
// second (width KVB, a.codes_b, a.m_b rows starting at row a.row0_b); the
// part is uniform per workgroup, and the tile loop is built for each width.
// The hot scalar arguments lead (14 dwords, preloaded into SGPRs at wave
// launch, so the table, activation and code loads need no round trip to the
// argument segment); the rest stay in the struct.
#define QDEC_GEMV_PARAMS                                                                              \
  const uint32_t *lut_, const uint32_t *codes_, const uint16_t *x_, const uint32_t *sgin_, int n_, int m_, \
      int Kc_, int Q_, int hin_, int grida_
#define QDEC_GEMV_ARGS(a)                                                                             \
  (a).L.lut, (a).L.codes, (a).x, (a).L.sign_in, (int)(a).L.n, (int)(a).L.m, (a).Kc, (a).L.Q, (a).L.had_in, (a).grid_a
template <int CODE, int KV, int NB, int PF, bool SL, bool XR, int KVB = 0>
__global__ __launch_bounds__(GEMV_THREADS) void gemv_kernel(QDEC_GEMV_PARAMS, GemvArgs a) {
  using G = LaneGeom<CODE, KV>;
  using GB = LaneGeom<CODE, KVB ? KVB : KV>;
  constexpr int V = G::V;
  constexpr int L = G::L;
  constexpr int NW = G::NW > GB::NW ? G::NW : GB::NW;   // ring words per slot
  constexpr int COPIES = GemvTable<CODE>::COPIES;
  extern __shared__ __align__(16) uint32_t smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar math
  const bool second = KVB != 0 && (int)blockIdx.x >= grida_;
  const int bid = second ? (int)blockIdx.x - grida_ : (int)blockIdx.x;
  // 32-bit index math (m, n <= 2^20): no 64-bit division in the prologue
  const int m = second ? (int)a.m_b : m_, n = n_;
  const int64_t row0 = second ? a.row0_b : a.row0;
  const int npanels = m >> 7;
  const int panel = bid % npanels;
  const int chunk = bid / npanels;
  const int Kc = Kc_;
  const int c0 = chunk * Kc;
  const int kcols = (int)((n - c0) < Kc ? (n - c0) : Kc);   // multiple of 16
  const int ntc = kcols >> 4;                                  // tile columns in chunk
  const int tpw = (ntc + 3) >> 2;
  const int tc_begin = wave * tpw;
  int tc_count = ntc - tc_begin;
  tc_count = tc_count < 0 ? 0 : (tc_count > tpw ? tpw : tc_count);

  // LDS carve-up
  const size_t regA_words = gemv_regA_bytes<CODE, KV, NB>(Q_, Kc, a.U) / 4;
  uint32_t* regA = smem;
  float* fA = reinterpret_cast<float*>(smem);
  uint32_t* xh = smem + regA_words;                 // [NB][Kc/2] fp16 pairs
  uint32_t* xd = xh + (size_t)NB * Kc / 2;           // [NB][Kc] duplicated (3INST)
  const bool wred_sep = NB == 1 && Kc <= GEMV_WRED_SEP_MAX;
  float* wred = wred_sep ? reinterpret_cast<float*>(xd + (CODE == INST3 ? (size_t)NB * Kc : 0)) : fA;   // [4][Kc]
  __shared__ float sx_sum[NB];

  // ---- 0. (b = 1) the activations of the input RHT: issued first, so the
  // RHT's wait on them does not also wait on the (slower) code loads --
  // vector-memory counters drain in issue order.  With b > 1, x' comes
  // precomputed (args.xr) and step 2 loads the chunk's slice of it instead.
  const int Bi = hin_;
  const int arows = Kc < Bi ? Bi / Kc : 1;
  const int rbase = Kc < Bi ? (c0 / Bi) * Bi : c0;
  const int jhi = Kc < Bi ? (c0 - rbase) / Kc : 0;
  const int CG = kcols >> 3;                       // groups of 8 columns
  const int RG = CG >= GEMV_THREADS ? 1 : GEMV_THREADS / CG;
  constexpr int MAXR = XR ? 1 : (SL ? 2 : 8);   // arows / RG = B_in / 2048 (B_in <= 16384)
  uint4 xraw[MAXR];
  uint32_t xsb[MAXR];
  // the lookup table's words, requested up front too: word tid + 256 i
  // (HYB: 2^Q <= 256 TW words; VQ 2^(2k) <= 256; NUQ 2^k <= 16)
  constexpr int TW = (CODE == HYB || CODE == HYB1) ? (SL ? 2 : 8) : 1;
  const int nlut = (CODE == HYB || CODE == HYB1) ? (1 << Q_)
                 : (CODE == VQ || CODE == NUQ) ? (1 << KV) : 0;   // LUT: filled below
  uint32_t lw[TW];
  {
    const auto lrs = make_rsrc(lut_, (uint32_t)nlut * 4u);
#pragma unroll
    for (int i = 0; i < TW; ++i) {
      const int e = tid + i * GEMV_THREADS;
      lw[i] = buf_load_u32(lrs, e < nlut ? (uint32_t)e * 4u : BUF_OFF);
    }
  }
  if constexpr (!XR) {
    // x as a buffer of one row; the sign bits as a buffer that is empty when
    // the layer has no input signs (its loads then read zero: all signs +1).
    // xsb[r] is the whole sign word: the group's 8 signs start at bit
    // (cg * 8) & 31, as rbase and Kc are multiples of 64.
    const auto xrs = make_rsrc(x_, (uint32_t)(n * 2));
    const auto srs = make_rsrc(sgin_, sgin_ ? (uint32_t)(((n + 31) >> 5) * 4) : 0u);
    const int cg = tid % CG, rg = tid / CG;
#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
      const int ih = rg + r * RG;
      const int64_t col = rbase + (int64_t)ih * Kc + cg * 8;
      const bool ok = tid < CG * RG && ih < arows;
      xraw[r] = buf_load_u4(xrs, ok ? (uint32_t)(col * 2) : BUF_OFF);
      xsb[r] = buf_load_u32(srs, ok ? (uint32_t)((col >> 5) * 4) : BUF_OFF);
    }
    __builtin_amdgcn_sched_barrier(0);   // keep these ahead of the code loads
  }

  // ---- 1. issue the code loads ------------------------------------------
  // A buffer over this panel's tile columns of the chunk (each 8 tiles of
  // TILE_WORDS words); the wave's tile columns tc_begin .. tc_begin+tc_count-1
  // stream through a PF-deep ring of registers, the first PF requested here.
  // Lane q of tile row tl loads NW words from word lane_word(q) of its tile.
  // (with two parts the ring slots take the wider part's word count; the
  // narrower one's extra words are unused, or read zero past the buffer)
  const uint32_t TWS = second ? (uint32_t)GB::TILE_WORDS : (uint32_t)G::TILE_WORDS;
  const uint32_t TCB = 8u * 4u * TWS;                 // bytes per tile column
  const int64_t tiles_row = n >> 4;
  const uint32_t* pchunk = (second ? a.codes_b : codes_) + ((int64_t)panel * tiles_row + (c0 >> 4)) * (8 * TWS);
  const auto crs = make_rsrc(pchunk, (uint32_t)ntc * TCB);
  const uint32_t lane_off = (uint32_t)(lane >> 3) * (4u * TWS) +
                            4u * (second ? GB::lane_word(lane & 7) : G::lane_word(lane & 7));
  auto code_off = [&](int j) -> uint32_t {
    return j < tc_count ? (uint32_t)(tc_begin + j) * TCB + lane_off : BUF_OFF;
  };
  uint32_t buf[PF][NW];
#pragma unroll
  for (int j = 0; j < PF; ++j) buf_load_words<NW>(crs, code_off(j), buf[j]);
  // NUQ: the fp16 group scales of the lane's two rows ride in the same ring
  const int gstride = CODE == NUQ ? n / a.L.group : 0;
  const int64_t grow0 = row0 + (int64_t)panel * 128 + (lane >> 3) * 16 + 2 * (lane & 7);
  const auto grs = make_rsrc(a.L.gscale, CODE == NUQ ? (uint32_t)(a.mz * gstride * 2) : 0u);
  uint32_t gsr[PF][2];
  auto gs_load = [&](int j, uint32_t* g) {
    if constexpr (CODE == NUQ) {
      const bool ok = j < tc_count;
      const int gcol = (c0 + (tc_begin + j) * 16) / a.L.group;
      g[0] = buf_load_u16(grs, ok ? (uint32_t)((grow0 * gstride + gcol) * 2) : BUF_OFF);
      g[1] = buf_load_u16(grs, ok ? (uint32_t)(((grow0 + 1) * gstride + gcol) * 2) : BUF_OFF);
    } else {
      (void)j; g[0] = g[1] = 0u;
    }
  };
#pragma unroll
  for (int j = 0; j < PF; ++j) gs_load(j, gsr[j]);
  __builtin_amdgcn_sched_barrier(0);   // all requests out before any wait

  // The LDS lookup table: HYB entry e and its sign-flipped twin e + 2^Q
  // (the flip covers both halves at V = 2, the low half at V = 1); VQ / NUQ
  // as stored; each replicated COPIES times (entry e of copy c at word
  // e * COPIES + c).  The pure lookup (LUT) copies its 128 KiB as it is, in
  // rounds of 8 x 16 bytes per thread.
  auto fill_table = [&]() {
    if constexpr (CODE == NUQ) {
      // the levels (lw[0] of threads below 2^k), then every pair from them
      constexpr int NP = 1 << (2 * KV);
      uint32_t* lv = regA + NP * NUQ_PAIR_COPIES;
      if (tid < nlut) lv[tid] = lw[0];
      __syncthreads();
      for (int e = tid; e < NP; e += GEMV_THREADS) {
        const uint32_t v = (lv[e >> KV] & 0xFFFFu) | (lv[e & ((1 << KV) - 1)] << 16);
#pragma unroll
        for (int c = 0; c < NUQ_PAIR_COPIES; ++c) regA[e * NUQ_PAIR_COPIES + c] = v;
      }
    }
    if constexpr (CODE == HYB || CODE == HYB1 || CODE == VQ) {
      constexpr uint32_t FLIP = CODE == HYB ? 0x80008000u : 0x00008000u;
#pragma unroll
      for (int i = 0; i < TW; ++i) {
        const int e = tid + i * GEMV_THREADS;
        if (e < nlut) {
#pragma unroll
          for (int c = 0; c < COPIES; ++c) {
            regA[e * COPIES + c] = lw[i];
            if constexpr (CODE == HYB || CODE == HYB1) regA[(e + nlut) * COPIES + c] = lw[i] ^ FLIP;
          }
        }
      }
    }
    if constexpr (CODE == LUT) {
      const auto trs = make_rsrc(lut_, (1u << 15) * 4u);
      for (int r0 = 0; r0 < (1 << 13); r0 += 8 * GEMV_THREADS) {   // 2^13 chunks of 16 bytes
        uint4 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = buf_load_u4(trs, (uint32_t)(r0 + tid + i * GEMV_THREADS) * 16u);
#pragma unroll
        for (int i = 0; i < 8; ++i) reinterpret_cast<uint4*>(regA)[r0 + tid + i * GEMV_THREADS] = v[i];
      }
    }
  };

  // ---- 2. input RHT of the chunk (b = 1), or load the precomputed x' ------
  // A full chunk of at most 512 columns takes the wave-level transform (one
  // barrier; with a separate exchange area the table is filled before it).
  const bool wave_rht = !XR && Kc <= GEMV_WAVE_RHT_MAX && kcols == Kc;
  if constexpr (XR) {
    // NB * Kc / 2 <= 2048 fp16 pairs: at most 8 per thread, all loads first
    const auto xrr = make_rsrc(a.xr, (uint32_t)(a.b * n * 2));
    const int hp = Kc >> 1, lhp = __builtin_ctz((unsigned)hp);
    uint32_t v[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int idx = tid + r * GEMV_THREADS;
      const int c = idx >> lhp, p = idx & (hp - 1);
      const bool ok = idx < NB * hp && 2 * p < kcols && c < a.b;
      v[r] = buf_load_u32(xrr, ok ? (uint32_t)(((int64_t)c * n + c0 + 2 * p) * 2) : BUF_OFF);
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int idx = tid + r * GEMV_THREADS;
      const int c = idx >> lhp, p = idx & (hp - 1);
      if (idx < NB * hp) {
        xh[idx] = v[r];
        if constexpr (CODE == INST3) {
          xd[c * Kc + 2 * p] = (v[r] & 0xFFFFu) * 0x10001u;
          xd[c * Kc + 2 * p + 1] = (v[r] >> 16) * 0x10001u;
        }
      }
    }
    __syncthreads();
  } else if (wave_rht) {
    // u = the +/- combination of the arows strided rows, as below, but with
    // lane = rgw * CG + cg: the row groups of a wave are summed with lane
    // shuffles, the four waves through LDS, and H on segments of
    // S = min(Kc, B_in) runs on the 8 values of a lane (index bits 0-2) and
    // across the CG lanes (bits 3 and up).  Every wave ends with the whole
    // x' of the chunk and stores the part its own tiles read.
    if (wred_sep) fill_table();
    const int cg = lane % CG;
    float part[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) part[e] = 0.f;
#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
      if (r * RG >= arows) break;                    // uniform: no thread has row r (its loads read zeros)
      const int ih = tid / CG + r * RG;
      const uint32_t chi = (uint32_t)__builtin_popcount((unsigned)(jhi & ih)) & 1u;
      const uint32_t rw[4] = {xraw[r].x, xraw[r].y, xraw[r].z, xraw[r].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = h2f((uint16_t)(rw[e >> 1] >> (16 * (e & 1))));
        const uint32_t neg = ((xsb[r] >> (((cg * 8) & 31) + e)) & 1u) ^ chi;
        part[e] += neg ? -v : v;
      }
    }
    for (int msk = CG; msk < 64; msk <<= 1) {
#pragma unroll
      for (int e = 0; e < 8; ++e) part[e] += __shfl_xor(part[e], msk, 64);
    }
    if (lane < CG) {
      float4* dst = reinterpret_cast<float4*>(wred + (wave * CG + cg) * 8);
      dst[0] = make_float4(part[0], part[1], part[2], part[3]);
      dst[1] = make_float4(part[4], part[5], part[6], part[7]);
    }
    __syncthreads();   // the partials of all waves, and the table
    float u[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) u[e] = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float4* src = reinterpret_cast<const float4*>(wred + (w * CG + cg) * 8);
      const float4 p0 = src[0], p1 = src[1];
      u[0] += p0.x; u[1] += p0.y; u[2] += p0.z; u[3] += p0.w;
      u[4] += p1.x; u[5] += p1.y; u[6] += p1.z; u[7] += p1.w;
    }
    const int S = Kc < Bi ? Kc : Bi;
#pragma unroll
    for (int h = 1; h < 8; h <<= 1) {
      if (h < S) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (!(e & h)) {
            const float x0 = u[e], x1 = u[e + h];
            u[e] = x0 + x1;
            u[e + h] = x0 - x1;
          }
        }
      }
    }
    for (int msk = 1; msk < (S >> 3); msk <<= 1) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float o = __shfl_xor(u[e], msk, 64);
        u[e] = (cg & msk) ? o - u[e] : u[e] + o;
      }
    }
    const float rs = 1.0f / sqrtf((float)Bi);
    uint32_t hp[4];
    float hsum = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = f2h_bits(u[2 * e] * rs), hi = f2h_bits(u[2 * e + 1] * rs);
      hp[e] = lo | (hi << 16);
      hsum += h2f((uint16_t)lo) + h2f((uint16_t)hi);
    }
    // this wave's tiles read column groups [2 tc_begin, 2 (tc_begin + tc_count))
    if (lane < CG && cg >= 2 * tc_begin && cg < 2 * (tc_begin + tc_count)) {
      *reinterpret_cast<uint4*>(xh + cg * 4) = make_uint4(hp[0], hp[1], hp[2], hp[3]);
      if constexpr (CODE == INST3) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xd[cg * 8 + 2 * e] = (hp[e] & 0xFFFFu) * 0x10001u;
          xd[cg * 8 + 2 * e + 1] = (hp[e] >> 16) * 0x10001u;
        }
      }
    }
    if constexpr (CODE == MAD1) {
      for (int msk = 1; msk < CG; msk <<= 1) hsum += __shfl_xor(hsum, msk, 64);
      if (wave == 0 && lane == 0) sx_sum[0] = hsum;   // read after the reduction's barriers
    }
  } else {
    // u = the +/- combination of the arows strided rows (row ih enters with
    // the sign H_arows[jhi][ih]), then H on segments of min(Kc, B_in)
    // Every thread takes part: rows that do not exist were loaded as zeros,
    // and thread tid writes red[8 tid .. 8 tid + 7] (rg * kcols + cg * 8 =
    // 8 tid), inside the 2048 words of the region; rows rg >= RG are unread.
    float* red = fA;                                 // [RG][kcols]
    float* u = fA + GEMV_THREADS * 8;                // [padded Kc]
    {
      const int rg = tid / CG, cg = tid % CG;
      float part[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) part[e] = 0.f;
#pragma unroll
      for (int r = 0; r < MAXR; ++r) {
        if (r * RG >= arows) break;                  // uniform: no thread has row r (its loads read zeros)
        const int ih = rg + r * RG;
        const uint32_t chi = (uint32_t)__builtin_popcount((unsigned)(jhi & ih)) & 1u;
        const uint32_t rw[4] = {xraw[r].x, xraw[r].y, xraw[r].z, xraw[r].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = h2f((uint16_t)(rw[e >> 1] >> (16 * (e & 1))));
          const uint32_t neg = ((xsb[r] >> (((cg * 8) & 31) + e)) & 1u) ^ chi;
          part[e] += neg ? -v : v;
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) red[rg * kcols + cg * 8 + e] = part[e];
    }
    __syncthreads();
    for (int col = tid; col < kcols; col += GEMV_THREADS) {
      float sum = 0.f;
      for (int rg = 0; rg < RG; ++rg) sum += red[rg * kcols + col];
      u[pad_index(col)] = sum;
    }
    __syncthreads();
    fwht_segments(u, kcols, Kc < Bi ? Kc : Bi, tid, GEMV_THREADS);
    const float rs = 1.0f / sqrtf((float)Bi);
    for (int p = tid; p < Kc / 2; p += GEMV_THREADS) {
      uint32_t v = 0;
      if (2 * p < kcols) {
        const uint32_t lo = f2h_bits(u[pad_index(2 * p)] * rs);
        const uint32_t hi = f2h_bits(u[pad_index(2 * p + 1)] * rs);
        v = lo | (hi << 16);
      }
      xh[p] = v;
      if constexpr (CODE == INST3) {
        xd[2 * p] = (v & 0xFFFFu) * 0x10001u;
        xd[2 * p + 1] = (v >> 16) * 0x10001u;
      }
    }
    __syncthreads();
  }
  if (CODE == MAD1 && !wave_rht) {
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
  if (!wave_rht || !wred_sep) {
    if (wave_rht) __syncthreads();   // every wave is done with the exchange area the table overwrites
    fill_table();
    __syncthreads();
  }

  // ---- 4. stream the tiles ------------------------------------------------
  constexpr int TCOPIES = CODE == NUQ ? NUQ_PAIR_COPIES : COPIES;
  const uint32_t* tabc = regA + (lane & (TCOPIES - 1));
  const int qshift = a.L.qshift;
  float acc[2][NB];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int c = 0; c < NB; ++c) acc[r][c] = 0.f;

  auto stream_tiles = [&](auto kx) {
    constexpr int KX = decltype(kx)::value;
    constexpr int NWX = LaneGeom<CODE, KX>::NW;
    for (int j0 = 0; j0 < tc_count; j0 += PF) {
#pragma unroll
    for (int jj = 0; jj < PF; ++jj) {
      const int j = j0 + jj;
      uint32_t w[NWX + 1];
#pragma unroll
      for (int i = 0; i < NWX; ++i) w[i] = buf[jj][i];
      const uint32_t g0 = gsr[jj][0], g1 = gsr[jj][1];
      (void)g0; (void)g1;
      // refill this ring slot with the tile column PF ahead (unconditionally:
      // past the wave's last column the load is switched off by its offset)
      buf_load_words<NW>(crs, code_off(j + PF), buf[jj]);
      gs_load(j + PF, gsr[jj]);
      if (j < tc_count) {
        const int tcl = tc_begin + j;   // tile column within the chunk
        lane_words_ready<CODE, KX>(w, lane);
        if constexpr (CODE == INST3) {
#pragma unroll
          for (int t = 0; t < 32; ++t) {
            const uint32_t s = window_at<L>(w, t * KX);
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
            uint32_t pairs[16];
            if constexpr (CODE == HYB) {
              hyb_lane_pairs<KX, COPIES>(w, tabc, qshift, pairs);
            } else {
#pragma unroll
              for (int t = 0; t < 16; ++t) pairs[t] = tabc[window_at<L>(w, t * KX) * COPIES];
            }
#pragma unroll
            for (int t = 0; t < 16; ++t) {
#pragma unroll
              for (int c = 0; c < NB; ++c)
                acc[t >> 3][c] = __builtin_amdgcn_fdot2(as_h2(pairs[t]), as_h2(xp[c][t & 7]),
                                                        acc[t >> 3][c], false);
            }
          } else if constexpr (CODE == MAD1) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const uint32_t s0 = window_at<L>(w, (2 * i) * KX);
              const uint32_t s1 = window_at<L>(w, (2 * i + 1) * KX);
              const uint32_t v0 = __builtin_amdgcn_sad_u8(mad1_lcg(s0), 0u, 0x6400u);
              const uint32_t v1 = __builtin_amdgcn_sad_u8(mad1_lcg(s1), 0u, 0x6400u);
              const uint32_t pv = v0 | (v1 << 16);
#pragma unroll
              for (int c = 0; c < NB; ++c)
                acc[i >> 3][c] = __builtin_amdgcn_fdot2(as_h2(pv), as_h2(xp[c][i & 7]),
                                                        acc[i >> 3][c], false);
            }
          } else if constexpr (CODE == HYB1 || CODE == LUT) {
            // one table value per state (V = 1): two states per fp16 pair
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const uint32_t s0 = CODE == HYB1 ? window_raw<L>(w, (2 * i) * KX) : window_at<L>(w, (2 * i) * KX);
              const uint32_t s1 = CODE == HYB1 ? window_raw<L>(w, (2 * i + 1) * KX) : window_at<L>(w, (2 * i + 1) * KX);
              uint32_t pv;
              if constexpr (CODE == HYB1) {
                pv = (tabc[hyb_signed_index(s0, qshift) * COPIES] & 0xFFFFu) |
                     (tabc[hyb_signed_index(s1, qshift) * COPIES] << 16);
              } else {
                const uint16_t* t16 = reinterpret_cast<const uint16_t*>(regA);
                pv = (uint32_t)t16[s0] | ((uint32_t)t16[s1] << 16);
              }
#pragma unroll
              for (int c = 0; c < NB; ++c)
                acc[i >> 3][c] = __builtin_amdgcn_fdot2(as_h2(pv), as_h2(xp[c][i & 7]),
                                                        acc[i >> 3][c], false);
            }
          } else {  // NUQ
            const float gs0 = h2f((uint16_t)g0);
            const float gs1 = h2f((uint16_t)g1);
            float part[2][NB];
#pragma unroll
            for (int r = 0; r < 2; ++r)
#pragma unroll
              for (int c = 0; c < NB; ++c) part[r][c] = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              // the 2k-bit field of weights 2i, 2i + 1 indexes their level pair
              const uint32_t e = window_at<2 * L>(w, (2 * i) * KX);
              const uint32_t pv = tabc[e * NUQ_PAIR_COPIES];
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
    }
  };
  if constexpr (KVB == 0) {
    stream_tiles(std::integral_constant<int, KV>{});
  } else {
    if (second) stream_tiles(std::integral_constant<int, KVB>{});
    else stream_tiles(std::integral_constant<int, KV>{});
  }

  // ---- 5. reduce the waves, store the chunk's slice -------------------------
  // Lane l of every wave holds partial sums of panel rows 2l and 2l + 1.
  // One wave per batch column adds the four waves' partials (in wave order)
  // and applies the output Hadamard stages that stay inside the panel
  // (H_min(Bo,128) on the 128 rows: row bit 0 in registers, bits 1-6 across
  // lanes), then stores the panel's sums into the chunk's slice of z; the
  // cross-panel stages, the scale and the signs are the finisher's.
  __syncthreads();   // the table region becomes the reduction buffer
  float* red = fA;   // [4 waves][NB][128 rows]
#pragma unroll
  for (int c = 0; c < NB; ++c)
    *reinterpret_cast<float2*>(red + (wave * NB + c) * 128 + 2 * lane) = make_float2(acc[0][c], acc[1][c]);
  __syncthreads();
  const int Bo = a.L.had_out;
  const int hbits = Bo >= 128 ? 7 : 31 - __builtin_clz((unsigned)Bo);
  for (int c = wave; c < NB; c += 4) {
    if (c < a.b) {
      float v0 = 0.f, v1 = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float2 p = *reinterpret_cast<const float2*>(red + (w * NB + c) * 128 + 2 * lane);
        v0 += p.x;
        v1 += p.y;
      }
      if constexpr (CODE == MAD1) {
        v0 -= MAD1_BIAS * sx_sum[c];
        v1 -= MAD1_BIAS * sx_sum[c];
      }
      if (hbits > 0) {
        const float t = v0 + v1;
        v1 = v0 - v1;
        v0 = t;
      }
      for (int msk = 1; msk < (1 << (hbits > 0 ? hbits - 1 : 0)); msk <<= 1) {
        const float o0 = __shfl_xor(v0, msk, 64), o1 = __shfl_xor(v1, msk, 64);
        const bool hi = lane & msk;
        v0 = hi ? o0 - v0 : v0 + o0;
        v1 = hi ? o1 - v1 : v1 + o1;
      }
      float* zr = a.z + ((int64_t)chunk * a.b + c) * a.mz + row0 + (int64_t)panel * 128 + 2 * lane;
      *reinterpret_cast<float2*>(zr) = make_float2(v0, v1);
    }
  }
}

template <int CODE, int KV, int NB, int PF, bool SL, bool XR, int KVB = 0>
hipError_t launch_gemv_v(const GemvArgs& a, hipStream_t stream) {
  const size_t lds = gemv_lds_bytes<CODE, KV, NB>(a.L.Q, a.Kc, a.U);
  static LdsLimit have;
  const hipError_t e =
      ensure_dynamic_lds(reinterpret_cast<const void*>(&gemv_kernel<CODE, KV, NB, PF, SL, XR, KVB>), lds, &have);
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)((a.L.m / 128 + (KVB ? a.m_b / 128 : 0)) * a.nchunks);
  hipLaunchKernelGGL((gemv_kernel<CODE, KV, NB, PF, SL, XR, KVB>), dim3(grid), dim3(GEMV_THREADS), lds, stream,
                     QDEC_GEMV_ARGS(a), a);
  return hipGetLastError();
}

// XR: x' comes precomputed (args.xr, always with more than one batch
// column; with one column for layers whose chunk transforms would cost
// more than the separate transform's launch).
template <int CODE, int KV, int NB, bool XR, int KVB = 0>
hipError_t launch_gemv_x(const GemvArgs& a, hipStream_t stream) {
  const bool sl = (XR || a.L.had_in <= 4096) && ((CODE != HYB && CODE != HYB1) || a.L.Q <= 9);
  if (a.Kc <= 128 && sl) return launch_gemv_v<CODE, KV, NB, 2, true, XR, KVB>(a, stream);
  if (a.Kc <= 256 && sl) return launch_gemv_v<CODE, KV, NB, 4, true, XR, KVB>(a, stream);
  if (sl) return launch_gemv_v<CODE, KV, NB, 8, true, XR, KVB>(a, stream);
  return launch_gemv_v<CODE, KV, NB, 8, false, XR, KVB>(a, stream);
}

// A two-part (half-TCQ) layer at one batch column with its x transform in
// the workgroups, in one launch: the width pairs one half-bit apart of HYB
// at V = 2.  Returns hipErrorNotSupported for the pairs not built here.
template <int CODE>
hipError_t launch_gemv_two_parts(const GemvArgs& a, int kvb, hipStream_t stream) {
  if constexpr (CODE == HYB) {
    const int kv = a.L.kv;
#define QDEC_GEMV_PAIR(A, B) \
    if (kv == A && kvb == B) return launch_gemv_x<CODE, A, 1, false, B>(a, stream);
    QDEC_GEMV_PAIR(4, 5) QDEC_GEMV_PAIR(5, 4) QDEC_GEMV_PAIR(5, 6) QDEC_GEMV_PAIR(6, 5)
    QDEC_GEMV_PAIR(6, 7) QDEC_GEMV_PAIR(7, 6) QDEC_GEMV_PAIR(7, 8) QDEC_GEMV_PAIR(8, 7)
#undef QDEC_GEMV_PAIR
  }
  (void)a; (void)kvb; (void)stream;
  return hipErrorNotSupported;
}

template <int CODE, int KV, int NB>
hipError_t launch_gemv_t(const GemvArgs& a, hipStream_t stream) {
  if constexpr (NB == 1) {
    if (!a.xr) return launch_gemv_x<CODE, KV, 1, false>(a, stream);
  }
  return launch_gemv_x<CODE, KV, NB, true>(a, stream);
}

template <int CODE, int KV>
hipError_t launch_gemv_k(const GemvArgs& a, hipStream_t stream) {
  if (a.b <= 1) return launch_gemv_t<CODE, KV, 1>(a, stream);
  if (a.b <= 2) return launch_gemv_t<CODE, KV, 2>(a, stream);
  if (a.b <= 4) return launch_gemv_t<CODE, KV, 4>(a, stream);
  return launch_gemv_t<CODE, KV, 8>(a, stream);
}

// The kernels of one code for the step widths in [KV_LO, KV_HI] that it is
// built for (one source file may take a sub-range).
template <int CODE, int KV_LO = 2, int KV_HI = 8>
hipError_t launch_gemv_code(const GemvArgs& a, hipStream_t stream) {
#define QDEC_GEMV_KV(KV)                                                          \
  case KV:                                                                       \
    if constexpr (kv_built(CODE, KV) && KV >= KV_LO && KV <= KV_HI)             \
      return launch_gemv_k<CODE, KV>(a, stream);                                 \
    break;
  switch (a.L.kv) {
    QDEC_GEMV_KV(2) QDEC_GEMV_KV(3) QDEC_GEMV_KV(4) QDEC_GEMV_KV(5)
    QDEC_GEMV_KV(6) QDEC_GEMV_KV(7) QDEC_GEMV_KV(8)
    default: break;
  }
#undef QDEC_GEMV_KV
  return hipErrorInvalidValue;
}

}  // namespace qdec
