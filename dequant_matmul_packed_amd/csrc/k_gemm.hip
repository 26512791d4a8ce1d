// Batched decode-and-multiply (qdec_gemm): decoded weights feed fp16 MFMA
// (v_mfma_f32_16x16x32_f16) with fp32 accumulation.
//
// A workgroup of 8 waves owns two panels of 128 output rows and NBT = 64
// batch columns (16 for small batches) and steps through K 64 input columns
// (4 tile columns) at a time.
// Wave w owns tile rows 2(w%4), 2(w%4)+1 of panel w/4 of the pair; per step
// it decodes its 8 tiles (2 tile rows x 4 tile columns) with the same
// 8-lanes-per-tile layout as the GEMV: lane q of tile t holds 32 weights,
// rows 2q and 2q+1 of the tile, as four 8-weight chunks of one row each.
// Placing tile t at (tile row t % 2, tile column t / 2) makes lanes l, l+16,
// l+32, l+48 hold the same weight row at four different k offsets -- the
// shape of an MFMA A fragment (lane l: row l % 16, k 8*(l/16) .. +8) under a
// fixed row permutation.  So every chunk is an A operand as decoded: the
// weights go from the code registers to the matrix cores without touching
// LDS.  The transformed activations X' (the B operand) are staged once per
// step in LDS (double buffered, 16-byte chunks XOR-swizzled by row) and read
// as fragments by every wave.  The lookup table of HYB/VQ/NUQ lives in LDS
// too, one per workgroup: the two panels share it, which leaves room for 16
// copies (a table per panel left room for half as many).
//
// The loop is software-pipelined: while step s is multiplied and step s+1
// decoded, the code words of steps s+2 .. s+5 and the X' of steps s+2 and
// s+3 are in flight.  With KSUB = 2 the workgroup holds two such 8-wave
// groups, each over one half of the K split's steps (see below).
#include "gemv_impl.hpp"
#include "qdec_device.hpp"
#include "qdec_internal.hpp"

namespace qdec {

// KSUB = 2 doubles the workgroup: two groups of 8 waves run the two halves
// of the K split's steps over the same two panels (one table, an X' buffer
// pair each) and add their sums in LDS at the end, so a layer that fills
// the chip with one such workgroup per CU writes half as many K-split
// slices (and the output transform reads half as many).
constexpr int GEMM_SUB_THREADS = 64 * GEMM_WAVES;
static_assert(GEMM_SUB_THREADS == 512, "at most one 16-byte X' chunk per thread and step (64 batch rows x 8 chunks)");

// LDS table copies: lane l reads copy l % COPIES.  HYB and VQ tables take
// GEMM_COPIES copies while two workgroups still fit a CU, else 8 (HYB with
// Q = 10 and 11); the NUQ levels and the pure lookup take one.
__host__ __device__ constexpr bool gemm_tabled(int code) { return code == HYB || code == HYB1 || code == VQ; }
template <int CODE, int KV, int COPIES>
__host__ __device__ constexpr int gemm_table_words(int Q) {
  return (CODE == HYB || CODE == HYB1) ? (2 << Q) * COPIES
       : CODE == VQ ? (1 << KV) * COPIES
       : CODE == NUQ ? (1 << KV)
       : CODE == LUT ? (1 << 15) : 0;   // LUT: 2^16 fp16 values, two per word
}

__device__ __forceinline__ int gemm_swz(int r, int k) {
  return r * 128 + ((((k >> 3) ^ (r & 7)) << 4) | ((k & 7) << 1));
}

// LDS: lookup table, then B[KSUB][2][NBT batch][64 k] fp16 (double
// buffered per K half); with KSUB = 2 the space is reused at the end for the
// second half's sums (8 waves x 2 NBT / 4 values x 64 lanes fp32).
template <int CODE, int KV, int COPIES>
__host__ __device__ inline size_t gemm_table_bytes(int Q) {
  return ((size_t)gemm_table_words<CODE, KV, COPIES>(Q) * 4 + 15) & ~(size_t)15;
}
template <int CODE, int KV, int COPIES, int KSUB, int NBT>
__host__ __device__ inline size_t gemm_lds_bytes(int Q) {
  const size_t main = gemm_table_bytes<CODE, KV, COPIES>(Q) + (size_t)KSUB * 2 * (NBT * 128);
  const size_t red = KSUB > 1 ? (size_t)GEMM_WAVES * (NBT / 2) * 64 * 4 : 0;
  return main > red ? main : red;
}

// Four waves per SIMD (at most 128 VGPRs): two 8-wave workgroups or one of
// 16 waves per CU; the pure lookup's 128 KiB table leaves room for one
// 8-wave workgroup, so it may use twice as many.
template <int CODE, int KV, int COPIES, int KSUB, int NBT>
// The hot scalar arguments lead (16 dwords, preloaded into SGPRs at wave
// launch: the table fill and the first code loads need no round trip to
// the argument segment); the NUQ group scales stay in the struct.
#define QDEC_GEMM_PARAMS                                                                            \
  const uint32_t *codes_, const uint32_t *lut_, const uint16_t *xr_, float *z_, int m_, int n_, int Q_, \
      int qshift_, int b_, int ksplit_, int mz_, int row0_
#define QDEC_GEMM_ARGS(a)                                                                        \
  (a).L.codes, (a).L.lut, (a).xr, (a).z, (int)(a).L.m, (int)(a).L.n, (a).L.Q, (a).L.qshift, (a).b, (a).ksplit, \
      (int)(a).mz, (int)(a).row0
__global__ __launch_bounds__(GEMM_SUB_THREADS * KSUB, CODE == LUT ? 2 : 4) void gemm_kernel(QDEC_GEMM_PARAMS,
                                                                                         GemmArgs a) {
  static_assert(NBT == 16 || NBT == 64, "batch tile of 16 or 64 columns");
  constexpr int GEMM_THREADS = GEMM_SUB_THREADS * KSUB;
  constexpr int NB4 = NBT / 16;                      // 16-column MFMA blocks
  using G = LaneGeom<CODE, KV>;
  constexpr int NW = G::NW;
  extern __shared__ __align__(16) uint32_t smem[];
  uint32_t* tab = smem;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wvall = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ksub = wvall / GEMM_WAVES;               // K half of this wave (0 with KSUB = 1)
  const int wv = wvall % GEMM_WAVES;                 // wave within its 8-wave group
  const int stid = tid % GEMM_SUB_THREADS;           // thread within its group
  const int wave = wv & 3;                           // wave within its panel
  char* Bs = reinterpret_cast<char*>(smem) + gemm_table_bytes<CODE, KV, COPIES>(Q_) + ksub * 2 * (NBT * 128);
  const int q = lane & 7, t = lane >> 3;           // tile t of the wave, lane q in it
  const int tr = t & 1, tc = t >> 1;                 // tile row / column within the step
  const int64_t m = (int64_t)m_, n = (int64_t)n_;
  const int npanels = (int)(m / 128);
  const int ngroups = (npanels + GEMM_PANELS - 1) / GEMM_PANELS;
  const int panel = (blockIdx.x % ngroups) * GEMM_PANELS + (wv >> 2);
  const bool panel_ok = panel < npanels;             // wave-uniform: the last group may be short
  const int split = blockIdx.x / ngroups;
  const int n0 = blockIdx.y * NBT;
  const int ntc = (int)(n >> 4);                    // tile columns (steps of 4)
  const int niter = (ntc + 3) >> 2;
  // steps per K split, a multiple of 4 (the loop's unroll) where possible;
  // with KSUB = 2 each half takes `steps` of them, also a multiple of 4,
  // the first half from s0 and the second from s0 + steps (steps past the
  // split's end read zeros)
  const int per = (((niter + ksplit_ - 1) / ksplit_) + 3) & ~3;
  const int sp0 = split * per;
  const int sp1 = (sp0 + per) < niter ? (sp0 + per) : niter;
  const int steps = sp0 < sp1 ? ((((sp1 - sp0) + KSUB - 1) / KSUB) + 3) & ~3 : 0;   // workgroup-uniform
  const int it0 = sp0 + ksub * steps;                // this half's first step
  const int it1 = (it0 + steps) < sp1 ? (it0 + steps) : sp1;   // its live end (<= it0: none live)

  if constexpr (CODE == HYB) fill_signed_table<COPIES>(tab, lut_, Q_, tid, GEMM_THREADS);
  if constexpr (CODE == HYB1) fill_signed_table<COPIES, 0x8000u>(tab, lut_, Q_, tid, GEMM_THREADS);
  if constexpr (CODE == LUT) fill_plain_table<1>(tab, lut_, 1 << 15, tid, GEMM_THREADS);
  if constexpr (CODE == VQ) fill_plain_table<COPIES>(tab, lut_, 1 << KV, tid, GEMM_THREADS);
  if constexpr (CODE == NUQ) fill_plain_table<1>(tab, lut_, 1 << KV, tid, GEMM_THREADS);
  const uint32_t* tabc = tab + (lane & (COPIES - 1));

  // Every global load goes through a buffer resource and is issued
  // unconditionally: a step beyond the split's range, a tile column beyond
  // n, or a batch row beyond b gets an out-of-range offset and reads zeros
  // without touching memory.  With no branch around them, the compiler
  // waits for exactly the loads a step needs.  A load of step it is live
  // while it is below the lane's limit (32-bit offsets: a panel's codes and
  // X' stay far below 4 GiB).
  // Code words of this lane: tile (row 2*wave + tr, column 4*it + tc) of the
  // panel; a panel's tile column is 8 tiles of TILE_WORDS words, and lane q
  // reads NW words from word lane_word(q) of its tile.
  constexpr uint32_t TB = 4u * G::TILE_WORDS;       // bytes per tile
  const auto crs = make_rsrc(codes_ + (int64_t)(panel_ok ? panel : 0) * ntc * (8 * G::TILE_WORDS),
                             panel_ok ? (uint32_t)ntc * (8u * TB) : 0u);
  const int itc = (ntc - tc + 3) >> 2 < it1 ? (ntc - tc + 3) >> 2 : it1;   // 4 it + tc < ntc
  const uint32_t cbase = (uint32_t)tc * (8u * TB) + (uint32_t)(2 * wave + tr) * TB + 4u * G::lane_word(q);
  // NUQ group scales of the lane's rows 2q, 2q+1 (fp16 [m][n/group]); a
  // group spans gpt tile columns
  const int gstride = CODE == NUQ ? (int)(n / a.L.group) : 0;
  const int gpt = CODE == NUQ ? a.L.group >> 4 : 1;
  const int grow0 = (int)(int64_t)row0_ + panel * 128 + (2 * wave + tr) * 16 + 2 * q;
  const auto grs = make_rsrc(a.L.gscale, CODE == NUQ ? (uint32_t)((int64_t)mz_ * gstride * 2) : 0u);
  auto load_codes = [&](int it, uint32_t* w) {
    const bool ok = it < itc;
    buf_load_words<NW>(crs, ok ? cbase + (uint32_t)it * (32u * TB) : BUF_OFF, w);
    if constexpr (CODE == NUQ) {
      const int g = (it * 4 + tc) / gpt;
      w[NW] = buf_load_u16(grs, ok ? (uint32_t)((grow0 * gstride + g) * 2) : BUF_OFF);
      w[NW + 1] = buf_load_u16(grs, ok ? (uint32_t)(((grow0 + 1) * gstride + g) * 2) : BUF_OFF);
    }
  };
  // X' chunk of this thread: batch row n0 + (stid >> 3), k chunk stid & 7;
  // chunk ch of step it is column 64 it + 8 ch.  A 16-row tile has 128
  // chunks: the group's waves 2 .. 7 stage nothing.
  const bool xmine = stid < NBT * 8;                 // wave-uniform
  const auto xrs = make_rsrc(xr_, (uint32_t)(b_ * n * 2));
  const int xrow = n0 + (stid >> 3), xch = stid & 7;
  const int xlim = (int)((n - xch * 8 + 63) >> 6);
  const int itx = (xmine && xrow < b_) ? (xlim < it1 ? xlim : it1) : 0;
  const uint32_t xbase = (uint32_t)(((int64_t)(xrow < b_ ? xrow : 0) * n + xch * 8) * 2);
  auto load_x = [&](int it, uint4& xv) {
    xv = buf_load_u4(xrs, it < itx ? xbase + (uint32_t)it * 128u : BUF_OFF);
  };
  auto store_x = [&](const uint4& xv, int buf) {
    if (!xmine) return;
    *reinterpret_cast<uint4*>(Bs + buf * (NBT * 128) + gemm_swz(stid >> 3, xch * 8)) = xv;
  };

  float4v acc[2][NB4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NB4; ++j) acc[i][j] = float4v{0.f, 0.f, 0.f, 0.f};

  // Decode step `it` (the lane's 32 weights) into the four A operands:
  // operand 2*ra + h is the chunk (tile row 2q + ra, columns 8h .. 8h+7).
  // A tile column beyond n (only in the last step) is decoded from zero
  // words and then zeroed, so no value of the table can leak into the sums.
  auto decode = [&](int it, const uint32_t* wc, uint4* A) {
    uint32_t w[NW + 1];
#pragma unroll
    for (int i = 0; i < NW; ++i) w[i] = wc[i];
    lane_words_ready<CODE, KV>(w, lane);
    float gs[2] = {0.f, 0.f};
    if constexpr (CODE == NUQ) {
      gs[0] = h2f((uint16_t)wc[NW]);
      gs[1] = h2f((uint16_t)wc[NW + 1]);
    }
    uint32_t out[16];
    lane_decode_exact<CODE, KV, COPIES>(w, tabc, qshift_, gs, out);
    if (it * 4 + 3 >= ntc || it >= it1) {             // wave-uniform: the ragged or padding step
      const bool live = it < it1 && it * 4 + tc < ntc;
#pragma unroll
      for (int i = 0; i < 16; ++i) out[i] = live ? out[i] : 0u;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) A[j] = make_uint4(out[4 * j], out[4 * j + 1], out[4 * j + 2], out[4 * j + 3]);
  };
  // B fragments of the step in LDS buffer `buf`, then the 4 NB4 MFMAs: the
  // B operand for column half h holds X'[batch][16*(l/16) + 8h .. +8].
  auto mma = [&](const uint4* A, int buf) {
    const char* Bt = Bs + buf * (NBT * 128);
    half8v bf[2][NB4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int nb = 0; nb < NB4; ++nb)
        bf[h][nb] = *reinterpret_cast<const half8v*>(Bt + gemm_swz(nb * 16 + (lane & 15), 16 * (lane >> 4) + 8 * h));
#pragma unroll
    for (int ra = 0; ra < 2; ++ra)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const half8v af = __builtin_bit_cast(half8v, A[2 * ra + h]);
#pragma unroll
        for (int nb = 0; nb < NB4; ++nb)
          acc[ra][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[h][nb], acc[ra][nb], 0, 0, 0);
      }
  };

  // Software pipeline, unrolled by 4.  At the top of step s: A[s % 2] holds
  // the decoded weights of s, LDS buffer s % 2 holds X'(s), code set
  // c[(s + j) % 4] holds the code words of step s + j (j = 1..3), and X' set
  // x[(s + 1) % 2] holds X'(s + 1).  A step multiplies s, then decodes s+1
  // (its VALU work overlaps the MFMAs in flight), stages X'(s+1) in the other
  // LDS buffer and refills the freed registers with steps s+5 and s+3.
  constexpr int CW = CODE == NUQ ? NW + 2 : NW;      // code words (+ NUQ scales) per step
  uint32_t c0[CW], c1[CW], c2[CW], c3[CW];
  uint4 x0, x1;
  uint4 A0[4], A1[4];
  auto one = [&](int s, const uint4* Acur, uint4* Anext, uint32_t* cnext, uint4& xnext, int buf) {
    __syncthreads();
    mma(Acur, buf);
    decode(s + 1, cnext, Anext);          // past the range: decoded, never used
    load_codes(s + 5, cnext);
    store_x(xnext, buf ^ 1);
    load_x(s + 3, xnext);
  };
  if (steps > 0) {                                   // workgroup-uniform: every wave meets every barrier
    load_codes(it0, c0);
    load_codes(it0 + 1, c1);
    load_codes(it0 + 2, c2);
    load_codes(it0 + 3, c3);
    load_x(it0, x0);
    load_x(it0 + 1, x1);
    __syncthreads();                                  // lookup table ready
    store_x(x0, 0);
    load_x(it0 + 2, x0);
    decode(it0, c0, A0);
    load_codes(it0 + 4, c0);
    // whole groups of 4 steps; steps past it1 read zeros and add nothing
    for (int s = it0; s < it0 + steps; s += 4) {
      one(s, A0, A1, c1, x1, 0);
      one(s + 1, A1, A0, c2, x0, 1);
      one(s + 2, A0, A1, c3, x1, 0);
      one(s + 3, A1, A0, c0, x0, 1);
    }
  }

  // ---- epilogue.  acc[ra][nb] holds D[i][j], i = 4*(lane/16) + e, j = lane % 16:
  // MFMA row i is weight row 16*(i/8) + 2*(i%8) + ra of the wave's 32 rows.
  // With KSUB = 2 the second half hands its sums to the first through LDS
  // (the table and X' are dead by then).  Each K split writes its own slice
  // of the workspace (no atomics); the output-RHT kernel sums the slices.
  if constexpr (KSUB > 1) {
    float* red = reinterpret_cast<float*>(smem) + (wv * (8 * NB4)) * 64 + lane;
    __syncthreads();
    if (ksub == 1) {
#pragma unroll
      for (int ra = 0; ra < 2; ++ra)
#pragma unroll
        for (int nb = 0; nb < NB4; ++nb)
#pragma unroll
          for (int e = 0; e < 4; ++e) red[((ra * NB4 + nb) * 4 + e) * 64] = acc[ra][nb][e];
    }
    __syncthreads();
    if (ksub == 1) return;
#pragma unroll
    for (int ra = 0; ra < 2; ++ra)
#pragma unroll
      for (int nb = 0; nb < NB4; ++nb)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[ra][nb][e] += red[((ra * NB4 + nb) * 4 + e) * 64];
  }
  if (!panel_ok) return;
  float* zs = z_ + (int64_t)split * b_ * (int64_t)mz_;
#pragma unroll
  for (int nb = 0; nb < NB4; ++nb) {
    const int bb = n0 + nb * 16 + (lane & 15);
    if (bb >= b_) continue;
    float* zrow = zs + (int64_t)bb * (int64_t)mz_ + (int64_t)row0_ + (int64_t)panel * 128 + 32 * wave;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * (lane >> 4) + e;
      const int r = 16 * (i >> 3) + 2 * (i & 7);
      *reinterpret_cast<float2*>(zrow + r) = make_float2(acc[0][nb][e], acc[1][nb][e]);
    }
  }
}

template <int CODE, int KV, int COPIES, int KSUB, int NBT>
static hipError_t launch_gemm_k(const GemmArgs& a, hipStream_t stream) {
  const size_t lds = gemm_lds_bytes<CODE, KV, COPIES, KSUB, NBT>(a.L.Q);
  static LdsLimit have;
  const hipError_t e =
      ensure_dynamic_lds(reinterpret_cast<const void*>(&gemm_kernel<CODE, KV, COPIES, KSUB, NBT>), lds, &have);
  if (e != hipSuccess) return e;
  const int64_t ngroups = (a.L.m / 128 + GEMM_PANELS - 1) / GEMM_PANELS;
  dim3 grid((unsigned)(ngroups * a.ksplit), (unsigned)((a.b + NBT - 1) / NBT));
  hipLaunchKernelGGL((gemm_kernel<CODE, KV, COPIES, KSUB, NBT>), grid, dim3(GEMM_SUB_THREADS * KSUB), lds, stream,
                     QDEC_GEMM_ARGS(a), a);
  return hipGetLastError();
}
// built: 64-column tiles with one or two K halves, 16-column tiles with one
template <int CODE, int KV, int COPIES>
static hipError_t launch_gemm_c(const GemmArgs& a, hipStream_t stream) {
  if (a.nbt == 16) return a.ksub == 1 ? launch_gemm_k<CODE, KV, COPIES, 1, 16>(a, stream) : hipErrorInvalidValue;
  if (a.nbt != 64) return hipErrorInvalidValue;
  if (a.ksub == 2) return launch_gemm_k<CODE, KV, COPIES, 2, 64>(a, stream);
  return launch_gemm_k<CODE, KV, COPIES, 1, 64>(a, stream);
}

template <int CODE, int KV>
static hipError_t launch_gemm_t(const GemmArgs& a, hipStream_t stream) {
  if constexpr (gemm_tabled(CODE)) {
    if (gemm_lds_bytes<CODE, KV, GEMM_COPIES, 1, 64>(a.L.Q) <= GEMM_LDS_BYTES / GEMM_WG_PER_CU)
      return launch_gemm_c<CODE, KV, GEMM_COPIES>(a, stream);
    return launch_gemm_c<CODE, KV, 8>(a, stream);
  } else {
    return launch_gemm_c<CODE, KV, 1>(a, stream);
  }
}

template <int CODE>
static hipError_t launch_gemm_code(const GemmArgs& a, hipStream_t stream) {
#define QDEC_GEMM_KV(KV)                                                       \
  case KV:                                                                    \
    if constexpr (kv_built(CODE, KV)) return launch_gemm_t<CODE, KV>(a, stream); \
    break;
  switch (a.L.kv) {
    QDEC_GEMM_KV(2) QDEC_GEMM_KV(3) QDEC_GEMM_KV(4) QDEC_GEMM_KV(5)
    QDEC_GEMM_KV(6) QDEC_GEMM_KV(7) QDEC_GEMM_KV(8)
    default: break;
  }
#undef QDEC_GEMM_KV
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream) {
  switch (a.L.code) {
    case HYB: return launch_gemm_code<HYB>(a, stream);
    case MAD1: return launch_gemm_code<MAD1>(a, stream);
    case INST3: return launch_gemm_code<INST3>(a, stream);
    case NUQ: return launch_gemm_code<NUQ>(a, stream);
    case VQ: return launch_gemm_code<VQ>(a, stream);
    case HYB1: return launch_gemm_code<HYB1>(a, stream);
    case LUT: return launch_gemm_code<LUT>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qdec
