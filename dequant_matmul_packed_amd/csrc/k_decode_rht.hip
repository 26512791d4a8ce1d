// qdec_decode_tile and qdec_rht kernels.
#include "gemv_impl.hpp"
#include "qdec_device.hpp"
#include "qdec_internal.hpp"

namespace qdec {

// ---------------------------------------------------------------------------
// Tile decode (the bit-exact parity surface).  32 tiles per workgroup, one
// 8-lane group per tile, the same window extraction and value maps the
// matmul kernels use.
template <int CODE, int KV>
__global__ __launch_bounds__(256) void decode_tile_kernel(DecodeArgs a) {
  using G = LaneGeom<CODE, KV>;
  constexpr int NW = G::NW;
  constexpr int COPIES = GemvTable<CODE>::COPIES;
  extern __shared__ __align__(16) uint32_t tab[];
  const int tid = threadIdx.x, lane = tid & 63, q = tid & 7;
  if constexpr (CODE == HYB) fill_signed_table<COPIES>(tab, a.L.lut, a.L.Q, tid, 256);
  if constexpr (CODE == HYB1) fill_signed_table<COPIES, 0x8000u>(tab, a.L.lut, a.L.Q, tid, 256);
  if constexpr (CODE == LUT) fill_plain_table<1>(tab, a.L.lut, 1 << 15, tid, 256);
  if constexpr (CODE == VQ) fill_plain_table<COPIES>(tab, a.L.lut, 1 << KV, tid, 256);
  if constexpr (CODE == NUQ) fill_plain_table<1>(tab, a.L.lut, 1 << KV, tid, 256);
  __syncthreads();

  // tiles [first, first + count) of this part; lane q of a tile reads NW
  // words from word lane_word(q) (a switched-off load past the range)
  const int64_t tile = a.first + (int64_t)blockIdx.x * 32 + (tid >> 3);
  const bool valid = tile < a.first + a.count;
  const auto crs = make_rsrc(a.L.codes + a.first * G::TILE_WORDS, (uint32_t)(a.count * G::TILE_WORDS * 4));
  uint32_t w[NW + 1];
  buf_load_words<NW>(crs, valid ? (uint32_t)((tile - a.first) * G::TILE_WORDS + G::lane_word(q)) * 4u : BUF_OFF, w);
  lane_words_ready<CODE, KV>(w, lane);
  if (!valid) return;

  float gs[2] = {0.f, 0.f};
  if constexpr (CODE == NUQ) {
    // storage index -> tile (R, C): panels of 8 tile rows, column by column
    const int64_t per_row = a.L.n >> 4;
    const int64_t r8 = tile & 7, rest = tile >> 3;
    const int64_t C = rest % per_row, R = (rest / per_row) * 8 + r8;
    const int64_t gstride = a.L.n / a.L.group;
    const int64_t g = (C * 16) / a.L.group;
#pragma unroll
    for (int r = 0; r < 2; ++r) gs[r] = h2f(a.L.gscale[(R * 16 + 2 * q + r) * gstride + g]);
  }
  uint32_t out[16];
  lane_decode_exact<CODE, KV, COPIES>(w, tab + (lane & (COPIES - 1)), a.L.qshift, gs, out);
  uint4* dst = reinterpret_cast<uint4*>(a.out + (tile - a.first) * 256 + q * 32);
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
}

template <int CODE, int KV>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  const size_t lds = (size_t)gemv_table_words<CODE, KV>(a.L.Q) * 4 + 16;
  static LdsLimit have;
  const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&decode_tile_kernel<CODE, KV>), lds, &have);
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)((a.count + 31) / 32);
  hipLaunchKernelGGL((decode_tile_kernel<CODE, KV>), dim3(grid), dim3(256), lds, stream, a);
  return hipGetLastError();
}

template <int CODE>
static hipError_t launch_decode_code(const DecodeArgs& a, hipStream_t stream) {
#define QDEC_DEC_KV(KV)                                                          \
  case KV:                                                                      \
    if constexpr (kv_built(CODE, KV)) return launch_decode_t<CODE, KV>(a, stream); \
    break;
  switch (a.L.kv) {
    QDEC_DEC_KV(2) QDEC_DEC_KV(3) QDEC_DEC_KV(4) QDEC_DEC_KV(5)
    QDEC_DEC_KV(6) QDEC_DEC_KV(7) QDEC_DEC_KV(8)
    default: break;
  }
#undef QDEC_DEC_KV
  return hipErrorInvalidValue;
}

hipError_t launch_decode_tile(const DecodeArgs& a, hipStream_t stream) {
  if (a.count <= 0) return hipSuccess;
  switch (a.L.code) {
    case HYB: return launch_decode_code<HYB>(a, stream);
    case MAD1: return launch_decode_code<MAD1>(a, stream);
    case INST3: return launch_decode_code<INST3>(a, stream);
    case NUQ: return launch_decode_code<NUQ>(a, stream);
    case VQ: return launch_decode_code<VQ>(a, stream);
    case HYB1: return launch_decode_code<HYB1>(a, stream);
    case LUT: return launch_decode_code<LUT>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------------------
// Randomized Hadamard transform of independent row blocks: one workgroup per
// (row, block), the block held in LDS in fp32.
//   mode 0: out = mult * H (s .* in);   mode 1: out = s .* (mult * H in)
// ("Incoherence Processing (W2)": the RHT is invertible up to rounding.)
// An fp32 input may be the sum of `nsum` slices `sum_stride` apart (the
// K-split partial sums of the batched path).

// Blocks of 1, 2 or 4 values: one value per thread.
__global__ __launch_bounds__(256) void rht_tiny_kernel(RhtArgs a) {
  extern __shared__ __align__(16) float buf[];
  const int tid = threadIdx.x;
  const int B = a.block;
  const int64_t nblk = a.n / B;
  const int64_t row = blockIdx.x / nblk;
  const int64_t c0 = (blockIdx.x % nblk) * B;
  const int64_t off = row * a.n + c0;
  for (int i = tid; i < B; i += 256) {
    float v = 0.f;
    if (a.in_f32) {
      for (int sl = 0; sl < a.nsum; ++sl) v += ((const float*)a.in)[sl * a.sum_stride + off + i];
    } else {
      v = h2f(((const uint16_t*)a.in)[off + i]);
    }
    if (a.mode == 0) v *= sign_of(a.signs, c0 + i);
    buf[pad_index(i)] = v;
  }
  __syncthreads();
  if (B > 1) fwht_segments(buf, B, B, tid, 256);
  for (int i = tid; i < B; i += 256) {
    float v = buf[pad_index(i)] * a.mult;
    if (a.mode == 1) v *= sign_of(a.signs, c0 + i);
    if (a.out_f32) ((float*)a.out)[off + i] = v;
    else ((uint16_t*)a.out)[off + i] = f2h_bits(v);
  }
}

// Blocks of 8 or more: chunks of 8 consecutive values, chunk tid + 256 j for
// j < J (J = B / 2048 rounded up to a power of two).  Every load goes
// through a buffer resource and is issued unconditionally -- a chunk or a
// slice that does not exist has an out-of-range offset and reads zeros --
// so a thread's loads (all of them for fp16 input; SU slices at a time for
// summed fp32 input) are in flight together.  The 3 butterfly stages inside
// a chunk run in registers, the rest in padded LDS.
template <bool IN_F32, int J>
__global__ __launch_bounds__(256) void rht_kernel(RhtArgs a) {
  extern __shared__ __align__(16) float buf[];
  constexpr int SU = IN_F32 ? (J >= 4 ? 1 : 4 / J) : 1;   // fp32 slices per round
  const int tid = threadIdx.x;
  const int B = a.block;
  const int64_t nblk = a.n / B;
  const int64_t row = blockIdx.x / nblk;
  const int64_t c0 = (blockIdx.x % nblk) * B;
  const int64_t off = row * a.n + c0;
  const int nch = B >> 3;
  const auto srs = make_rsrc(a.signs, a.signs ? (uint32_t)(((a.n + 31) >> 5) * 4) : 0u);
  uint32_t sw[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int ch = tid + 256 * j;
    sw[j] = buf_load_u32(srs, ch < nch ? (uint32_t)(((c0 + 8 * ch) >> 5) * 4) : BUF_OFF);
  }
  float v[J][8];
  if constexpr (IN_F32) {
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) v[j][e] = 0.f;
    const float* base = (const float*)a.in + off;
    const auto irs = make_rsrc(base, (uint32_t)(((a.nsum - 1) * a.sum_stride + B) * 4));
    for (int s0 = 0; s0 < a.nsum; s0 += SU) {
      uint4 p[SU][J][2];
#pragma unroll
      for (int su = 0; su < SU; ++su)
#pragma unroll
        for (int j = 0; j < J; ++j) {
          const int ch = tid + 256 * j;
          const bool ok = ch < nch && s0 + su < a.nsum;
          const uint32_t o = (uint32_t)(((s0 + su) * a.sum_stride + 8 * ch) * 4);
          p[su][j][0] = buf_load_u4(irs, ok ? o : BUF_OFF);
          p[su][j][1] = buf_load_u4(irs, ok ? o + 16u : BUF_OFF);
        }
#pragma unroll
      for (int su = 0; su < SU; ++su)
#pragma unroll
        for (int j = 0; j < J; ++j) {
          const uint32_t r[8] = {p[su][j][0].x, p[su][j][0].y, p[su][j][0].z, p[su][j][0].w,
                                 p[su][j][1].x, p[su][j][1].y, p[su][j][1].z, p[su][j][1].w};
#pragma unroll
          for (int e = 0; e < 8; ++e) v[j][e] += __builtin_bit_cast(float, r[e]);
        }
    }
  } else {
    const auto irs = make_rsrc((const uint16_t*)a.in + off, (uint32_t)B * 2u);
    uint4 p[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int ch = tid + 256 * j;
      p[j] = buf_load_u4(irs, ch < nch ? (uint32_t)ch * 16u : BUF_OFF);
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const uint32_t r[4] = {p[j].x, p[j].y, p[j].z, p[j].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) v[j][e] = h2f((uint16_t)(r[e >> 1] >> (16 * (e & 1))));
    }
  }
  // the chunk's 8 signs start at bit (c0 + 8 ch) & 31 of its word
#pragma unroll
  for (int j = 0; j < J; ++j) sw[j] >>= (c0 + 8 * (tid + 256 * j)) & 31;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int ch = tid + 256 * j;
    if (ch < nch) {
      if (a.mode == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if ((sw[j] >> e) & 1u) v[j][e] = -v[j][e];
      }
      fwht_regs<8>(v[j]);
#pragma unroll
      for (int e = 0; e < 8; ++e) buf[pad_index(8 * ch + e)] = v[j][e];
    }
  }
  __syncthreads();
  fwht_bits(buf, B, 3, 31 - __builtin_clz((unsigned)B), tid, 256);
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int ch = tid + 256 * j;
    if (ch < nch) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        o[e] = buf[pad_index(8 * ch + e)] * a.mult;
        if (a.mode == 1 && ((sw[j] >> e) & 1u)) o[e] = -o[e];
      }
      const int64_t e0 = off + 8 * (int64_t)ch;
      if (a.out_f32) {
        float* dst = (float*)a.out + e0;
        *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(o[4], o[5], o[6], o[7]);
      } else {
        uint32_t r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = f2h_bits(o[2 * e]) | ((uint32_t)f2h_bits(o[2 * e + 1]) << 16);
        *reinterpret_cast<uint4*>((uint16_t*)a.out + e0) = make_uint4(r[0], r[1], r[2], r[3]);
      }
    }
  }
}

// The RHT arguments as plain leading kernel arguments (13 dwords): the
// build preloads them into SGPRs at wave launch, so a workgroup issues its
// loads without a round trip to the argument segment.  Element counts stay
// below 2^30 (the boundary limits rows x n x 4 bytes below 2^32).
#define QDEC_RHT_PARAMS                                                                          \
  const void *ain, void *aout, const uint32_t *asg, int n32, int blk, int mode, int out_f32, int nsum, \
      int sum_stride, float mult
#define QDEC_RHT_ARGS(a)                                                                         \
  (a).in, (a).out, (a).signs, (int)(a).n, (a).block, (a).mode, (a).out_f32, (a).nsum, (int)(a).sum_stride, (a).mult

// Blocks of 2048 J values (J = 1, 2, 4): the chunks, loads and signs of
// rht_kernel, but one barrier.  Index 8 (tid + 256 j) + e: bits 0-2 (e) are
// butterflies in registers, bits 3-8 (lane bits 0-5) butterflies between
// lanes (DPP quad permutes for lanes ^1 and ^2, ds_swizzle for ^4, ^8, ^16,
// ds_bpermute for ^32); one exchange through LDS then gives thread t the
// indices t + 256 k (k < 8 J), whose bits 9 and up are butterflies in
// registers again, and the results are stored from there (one store of a
// wave covers 64 consecutive entries).  The stages run in ascending bit
// order, as rht_kernel's, and each is the same sum or difference, so both
// kernels give the same bits.  A workgroup reads its whole block before it
// writes: in place is safe.
template <bool IN_F32, int J>
__global__ __launch_bounds__(256) void rht_lanes_kernel(QDEC_RHT_PARAMS) {
  extern __shared__ __align__(16) float buf[];
  constexpr int SU = IN_F32 ? (J >= 4 ? 1 : 4 / J) : 1;   // fp32 slices per round
  constexpr int K = 8 * J;                                 // values per thread
  const int tid = threadIdx.x, lane = tid & 63;
  const int B = 2048 * J;
  (void)blk;
  const int nblk = n32 / B;
  const int row = (int)blockIdx.x / nblk;
  const int c0 = ((int)blockIdx.x - row * nblk) * B;
  const int64_t off = (int64_t)row * n32 + c0;
  const bool out_signs = mode == 1;
  // sign words: on the input side those of the thread's chunks (8 tid +
  // 2048 j), on the output side those of its outputs (tid + 256 k)
  const auto srs = make_rsrc(asg, asg ? (uint32_t)(((n32 + 31) >> 5) * 4) : 0u);
  uint32_t sw[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int64_t i = out_signs ? c0 + tid + 256 * k : c0 + 8 * (tid + 256 * k);
    sw[k] = buf_load_u32(srs, (out_signs || k < J) ? (uint32_t)((i >> 5) * 4) : BUF_OFF);
  }
  float v[J][8];
  if constexpr (IN_F32) {
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) v[j][e] = 0.f;
    const float* base = (const float*)ain + off;
    const auto irs = make_rsrc(base, (uint32_t)(((nsum - 1) * (int64_t)sum_stride + B) * 4));
    for (int s0 = 0; s0 < nsum; s0 += SU) {
      uint4 p[SU][J][2];
#pragma unroll
      for (int su = 0; su < SU; ++su)
#pragma unroll
        for (int j = 0; j < J; ++j) {
          const int ch = tid + 256 * j;
          const bool ok = s0 + su < nsum;
          const uint32_t o = (uint32_t)(((int64_t)(s0 + su) * sum_stride + 8 * ch) * 4);
          p[su][j][0] = buf_load_u4(irs, ok ? o : BUF_OFF);
          p[su][j][1] = buf_load_u4(irs, ok ? o + 16u : BUF_OFF);
        }
#pragma unroll
      for (int su = 0; su < SU; ++su)
#pragma unroll
        for (int j = 0; j < J; ++j) {
          const uint32_t r[8] = {p[su][j][0].x, p[su][j][0].y, p[su][j][0].z, p[su][j][0].w,
                                 p[su][j][1].x, p[su][j][1].y, p[su][j][1].z, p[su][j][1].w};
#pragma unroll
          for (int e = 0; e < 8; ++e) v[j][e] += __builtin_bit_cast(float, r[e]);
        }
    }
  } else {
    const auto irs = make_rsrc((const uint16_t*)ain + off, (uint32_t)B * 2u);
    uint4 p[J];
#pragma unroll
    for (int j = 0; j < J; ++j) p[j] = buf_load_u4(irs, (uint32_t)(tid + 256 * j) * 16u);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const uint32_t r[4] = {p[j].x, p[j].y, p[j].z, p[j].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) v[j][e] = h2f((uint16_t)(r[e >> 1] >> (16 * (e & 1))));
    }
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (!out_signs) {
      const uint32_t sg = sw[j] >> ((c0 + 8 * (tid + 256 * j)) & 31);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if ((sg >> e) & 1u) v[j][e] = -v[j][e];
    }
    fwht_regs<8>(v[j]);
  }
  // bits 3-8 between lanes: the lower lane keeps the sum, the upper one the
  // difference (fma(v, -1, o) = o - v exactly)
  auto stage = [&](int lbit, auto&& partner) {
    const float sgn = (lane >> lbit) & 1 ? -1.f : 1.f;
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) v[j][e] = __builtin_fmaf(v[j][e], sgn, partner(v[j][e]));
  };
  stage(0, [](float x) { return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true)); });
  stage(1, [](float x) { return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, true)); });
  stage(2, [](float x) { return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x1F | (4 << 10))); });
  stage(3, [](float x) { return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x1F | (8 << 10))); });
  stage(4, [](float x) { return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x1F | (16 << 10))); });
  stage(5, [](float x) { return __shfl_xor(x, 32, 64); });
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) buf[pad_index(8 * (tid + 256 * j) + e)] = v[j][e];
  __syncthreads();
  float w[K];
#pragma unroll
  for (int k = 0; k < K; ++k) w[k] = buf[pad_index(tid + 256 * k)];
  // bits 9 and up: k bits 1 and up
#pragma unroll
  for (int h = 2; h < K; h <<= 1) {
#pragma unroll
    for (int i = 0; i < K; ++i) {
      if (!(i & h)) {
        const float x0 = w[i], x1 = w[i + h];
        w[i] = x0 + x1;
        w[i + h] = x0 - x1;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int64_t i = c0 + tid + 256 * k;
    float o = w[k] * mult;
    if (out_signs && ((sw[k] >> (i & 31)) & 1u)) o = -o;
    if (out_f32) ((float*)aout)[(int64_t)row * n32 + i] = o;
    else ((uint16_t*)aout)[(int64_t)row * n32 + i] = f2h_bits(o);
  }
}

// fp16 input with few (row, block) pairs: each block is cut over S
// workgroups.  With Sylvester ordering H_B = H_S (x) H_Bs (Bs = B / S), so
// outputs [j Bs, (j+1) Bs) of a block are H_Bs applied to u = sum over a of
// H_S[j][a] x_a, x_a the a-th Bs-slice (input signs applied): every
// workgroup reads the whole block, forms its own +/- combination and runs a
// Bs-point transform.  Chunks of 8 values as in rht_kernel, J per thread.
template <int S, int J>
__global__ __launch_bounds__(256) void rht_split_kernel(QDEC_RHT_PARAMS) {
  extern __shared__ __align__(16) float buf[];
  const int tid = threadIdx.x;
  (void)nsum;
  (void)sum_stride;
  const int B = blk, Bs = B / S;
  const int nblk = n32 / B;
  const int jpart = (int)(blockIdx.x % S);
  const int rb = (int)(blockIdx.x / S);
  const int row = rb / nblk;
  const int c0 = (rb - row * nblk) * B;
  const int64_t off = (int64_t)row * n32 + c0;
  const int nch = Bs >> 3;
  const auto srs = make_rsrc(asg, asg ? (uint32_t)(((n32 + 31) >> 5) * 4) : 0u);
  const auto irs = make_rsrc((const uint16_t*)ain + off, (uint32_t)B * 2u);
  uint4 p[S][J];
  uint32_t sw[S][J];
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int ch = tid + 256 * j;
      const bool ok = ch < nch;
      p[s][j] = buf_load_u4(irs, ok ? (uint32_t)(s * Bs + 8 * ch) * 2u : BUF_OFF);
      sw[s][j] = buf_load_u32(srs, ok && mode == 0 ? (uint32_t)(((c0 + s * Bs + 8 * ch) >> 5) * 4) : BUF_OFF);
    }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int ch = tid + 256 * j;
    if (ch < nch) {
      float u[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) u[e] = 0.f;
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const uint32_t r[4] = {p[s][j].x, p[s][j].y, p[s][j].z, p[s][j].w};
        const uint32_t sg = sw[s][j] >> ((c0 + s * Bs + 8 * ch) & 31);
        const bool neg_s = __builtin_popcount((unsigned)(jpart & s)) & 1;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = h2f((uint16_t)(r[e >> 1] >> (16 * (e & 1))));
          const bool neg = (((sg >> e) & 1u) != 0) != neg_s;
          u[e] += neg ? -v : v;
        }
      }
      fwht_regs<8>(u);
#pragma unroll
      for (int e = 0; e < 8; ++e) buf[pad_index(8 * ch + e)] = u[e];
    }
  }
  __syncthreads();
  fwht_bits(buf, Bs, 3, 31 - __builtin_clz((unsigned)Bs), tid, 256);
  const int64_t o0 = off + (int64_t)jpart * Bs;
  const auto ors = make_rsrc(asg, asg ? (uint32_t)(((n32 + 31) >> 5) * 4) : 0u);
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int ch = tid + 256 * j;
    if (ch < nch) {
      const uint32_t sg = mode == 1 ? buf_load_u32(ors, (uint32_t)(((c0 + jpart * Bs + 8 * ch) >> 5) * 4)) >>
                                            ((c0 + jpart * Bs + 8 * ch) & 31)
                                      : 0u;
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        o[e] = buf[pad_index(8 * ch + e)] * mult;
        if ((sg >> e) & 1u) o[e] = -o[e];
      }
      const int64_t e0 = o0 + 8 * (int64_t)ch;
      if (out_f32) {
        float* dst = (float*)aout + e0;
        *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(o[4], o[5], o[6], o[7]);
      } else {
        uint32_t r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = f2h_bits(o[2 * e]) | ((uint32_t)f2h_bits(o[2 * e + 1]) << 16);
        *reinterpret_cast<uint4*>((uint16_t*)aout + e0) = make_uint4(r[0], r[1], r[2], r[3]);
      }
    }
  }
}

template <int S>
static hipError_t launch_rht_split(const RhtArgs& a, hipStream_t stream) {
  const int Bs = a.block / S;
  const size_t lds = (size_t)padded_words(Bs) * 4;
  const unsigned grid = (unsigned)(a.rows * (a.n / a.block) * S);
  const int nch = Bs >> 3;
#define QDEC_SPLIT_J(JJ)                                                                            \
  {                                                                                                 \
    static LdsLimit have;                                                                         \
    const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&rht_split_kernel<S, JJ>), lds, &have); \
    if (e != hipSuccess) return e;                                                                  \
    hipLaunchKernelGGL((rht_split_kernel<S, JJ>), dim3(grid), dim3(256), lds, stream, QDEC_RHT_ARGS(a)); \
    return hipGetLastError();                                                                       \
  }
  if (nch <= 256) QDEC_SPLIT_J(1)
  if (nch <= 512) QDEC_SPLIT_J(2)
  QDEC_SPLIT_J(4)
#undef QDEC_SPLIT_J
}

template <bool IN_F32, int J>
static hipError_t launch_rht_j(const RhtArgs& a, hipStream_t stream) {
  static LdsLimit have;
  const size_t lds = (size_t)padded_words(a.block) * 4;
  const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&rht_kernel<IN_F32, J>), lds, &have);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((rht_kernel<IN_F32, J>), dim3((unsigned)(a.rows * (a.n / a.block))), dim3(256), lds,
                     stream, a);
  return hipGetLastError();
}

template <bool IN_F32, int J>
static hipError_t launch_rht_lanes(const RhtArgs& a, hipStream_t stream) {
  static LdsLimit have;
  const size_t lds = (size_t)padded_words(a.block) * 4;
  const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&rht_lanes_kernel<IN_F32, J>), lds, &have);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((rht_lanes_kernel<IN_F32, J>), dim3((unsigned)(a.rows * (a.n / a.block))), dim3(256), lds,
                     stream, QDEC_RHT_ARGS(a));
  return hipGetLastError();
}

template <bool IN_F32>
static hipError_t launch_rht_in(const RhtArgs& a, hipStream_t stream) {
  // blocks of 2048, 4096 and 8192 values: one barrier (rht_lanes_kernel)
  if (a.block == 2048) return launch_rht_lanes<IN_F32, 1>(a, stream);
  if (a.block == 4096) return launch_rht_lanes<IN_F32, 2>(a, stream);
  if (a.block == 8192) return launch_rht_lanes<IN_F32, 4>(a, stream);
  const int nch = a.block >> 3;
  if (nch <= 256) return launch_rht_j<IN_F32, 1>(a, stream);
  if (nch <= 512) return launch_rht_j<IN_F32, 2>(a, stream);
  if (nch <= 1024) return launch_rht_j<IN_F32, 4>(a, stream);
  return launch_rht_j<IN_F32, 8>(a, stream);
}

// Blocks cut over S workgroups (fp16 input): S grows while there are
// fewer than 256 workgroups and the pieces keep at least 512 values.  Never
// in place: every workgroup of a cut block reads the whole block but writes
// only its own slice, so a workgroup that finishes first would overwrite
// inputs that the others have not read yet.
int rht_split_factor(const RhtArgs& a) {
  if (a.in_f32 || a.block < 1024 || a.in == a.out) return 1;
  const int64_t wg = a.rows * (a.n / a.block);
  int S = 1;
  while (S < 8 && wg * S < 256 && a.block / (2 * S) >= 512) S *= 2;
  return S;
}

static hipError_t launch_rht_impl(const RhtArgs& a, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  if (a.block < 8) {
    const size_t lds = (size_t)padded_words(a.block) * 4;
    hipLaunchKernelGGL(rht_tiny_kernel, dim3((unsigned)(a.rows * (a.n / a.block))), dim3(256), lds, stream, a);
    return hipGetLastError();
  }
  switch (rht_split_factor(a)) {
    case 2: return launch_rht_split<2>(a, stream);
    case 4: return launch_rht_split<4>(a, stream);
    case 8: return launch_rht_split<8>(a, stream);
    default: break;
  }
  return a.in_f32 ? launch_rht_in<true>(a, stream) : launch_rht_in<false>(a, stream);
}

hipError_t launch_rht(const RhtArgs& a, hipStream_t stream) {
  RhtArgs b = a;
  if (b.nsum < 1) b.nsum = 1;
  return launch_rht_impl(b, stream);
}

hipError_t launch_rht_out_f32(const float* z, int nsum, uint16_t* y, int64_t rows, int64_t m, int block,
                              const uint32_t* signs, float mult, hipStream_t stream) {
  RhtArgs a;
  a.in = z;
  a.out = y;
  a.in_f32 = 1;
  a.out_f32 = 0;
  a.rows = rows;
  a.n = m;
  a.block = block;
  a.signs = signs;
  a.mode = 1;
  a.mult = mult;
  a.nsum = nsum;
  a.sum_stride = rows * m;
  return launch_rht_impl(a, stream);
}

}  // namespace qdec

namespace qdec {
// Output side of qdec_gemv, one launch for every layer of a call.  Each
// layer's K slices hold, per 128-row panel, partial sums already multiplied
// by H_min(Bo,128) (the stages inside a panel, done by the GEMV
// workgroups).  With Sylvester ordering H_Bo = H_P (x) H_128 (P = Bo/128), so
// what is left are the index bits 7 .. log2(Bo) of the transform.  One
// workgroup per (rows_wg rows, batch column): its threads add the slices in
// slice order (a fixed order: the output is reproducible bit for bit), run
// the remaining stages in LDS, scale, apply the output signs and write fp16.
template <int J>   // float4 chunks per thread: rows_wg <= 4096 J
__global__ __launch_bounds__(1024) void gemv_finish_kernel(QDEC_BOUNDS_PARAMS, FinishArgs a) {
  extern __shared__ __align__(16) float buf[];
  constexpr int SU = 16 / J;                      // slices per round of loads (16 float4 per thread)
  (void)nl_;
  const int li = QDEC_LAYER_OF((int)blockIdx.x);
  const float* z = a.lay[li].z;
  const int64_t sstride = a.lay[li].slice_stride, m = a.lay[li].m;
  const int nsl = a.lay[li].nslices, Bo = a.lay[li].Bo, R = a.lay[li].rows_wg;
  const int lw = (int)blockIdx.x - a.lay[li].wg0;
  const int nseg = (int)(m / R);
  const int seg = lw % nseg, c = lw / nseg;
  const int tid = threadIdx.x, nch = R >> 2;
  const int64_t r0 = (int64_t)seg * R;
  // the workgroup's rows of every slice, through one buffer resource
  const auto zrs = make_rsrc(z + (int64_t)c * m + r0, (uint32_t)(((int64_t)(nsl - 1) * sstride + R) * 4));
  // the sign words (the 4 rows of a chunk share one word: 4-row groups never
  // straddle one), requested with the first slices
  const uint32_t* sg = a.lay[li].sign_out;
  const auto srs = make_rsrc(sg, sg ? (uint32_t)(((m + 31) >> 5) * 4) : 0u);
  uint32_t sw[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int ch = tid + 1024 * j;
    sw[j] = buf_load_u32(srs, ch < nch ? (uint32_t)(((r0 + 4 * ch) >> 5) * 4) : BUF_OFF);
  }
  float acc[J][4];
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[j][e] = 0.f;
  for (int s0 = 0; s0 < nsl; s0 += SU) {
    uint4 v[SU][J];
#pragma unroll
    for (int su = 0; su < SU; ++su)
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int ch = tid + 1024 * j;
        const bool ok = ch < nch && s0 + su < nsl;
        v[su][j] = buf_load_u4(zrs, ok ? (uint32_t)(((int64_t)(s0 + su) * sstride + 4 * ch) * 4) : BUF_OFF);
      }
#pragma unroll
    for (int su = 0; su < SU; ++su)
#pragma unroll
      for (int j = 0; j < J; ++j) {
        acc[j][0] += __builtin_bit_cast(float, v[su][j].x);
        acc[j][1] += __builtin_bit_cast(float, v[su][j].y);
        acc[j][2] += __builtin_bit_cast(float, v[su][j].z);
        acc[j][3] += __builtin_bit_cast(float, v[su][j].w);
      }
  }
  if (Bo > 128) {                                  // workgroup-uniform
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int ch = tid + 1024 * j;
      if (ch < nch) {
#pragma unroll
        for (int e = 0; e < 4; ++e) buf[pad_index(4 * ch + e)] = acc[j][e];
      }
    }
    __syncthreads();
    fwht_bits<3>(buf, R, 7, 31 - __builtin_clz((unsigned)Bo), tid, 1024);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int ch = tid + 1024 * j;
      if (ch < nch) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[j][e] = buf[pad_index(4 * ch + e)];
      }
    }
  }
  const float mult = a.lay[li].mult;
  uint16_t* yc = a.lay[li].y + (int64_t)c * m + r0;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int ch = tid + 1024 * j;
    const uint32_t swj = sw[j] >> ((r0 + 4 * ch) & 31);
    if (ch < nch) {
      uint32_t h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = acc[j][e] * mult;
        h[e] = f2h_bits(((swj >> e) & 1u) ? -v : v);
      }
      *reinterpret_cast<uint2*>(yc + 4 * ch) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
    }
  }
}

static LayerBounds finish_bounds(const FinishArgs& a) {
  LayerBounds b;
  b.w[0] = a.nl;
  for (int i = 1; i < GEMV_GROUP_MAX; ++i) b.w[i] = i < a.nl ? a.lay[i].wg0 : INT_MAX;
  return b;
}

template <int J>
static hipError_t launch_finish_j(const FinishArgs& a, unsigned grid, size_t lds, hipStream_t stream) {
  static LdsLimit have;
  const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&gemv_finish_kernel<J>), lds, &have);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gemv_finish_kernel<J>), dim3(grid), dim3(1024), lds, stream, QDEC_BOUNDS_ARGS(finish_bounds(a)),
                     a);
  return hipGetLastError();
}

// The same finish with the cross-panel stages between lanes, for blocks of
// P <= 32 panels (P = Bo / 128, 1 below): thread t of a (layer, column)
// takes row blk Rb + p 128 + i of block blk (Rb = 128 P rows) with
// p = t mod P, i = (t mod Rb) / P, so the P rows at one in-panel index sit
// in P neighbouring lanes and stage h of H_P pairs lanes t and t ^ h (one
// ds_swizzle each: no LDS buffer, no barrier).  One wave per workgroup,
// rows past m idle; each layer's workgroups are ceil(m / 64) per column,
// column major.  Slices are added in slice order, as above.
// One butterfly stage between lanes t and t ^ H (H < 32): ds_swizzle in
// bit-mask mode (offset bit 15 clear: within each 32 lanes, lane j reads
// lane ((j & 31) | 0) ^ H).  The lower lane keeps the sum, the upper one the
// difference.
template <int H>
__device__ __forceinline__ void lane_butterfly(float& v, int lane) {
  const float o = __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x1F | (H << 10)));
  v = (lane & H) ? o - v : v + o;
}

// One wave per workgroup: the slice loads (each wave load spans up to 32
// cache lines) spread over as many CUs as there are waves.
constexpr int FIN_LANES_THREADS = 64;

// The work of one lane-finisher workgroup, lw its index within the layer.
__device__ __forceinline__ void finish_lanes(int lw, const float* zl, uint16_t* yl, const uint32_t* sg, int m,
                                             int Bo, int nsl, int ncol, int64_t sstride, float mult) {
  const int P = Bo >= 128 ? Bo >> 7 : 1;           // workgroup-uniform, a power of two
  const int lp = 31 - __builtin_clz((unsigned)P);
  const int wpc = (m + FIN_LANES_THREADS - 1) / FIN_LANES_THREADS;   // workgroups per column
  // Workgroups are dealt to the 8 XCDs in turn, and one wave holds only
  // 64 / P consecutive rows of each panel, so the workgroups that share a
  // cache line of a slice are logical neighbours: the layer's first
  // 8 floor(nwg / 8) workgroups take their logical index in XCD-major
  // order, which puts logical neighbours on one XCD and its L2.
  const int nq = (wpc * ncol) & ~7;
  if (lw < nq) lw = (lw & 7) * (nq >> 3) + (lw >> 3);
  const int c = lw / wpc;
  const int64_t g = (int64_t)(lw - c * wpc) * FIN_LANES_THREADS + threadIdx.x;
  const int lane = threadIdx.x & 63;
  const int Rb = 128 * P;
  const int t = (int)(g & (Rb - 1));
  const int64_t row = (g & ~(int64_t)(Rb - 1)) + (int64_t)(t & (P - 1)) * 128 + (t >> lp);
  const bool live = g < m;
  const float* zc = zl + (int64_t)c * m + row;
  // the sign word first: issued with the slices, not after the butterflies
  const uint32_t sgw = live && sg ? sg[row >> 5] : 0u;
  float acc = 0.f;
  for (int s0 = 0; s0 < nsl; s0 += 16) {
    float v[16];
#pragma unroll
    for (int su = 0; su < 16; ++su) v[su] = live && s0 + su < nsl ? zc[(int64_t)(s0 + su) * sstride] : 0.f;
#pragma unroll
    for (int su = 0; su < 16; ++su)
      if (s0 + su < nsl) acc += v[su];
  }
  if (P > 1) lane_butterfly<1>(acc, lane);
  if (P > 2) lane_butterfly<2>(acc, lane);
  if (P > 4) lane_butterfly<4>(acc, lane);
  if (P > 8) lane_butterfly<8>(acc, lane);
  if (P > 16) lane_butterfly<16>(acc, lane);
  if (live) {
    const bool neg = (sgw >> (row & 31)) & 1u;
    const float v = acc * mult;
    yl[(int64_t)c * m + row] = f2h_bits(neg ? -v : v);
  }
}

// Several layers: the layer bounds are preloaded, the layer's fields come
// from the argument struct in one round of scalar loads.
__global__ __launch_bounds__(FIN_LANES_THREADS) void gemv_finish_lanes_kernel(QDEC_BOUNDS_PARAMS, FinishArgs a) {
  (void)nl_;
  const int li = QDEC_LAYER_OF((int)blockIdx.x);
  const int m = (int)a.lay[li].m;
  const int Bo = a.lay[li].Bo, wg0 = a.lay[li].wg0, nsl = a.lay[li].nslices, ncol = a.lay[li].b;
  const int64_t sstride = a.lay[li].slice_stride;
  const float* zl = a.lay[li].z;
  const uint32_t* sg = a.lay[li].sign_out;
  const float mult = a.lay[li].mult;
  uint16_t* yl = a.lay[li].y;
  asm volatile("" ::"s"(m), "s"(Bo), "s"(wg0), "s"(nsl), "s"(ncol), "s"(sstride), "s"(zl), "s"(sg), "s"(mult),
               "s"(yl));
  finish_lanes((int)blockIdx.x - wg0, zl, yl, sg, m, Bo, nsl, ncol, sstride, mult);
}

// One layer: every field is a leading scalar argument, all preloaded into
// SGPRs at wave launch (12 of them), so no argument is loaded from memory.
__global__ __launch_bounds__(FIN_LANES_THREADS) void gemv_finish_lanes1_kernel(const float* z, uint16_t* y,
                                                                               const uint32_t* sg, int m, int Bo,
                                                                               int nsl, int ncol, int sstride,
                                                                               float mult) {
  finish_lanes((int)blockIdx.x, z, y, sg, m, Bo, nsl, ncol, sstride, mult);
}

// Two layers of one shape (gate and up): the slices and sign vectors of
// both, the second layer's first workgroup, the shape (m and log2 B_out;
// slices and columns) and the slice stride are preloaded (12 SGPRs); the
// outputs and scales, needed only at the store, come from the struct.
__global__ __launch_bounds__(FIN_LANES_THREADS) void gemv_finish_lanes2_kernel(const float* z0, const float* z1,
                                                                               const uint32_t* sg0,
                                                                               const uint32_t* sg1, int w1,
                                                                               uint32_t shape0, uint32_t shape1,
                                                                               int sstride, FinishArgs a) {
  const int li = (int)blockIdx.x >= w1 ? 1 : 0;
  finish_lanes((int)blockIdx.x - (li ? w1 : 0), li ? z1 : z0, a.lay[li].y, li ? sg1 : sg0,
               (int)(shape0 & 0xFFFFFFu), 1 << (shape0 >> 24), (int)(shape1 & 0xFFFFu), (int)(shape1 >> 16), sstride,
               a.lay[li].mult);
}

hipError_t launch_gemv_finish(const FinishArgs& a, hipStream_t stream) {
  // the lane finisher where every block is at most 32 panels
  bool lanes = a.nl > 0;
  for (int l = 0; l < a.nl; ++l)
    if (a.lay[l].Bo > 32 * 128) lanes = false;
  if (lanes) {
    FinishArgs b = a;
    unsigned grid = 0;
    for (int l = 0; l < b.nl; ++l) {
      b.lay[l].wg0 = (int)grid;
      grid += (unsigned)(((b.lay[l].m + FIN_LANES_THREADS - 1) / FIN_LANES_THREADS) * b.lay[l].b);
    }
    if (grid == 0) return hipSuccess;
    const FinishLayer& f = b.lay[0];
    if (b.nl == 1 && f.slice_stride <= INT32_MAX) {
      hipLaunchKernelGGL(gemv_finish_lanes1_kernel, dim3(grid), dim3(FIN_LANES_THREADS), 0, stream, f.z, f.y,
                         f.sign_out, (int)f.m, f.Bo, f.nslices, f.b, (int)f.slice_stride, f.mult);
      return hipGetLastError();
    }
    const FinishLayer& g = b.lay[1];
    if (b.nl == 2 && f.m == g.m && f.Bo == g.Bo && f.nslices == g.nslices && f.b == g.b &&
        f.slice_stride == g.slice_stride && f.slice_stride <= INT32_MAX && f.m < (1 << 24) && f.Bo > 0 &&
        (f.Bo & (f.Bo - 1)) == 0 && f.nslices < (1 << 16) && f.b < (1 << 16)) {
      const uint32_t shape0 = (uint32_t)f.m | ((uint32_t)(31 - __builtin_clz((unsigned)f.Bo)) << 24);
      const uint32_t shape1 = (uint32_t)f.nslices | ((uint32_t)f.b << 16);
      hipLaunchKernelGGL(gemv_finish_lanes2_kernel, dim3(grid), dim3(FIN_LANES_THREADS), 0, stream, f.z, g.z,
                         f.sign_out, g.sign_out, g.wg0, shape0, shape1, (int)f.slice_stride, b);
      return hipGetLastError();
    }
    hipLaunchKernelGGL(gemv_finish_lanes_kernel, dim3(grid), dim3(FIN_LANES_THREADS), 0, stream,
                       QDEC_BOUNDS_ARGS(finish_bounds(b)),
                       b);
    return hipGetLastError();
  }
  unsigned grid = 0;
  size_t lds = 0;
  int rmax = 0;
  for (int l = 0; l < a.nl; ++l) {
    const FinishLayer& f = a.lay[l];
    if (f.wg0 != (int)grid) return hipErrorInvalidValue;
    grid += (unsigned)((f.m / f.rows_wg) * f.b);
    if (f.Bo > 128 && (size_t)padded_words(f.rows_wg) * 4 > lds) lds = (size_t)padded_words(f.rows_wg) * 4;
    if (f.rows_wg > rmax) rmax = f.rows_wg;
  }
  if (grid == 0) return hipSuccess;
  if (rmax <= 4096) return launch_finish_j<1>(a, grid, lds, stream);
  if (rmax <= 8192) return launch_finish_j<2>(a, grid, lds, stream);
  return launch_finish_j<4>(a, grid, lds, stream);
}
}  // namespace qdec
