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
  static size_t have = 0;
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

// fp16 input with few (row, block) pairs: each block is cut over S
// workgroups.  With Sylvester ordering H_B = H_S (x) H_Bs (Bs = B / S), so
// outputs [j Bs, (j+1) Bs) of a block are H_Bs applied to u = sum over a of
// H_S[j][a] x_a, x_a the a-th Bs-slice (input signs applied): every
// workgroup reads the whole block, forms its own +/- combination and runs a
// Bs-point transform.  Chunks of 8 values as in rht_kernel, J per thread.
template <int S, int J>
__global__ __launch_bounds__(256) void rht_split_kernel(RhtArgs a) {
  extern __shared__ __align__(16) float buf[];
  const int tid = threadIdx.x;
  const int B = a.block, Bs = B / S;
  const int64_t nblk = a.n / B;
  const int jpart = (int)(blockIdx.x % S);
  const int64_t rb = blockIdx.x / S;
  const int64_t row = rb / nblk;
  const int64_t c0 = (rb % nblk) * B;
  const int64_t off = row * a.n + c0;
  const int nch = Bs >> 3;
  const auto srs = make_rsrc(a.signs, a.signs ? (uint32_t)(((a.n + 31) >> 5) * 4) : 0u);
  const auto irs = make_rsrc((const uint16_t*)a.in + off, (uint32_t)B * 2u);
  uint4 p[S][J];
  uint32_t sw[S][J];
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int ch = tid + 256 * j;
      const bool ok = ch < nch;
      p[s][j] = buf_load_u4(irs, ok ? (uint32_t)(s * Bs + 8 * ch) * 2u : BUF_OFF);
      sw[s][j] = buf_load_u32(srs, ok && a.mode == 0 ? (uint32_t)(((c0 + s * Bs + 8 * ch) >> 5) * 4) : BUF_OFF);
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
  const auto ors = make_rsrc(a.signs, a.signs ? (uint32_t)(((a.n + 31) >> 5) * 4) : 0u);
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int ch = tid + 256 * j;
    if (ch < nch) {
      const uint32_t sg = a.mode == 1 ? buf_load_u32(ors, (uint32_t)(((c0 + jpart * Bs + 8 * ch) >> 5) * 4)) >>
                                            ((c0 + jpart * Bs + 8 * ch) & 31)
                                      : 0u;
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        o[e] = buf[pad_index(8 * ch + e)] * a.mult;
        if ((sg >> e) & 1u) o[e] = -o[e];
      }
      const int64_t e0 = o0 + 8 * (int64_t)ch;
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

template <int S>
static hipError_t launch_rht_split(const RhtArgs& a, hipStream_t stream) {
  const int Bs = a.block / S;
  const size_t lds = (size_t)padded_words(Bs) * 4;
  const unsigned grid = (unsigned)(a.rows * (a.n / a.block) * S);
  const int nch = Bs >> 3;
#define QDEC_SPLIT_J(JJ)                                                                            \
  {                                                                                                 \
    static size_t have = 0;                                                                         \
    const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&rht_split_kernel<S, JJ>), lds, &have); \
    if (e != hipSuccess) return e;                                                                  \
    hipLaunchKernelGGL((rht_split_kernel<S, JJ>), dim3(grid), dim3(256), lds, stream, a);           \
    return hipGetLastError();                                                                       \
  }
  if (nch <= 256) QDEC_SPLIT_J(1)
  if (nch <= 512) QDEC_SPLIT_J(2)
  QDEC_SPLIT_J(4)
#undef QDEC_SPLIT_J
}

template <bool IN_F32, int J>
static hipError_t launch_rht_j(const RhtArgs& a, hipStream_t stream) {
  static size_t have = 0;
  const size_t lds = (size_t)padded_words(a.block) * 4;
  const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&rht_kernel<IN_F32, J>), lds, &have);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((rht_kernel<IN_F32, J>), dim3((unsigned)(a.rows * (a.n / a.block))), dim3(256), lds,
                     stream, a);
  return hipGetLastError();
}

template <bool IN_F32>
static hipError_t launch_rht_in(const RhtArgs& a, hipStream_t stream) {
  const int nch = a.block >> 3;
  if (nch <= 256) return launch_rht_j<IN_F32, 1>(a, stream);
  if (nch <= 512) return launch_rht_j<IN_F32, 2>(a, stream);
  if (nch <= 1024) return launch_rht_j<IN_F32, 4>(a, stream);
  return launch_rht_j<IN_F32, 8>(a, stream);
}

// Blocks cut over S workgroups (fp16 input): S grows while there are
// fewer than 256 workgroups and the pieces keep at least 512 values.
int rht_split_factor(const RhtArgs& a) {
  if (a.in_f32 || a.block < 1024) return 1;
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
// Output side of qdec_gemv.  z (fp32 [b][m]) holds, for every 128-row panel,
// the scaled sums already multiplied by H_min(Bo,128) (the stages inside a
// panel, done by the GEMV workgroups).  With Sylvester ordering
// H_Bo = H_P (x) H_128 for P = Bo/128, so the stages left are P-point
// transforms across the P panels of a block at a fixed row offset i: one
// thread per (block, i, batch column), the P values in registers.  The
// thread then applies the output signs, writes fp16 y and re-zeroes z.
template <int P>
__global__ __launch_bounds__(128) void gemv_finish_kernel(float* z, uint16_t* y, int64_t m,
                                                        const uint32_t* sign_out) {
  const int i = threadIdx.x;
  const int64_t blk = blockIdx.x;
  const int64_t c = blockIdx.y;
  const int64_t row0 = blk * (P * 128) + i;
  float* zc = z + c * m + row0;
  float v[P];
  uint32_t sg[P];
  // sign words through a buffer that is empty without output signs (its
  // loads read zero): no branch, so all 2P loads are in flight together
  const auto srs = make_rsrc(sign_out, sign_out ? (uint32_t)(((m + 31) >> 5) * 4) : 0u);
#pragma unroll
  for (int j = 0; j < P; ++j) sg[j] = buf_load_u32(srs, (uint32_t)(((row0 + j * 128) >> 5) * 4));
#pragma unroll
  for (int j = 0; j < P; ++j) v[j] = zc[j * 128];
#pragma unroll
  for (int j = 0; j < P; ++j) sg[j] = (sg[j] >> ((row0 + j * 128) & 31)) & 1u;
#pragma unroll
  for (int j = 0; j < P; ++j) zc[j * 128] = 0.f;
  fwht_regs<P>(v);
  uint16_t* yc = y + c * m + row0;
#pragma unroll
  for (int j = 0; j < P; ++j) yc[j * 128] = f2h_bits(sg[j] ? -v[j] : v[j]);
}

template <int P>
static hipError_t launch_finish_p(const GemvArgs& a, hipStream_t stream) {
  dim3 grid((unsigned)(a.L.m / (P * 128)), (unsigned)a.b);
  hipLaunchKernelGGL((gemv_finish_kernel<P>), grid, dim3(128), 0, stream, a.z, a.y, a.L.m, a.L.sign_out);
  return hipGetLastError();
}

hipError_t launch_gemv_finish(const GemvArgs& a, hipStream_t stream) {
  const int P = a.L.had_out > 128 ? a.L.had_out / 128 : 1;
  switch (P) {
    case 1: return launch_finish_p<1>(a, stream);
    case 2: return launch_finish_p<2>(a, stream);
    case 4: return launch_finish_p<4>(a, stream);
    case 8: return launch_finish_p<8>(a, stream);
    case 16: return launch_finish_p<16>(a, stream);
    case 32: return launch_finish_p<32>(a, stream);
    case 64: return launch_finish_p<64>(a, stream);
    case 128: return launch_finish_p<128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace qdec
