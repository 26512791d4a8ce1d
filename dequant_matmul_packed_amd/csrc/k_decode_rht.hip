// qdec_decode_tile and qdec_rht kernels.
#include "gemv_impl.hpp"
#include "qdec_device.hpp"
#include "qdec_internal.hpp"

namespace qdec {

// ---------------------------------------------------------------------------
// Tile decode (the bit-exact parity surface).  32 tiles per workgroup, one
// 8-lane group per tile, the same window extraction and value maps the
// matmul kernels use.
template <int CODE, int K>
__global__ __launch_bounds__(256) void decode_tile_kernel(DecodeArgs a) {
  constexpr int COPIES = GemvTable<CODE>::COPIES;
  extern __shared__ __align__(16) uint32_t tab[];
  const int tid = threadIdx.x, lane = tid & 63, q = tid & 7;
  if constexpr (CODE == HYB) fill_signed_table<COPIES>(tab, a.L.lut, a.L.Q, tid, 256);
  if constexpr (CODE == VQ) fill_plain_table<COPIES>(tab, a.L.lut, 1 << (2 * K), tid, 256);
  if constexpr (CODE == NUQ) fill_plain_table<1>(tab, a.L.lut, 1 << K, tid, 256);
  __syncthreads();

  const int64_t tile = a.first + (int64_t)blockIdx.x * 32 + (tid >> 3);
  const bool valid = tile < a.first + a.count;
  uint32_t w[K + 1];
#pragma unroll
  for (int i = 0; i <= K; ++i) w[i] = 0u;
  if (valid) load_words<K>(a.L.codes + tile * (8 * K) + q * K, w);
  w[K] = next_lane_word(w[0], lane);
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
  lane_decode_exact<CODE, K, COPIES>(w, tab + (lane & (COPIES - 1)), a.L.qshift, gs, out);
  uint4* dst = reinterpret_cast<uint4*>(a.out + (tile - a.first) * 256 + q * 32);
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
}

template <int CODE, int K>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  constexpr int COPIES = GemvTable<CODE>::COPIES;
  const size_t lds = (size_t)gemv_table_words<CODE, K>(a.L.Q) * 4 + 16;
  (void)COPIES;
  const unsigned grid = (unsigned)((a.count + 31) / 32);
  hipLaunchKernelGGL((decode_tile_kernel<CODE, K>), dim3(grid), dim3(256), lds, stream, a);
  return hipGetLastError();
}

template <int CODE>
static hipError_t launch_decode_code(const DecodeArgs& a, hipStream_t stream) {
  switch (a.L.k) {
    case 2: return launch_decode_t<CODE, 2>(a, stream);
    case 3: return launch_decode_t<CODE, 3>(a, stream);
    case 4: return launch_decode_t<CODE, 4>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_tile(const DecodeArgs& a, hipStream_t stream) {
  if (a.count <= 0) return hipSuccess;
  switch (a.L.code) {
    case HYB: return launch_decode_code<HYB>(a, stream);
    case MAD1: return launch_decode_code<MAD1>(a, stream);
    case INST3: return launch_decode_code<INST3>(a, stream);
    case NUQ: return launch_decode_code<NUQ>(a, stream);
    case VQ: return launch_decode_code<VQ>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

bool decode_supported(int code, int k) {
  return code >= HYB && code <= VQ && k >= 2 && k <= 4;
}

// ---------------------------------------------------------------------------
// Randomized Hadamard transform of independent row blocks: one workgroup per
// (row, block), the block held in LDS in fp32.
//   mode 0: out = mult * H (s .* in);   mode 1: out = s .* (mult * H in)
// ("Incoherence Processing (W2)": the RHT is invertible up to rounding.)
// An fp32 input may be the sum of `nsum` slices `sum_stride` apart (the
// K-split partial sums of the batched path).
__global__ __launch_bounds__(256) void rht_kernel(RhtArgs a) {
  extern __shared__ __align__(16) float buf[];
  constexpr int MAXJ = 8;            // 256 threads x 8 chunks x 8 values = 16384
  const int tid = threadIdx.x;
  const int B = a.block;
  const int64_t nblk = a.n / B;
  const int64_t row = blockIdx.x / nblk;
  const int64_t c0 = (blockIdx.x % nblk) * B;
  const int64_t off = row * a.n + c0;
  if (B < 8) {                       // tiny blocks: one value per thread
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
    return;
  }
  // Chunks of 8 consecutive values.  Every global load (values and the
  // chunk's sign word) is issued before any is used, with addresses clamped
  // in bounds; the 3 butterfly stages inside a chunk run in registers, the
  // rest in padded LDS.
  const int nch = B >> 3;
  float v[MAXJ][8];
  uint32_t sw[MAXJ];
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    const int ch = tid + 256 * j;
    const int chc = ch < nch ? ch : 0;
    const int64_t e0 = off + 8 * (int64_t)chc;
    if (a.in_f32) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[j][e] = 0.f;
      for (int sl = 0; sl < a.nsum; ++sl) {     // K-split slices of a GEMM
        const float* src = (const float*)a.in + sl * a.sum_stride + e0;
        const float4 p0 = *reinterpret_cast<const float4*>(src);
        const float4 p1 = *reinterpret_cast<const float4*>(src + 4);
        v[j][0] += p0.x; v[j][1] += p0.y; v[j][2] += p0.z; v[j][3] += p0.w;
        v[j][4] += p1.x; v[j][5] += p1.y; v[j][6] += p1.z; v[j][7] += p1.w;
      }
    } else {
      const uint4 p = *reinterpret_cast<const uint4*>((const uint16_t*)a.in + e0);
      const uint32_t r[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) v[j][e] = h2f((uint16_t)(r[e >> 1] >> (16 * (e & 1))));
    }
    const int64_t g = c0 + 8 * (int64_t)chc;
    sw[j] = a.signs ? (a.signs[g >> 5] >> (g & 31)) : 0u;
  }
  const int lowbits = B >= 8 ? 3 : 0;
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
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
  fwht_bits(buf, B, lowbits, 31 - __builtin_clz((unsigned)B), tid, 256);
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
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

static hipError_t launch_rht_impl(const RhtArgs& a, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  static size_t have = 0;
  const hipError_t e =
      ensure_dynamic_lds(reinterpret_cast<const void*>(&rht_kernel), (size_t)padded_words(a.block) * 4, &have);
  if (e != hipSuccess) return e;
  const int64_t blocks = a.rows * (a.n / a.block);
  hipLaunchKernelGGL(rht_kernel, dim3((unsigned)blocks), dim3(256), (size_t)padded_words(a.block) * 4, stream, a);
  return hipGetLastError();
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
