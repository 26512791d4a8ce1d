// Batched decode-and-multiply (qdec_gemm): decoded tiles staged in LDS and
// fed to fp16 MFMA (v_mfma_f32_16x16x32_f16) with fp32 accumulation.
//
// A workgroup (4 waves) owns one panel of 128 output rows and 64 batch
// columns; the K loop steps 64 input columns (4 tile columns) at a time:
// wave w decodes tile column 4*it + w of the panel (8 tiles, 8 lanes each)
// into the A tile, all threads stage the matching 64x64 slice of the
// transformed activations X' in the B tile, and each wave then runs the MFMAs
// for its 32 rows x 64 columns.  Both LDS tiles are [rows][64] fp16 with
// 16-byte chunks XOR-swizzled by row, so the MFMA operand reads (16 rows x
// one 16-byte chunk) hit distinct banks.  The dense contraction is where
// MFMA belongs; the decode stays on the VALU and the LUT on the LDS.
#include "gemv_impl.hpp"
#include "qdec_device.hpp"
#include "qdec_internal.hpp"

namespace qdec {

constexpr int GEMM_THREADS = 256;

__device__ __forceinline__ int gemm_swz(int r, int k) {
  return r * 128 + ((((k >> 3) ^ (r & 7)) << 4) | ((k & 7) << 1));
}

template <int CODE, int K>
__host__ __device__ inline size_t gemm_lds_bytes(int Q) {
  const size_t tab = ((size_t)gemv_table_words<CODE, K>(Q) * 4 + 15) & ~(size_t)15;
  return tab + 128 * 128 + 64 * 128;
}

template <int CODE, int K>
__global__ __launch_bounds__(GEMM_THREADS) void gemm_kernel(GemmArgs a) {
  constexpr int COPIES = GemvTable<CODE>::COPIES;
  extern __shared__ __align__(16) uint32_t smem[];
  const size_t tab_bytes = ((size_t)gemv_table_words<CODE, K>(a.L.Q) * 4 + 15) & ~(size_t)15;
  uint32_t* tab = smem;
  char* As = reinterpret_cast<char*>(smem) + tab_bytes;
  char* Bs = As + 128 * 128;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, q = tid & 7, tl = lane >> 3;
  const int64_t m = a.L.m, n = a.L.n;
  const int npanels = (int)(m / 128);
  const int panel = blockIdx.x % npanels;
  const int split = blockIdx.x / npanels;
  const int n0 = blockIdx.y * 64;
  const int64_t ntc = n >> 4;
  const int64_t niter = (ntc + 3) >> 2;
  const int64_t per = (niter + a.ksplit - 1) / a.ksplit;
  const int64_t it0 = split * per;
  const int64_t it1 = (it0 + per) < niter ? (it0 + per) : niter;

  if constexpr (CODE == HYB) fill_signed_table<COPIES>(tab, a.L.lut, a.L.Q, tid, GEMM_THREADS);
  if constexpr (CODE == VQ) fill_plain_table<COPIES>(tab, a.L.lut, 1 << (2 * K), tid, GEMM_THREADS);
  if constexpr (CODE == NUQ) fill_plain_table<1>(tab, a.L.lut, 1 << K, tid, GEMM_THREADS);
  __syncthreads();

  const uint32_t* tabc = tab + (lane & (COPIES - 1));
  float4v acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = float4v{0.f, 0.f, 0.f, 0.f};

  for (int64_t it = it0; it < it1; ++it) {
    // ---- decode one tile column per wave into the A tile ----
    const int64_t tc = it * 4 + wave;
    uint32_t out[16];
    uint32_t w[K + 1];
#pragma unroll
    for (int i = 0; i <= K; ++i) w[i] = 0u;
    if (tc < ntc) load_words<K>(a.L.codes + ((panel * ntc + tc) * 8) * (8 * K) + lane * K, w);
    w[K] = next_lane_word(w[0], lane);
    if (tc < ntc) {
      float gs[2] = {0.f, 0.f};
      if constexpr (CODE == NUQ) {
        const int64_t gstride = n / a.L.group;
        const int64_t g = (tc * 16) / a.L.group;
        const int64_t row0 = (int64_t)panel * 128 + tl * 16 + 2 * q;
        gs[0] = h2f(a.L.gscale[row0 * gstride + g]);
        gs[1] = h2f(a.L.gscale[(row0 + 1) * gstride + g]);
      }
      lane_decode_exact<CODE, K, COPIES>(w, tabc, a.L.qshift, gs, out);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) out[i] = 0u;
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row = tl * 16 + 2 * q + r;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        *reinterpret_cast<uint4*>(As + gemm_swz(row, wave * 16 + 8 * h)) =
            make_uint4(out[8 * r + 4 * h], out[8 * r + 4 * h + 1], out[8 * r + 4 * h + 2],
                       out[8 * r + 4 * h + 3]);
      }
    }
    // ---- stage X' [n0 .. n0+64) x [it*64 .. it*64+64) in the B tile ----
#pragma unroll
    for (int rep = 0; rep < 2; ++rep) {
      const int c = tid + rep * GEMM_THREADS;
      const int bb = c >> 3, ch = c & 7;
      const int64_t kcol = it * 64 + ch * 8;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (n0 + bb < a.b && kcol < n)
        v = *reinterpret_cast<const uint4*>(a.xr + (int64_t)(n0 + bb) * n + kcol);
      *reinterpret_cast<uint4*>(Bs + gemm_swz(bb, ch * 8)) = v;
    }
    __syncthreads();
    // ---- MFMA: wave rows [32w, 32w+32) x 64 batch columns, K = 64 ----
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int kk = ks * 32 + 8 * (lane >> 4);
      half8v af[2], bf[4];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        af[mb] = *reinterpret_cast<const half8v*>(As + gemm_swz(wave * 32 + mb * 16 + (lane & 15), kk));
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        bf[nb] = *reinterpret_cast<const half8v*>(Bs + gemm_swz(nb * 16 + (lane & 15), kk));
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[mb], bf[nb], acc[mb][nb], 0, 0, 0);
    }
    __syncthreads();
  }

  // ---- epilogue: D[i][j] with i = 4*(lane/16) + e, j = lane % 16 ----
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int bb = n0 + nb * 16 + (lane & 15);
      if (bb >= a.b) continue;
      const int64_t row = (int64_t)panel * 128 + wave * 32 + mb * 16 + 4 * (lane >> 4);
      float* dst = a.z + (int64_t)bb * m + row;
      if (a.ksplit == 1) {
        *reinterpret_cast<float4v*>(dst) = acc[mb][nb];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          __hip_atomic_fetch_add(dst + e, acc[mb][nb][e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

template <int CODE, int K>
static hipError_t launch_gemm_t(const GemmArgs& a, hipStream_t stream) {
  const size_t lds = gemm_lds_bytes<CODE, K>(a.L.Q);
  static size_t have = 0;
  const hipError_t e =
      ensure_dynamic_lds(reinterpret_cast<const void*>(&gemm_kernel<CODE, K>), lds, &have);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)((a.L.m / 128) * a.ksplit), (unsigned)((a.b + 63) / 64));
  hipLaunchKernelGGL((gemm_kernel<CODE, K>), grid, dim3(GEMM_THREADS), lds, stream, a);
  return hipGetLastError();
}

template <int CODE>
static hipError_t launch_gemm_code(const GemmArgs& a, hipStream_t stream) {
  switch (a.L.k) {
    case 2: return launch_gemm_t<CODE, 2>(a, stream);
    case 3: return launch_gemm_t<CODE, 3>(a, stream);
    case 4: return launch_gemm_t<CODE, 4>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream) {
  switch (a.L.code) {
    case HYB: return launch_gemm_code<HYB>(a, stream);
    case MAD1: return launch_gemm_code<MAD1>(a, stream);
    case INST3: return launch_gemm_code<INST3>(a, stream);
    case NUQ: return launch_gemm_code<NUQ>(a, stream);
    case VQ: return launch_gemm_code<VQ>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

bool gemm_supported(int code, int k) { return code >= HYB && code <= VQ && k >= 2 && k <= 4; }

}  // namespace qdec
