// Host/device interface between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "qdec.h"

namespace qdec {

// A validated layer, as the kernels see it: one part of rows (a half-TCQ
// layer is launched part by part, each with its own codes, rows and kV).
struct LayerArgs {
  const uint32_t* codes;
  const uint32_t* lut;
  const uint16_t* gscale;
  const uint32_t* sign_in;
  const uint32_t* sign_out;
  int64_t m, n;        // rows of this part, columns
  int code, kv, Q, qshift, group;   // kv: bits per trellis step (or index bits)
  int had_in, had_out;
  float scale;
};

// The row parts of a layer: rows [0, m_a) at kv, then [m_a, m) at kv_b
// (half-TCQ), each a panel-ordered tile array of its own.
struct LayerParts {
  int count;
  LayerArgs part[2];
  int64_t row0[2];     // first output row of each part
  int64_t tile0[2];    // storage index of each part's first tile
};

struct GemvArgs {
  LayerArgs L;
  const uint16_t* x;   // [b][n] fp16
  uint16_t* y;         // [b][m] fp16
  int b;
  const uint16_t* xr;  // precomputed x' = RHT_in(x), fp16 [b][n], or NULL
  float* z;            // [b][mz] fp32 split-K accumulator (workspace; zero on entry, left zero)
  int64_t row0;        // first row of L (a part of the layer) in the layer
  int64_t mz;          // rows of the whole layer (z's row stride)
  // one launch over both parts of a half-TCQ layer: the second part
  const uint32_t* codes_b = nullptr;
  int64_t m_b = 0, row0_b = 0;
  int grid_a = 0;      // workgroups of the first part
  int Kc;              // columns per chunk (power of two, 64 .. 2048; Kc * b <= 4096)
  int nchunks;         // ceil(n / Kc)
  int U;               // rows per output block = max(had_out, 128)
  float out_mult;      // layer scale x code factor / sqrt(had_out)
};

struct DecodeArgs {
  LayerArgs L;
  int64_t first, count;
  uint16_t* out;       // [count][256] fp16
};

struct RhtArgs {
  const void* in;
  void* out;
  int in_f32, out_f32;
  int64_t rows, n;
  int block;
  const uint32_t* signs;
  int mode;
  float mult;          // scale / sqrt(block)
  int nsum = 1;        // fp32 input: sum of nsum slices ...
  int64_t sum_stride = 0;  // ... sum_stride elements apart
};

struct GemmArgs {
  LayerArgs L;
  const uint16_t* xr;  // [b][n] fp16, input RHT already applied
  float* z;            // [ksplit][b][mz] fp32 partial sums, one slice per K split
  int64_t row0;        // first row of L (a part of the layer) in the layer
  int64_t mz;          // rows of the whole layer
  int b;
  int ksplit;          // K split factor
  int ksub;            // K halves per workgroup (1 or 2, gemm_ksub)
  int nbt;             // batch columns per workgroup: 16 or 64 (gemm_batch_tile)
};

// The encoder: one part of a layer, its targets and its output codes.
struct EncodeArgs {
  LayerArgs L;         // the part (its kv, rows m and tile count)
  const float* w;      // [layer m][n] fp32 targets (row-major, whole layer)
  int64_t row0;        // first row of the part in w
  uint32_t* codes;     // the part's output code words
  uint32_t* bp;        // workspace: [ENCODE_GRID][256/V][1024] backpointer words
  int64_t ntiles;      // tiles of the part
};
// Workgroups of the encoder (one tile each at a time, 1024 threads).
constexpr int ENCODE_GRID = 256;
inline size_t encode_ws_bytes(int V) { return (size_t)ENCODE_GRID * (256 / V) * 1024 * 4; }

// Workspace layout of qdec_gemv: the fp32 accumulator z (must start at zero;
// left zero), sized for the largest batch (8 columns) whatever the call's
// batch, so that no call's scratch (x', K-split slices) lands where a call of
// another batch expects zeros; then the fp16 x' [b][n] of the separate-RHT
// path.
inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
constexpr int GEMV_MAX_BATCH = 8;
inline int gemv_unit_rows(int had_out) { return had_out > 128 ? had_out : 128; }
// Input-chunk width of the fused GEMV: about two (panel, chunk) workgroups
// per CU, chunks a power of two in [64, 2048].
int gemv_chunk(int64_t m, int64_t n, int64_t b);
struct GemvWs {
  size_t z, xr, total;
};
inline GemvWs gemv_ws_layout(int64_t m, int64_t n, int64_t b) {
  GemvWs l;
  l.z = 0;
  l.xr = align256((size_t)(GEMV_MAX_BATCH * m) * 4);
  l.total = l.xr + align256((size_t)(b * n) * 2);
  return l;
}
// Workspace layout of qdec_gemm: X' (fp16 [b][n]) then the K-split partial
// sums Z (fp32 [ksplit][b][m]).  Nothing in it needs initialising.
// Batched-path geometry: a workgroup of 8 waves covers two panels of 128
// rows (four waves each) and shares one lookup table of 16 copies and the
// staged X'; two such workgroups fit a CU (80 KiB of LDS each for a
// 2^9-pair table).
constexpr int GEMM_WAVES = 8;
constexpr int GEMM_PANELS = GEMM_WAVES / 4;
constexpr int GEMM_COPIES = 16;
constexpr int GEMM_WG_PER_CU = 2;
constexpr size_t GEMM_LDS_BYTES = 160 * 1024;      // LDS of one CU
int gemm_batch_tile(int64_t b);
int gemm_ksub(int64_t m, int64_t n, int64_t b);
int gemm_ksplit(int64_t m, int64_t n, int64_t b);
inline size_t gemm_ws_bytes(int64_t m, int64_t n, int64_t b) {
  return align256((size_t)(b * n) * 2) + align256((size_t)(gemm_ksplit(m, n, b) * b * m) * 4);
}

// Raise a kernel's dynamic-LDS limit to `bytes` when a launch needs more than
// the default 64 KiB; *have caches the largest limit set so far.
inline hipError_t ensure_dynamic_lds(const void* kernel, size_t bytes, size_t* have) {
  if (bytes <= 65536 || bytes <= *have) return hipSuccess;
  const hipError_t e =
      hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) *have = bytes;
  return e;
}

// Kernel launchers (return hipSuccess or the launch error).
// launch_gemv: the decode-and-multiply kernel of one part (adds into z);
// launch_gemv_finish: the output side over the whole layer.
hipError_t launch_gemv(const GemvArgs& a, hipStream_t stream);
hipError_t launch_gemv_finish(const GemvArgs& a, hipStream_t stream);
// both parts of a half-TCQ layer in one launch (b = 1, transform in the
// workgroups); hipErrorNotSupported when that width pair is not built
hipError_t launch_gemv_hyb_two_parts(const GemvArgs& a, int kvb, hipStream_t stream);
hipError_t launch_decode_tile(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_rht(const RhtArgs& a, hipStream_t stream);
hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream);
hipError_t launch_encode(const EncodeArgs& a, hipStream_t stream);
// Output side of the batched path: y = fp16(s_out .* (mult * H z)); z zeroed.
hipError_t launch_rht_out_f32(const float* z, int nsum, uint16_t* y, int64_t rows, int64_t m, int block,
                              const uint32_t* signs, float mult, hipStream_t stream);

}  // namespace qdec
