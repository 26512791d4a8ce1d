// Host/device interface between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

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
  float* z;            // [nchunks][b][mz] fp32 partial sums, one slice per input chunk (plain stores)
  int64_t row0;        // first row of L (a part of the layer) in the layer
  int64_t mz;          // rows of the whole layer (z's row stride)
  // one launch over both parts of a half-TCQ layer: the second part
  const uint32_t* codes_b = nullptr;
  int64_t m_b = 0, row0_b = 0;
  int grid_a = 0;      // workgroups of the first part
  int Kc;              // columns per chunk (power of two, 64 .. 2048; Kc * b <= 4096)
  int nchunks;         // ceil(n / Kc)
  int U;               // rows per output block = max(had_out, 128)
  float out_mult;      // layer scale x code factor / sqrt(had_out) (applied by the finisher)
};

// Layers of one launch of a grouped call (independent products of one
// batch column, launched together).
constexpr int GEMV_GROUP_MAX = 8;

// Output side of qdec_gemv, one entry per layer: the K slices z hold, per
// 128-row panel, partial sums already multiplied by H_min(Bo,128); the
// finisher adds the slices in slice order, applies the cross-panel stages of
// H_Bo, mult and the output signs, and writes fp16 y.
struct FinishLayer {
  const float* z;          // slice 0: z[s * slice_stride + c * m + row]
  int64_t slice_stride;    // elements between slices
  int64_t m;               // rows (also the column stride inside a slice)
  uint16_t* y;             // [b][m] fp16
  const uint32_t* sign_out;
  int nslices, Bo, b;
  int rows_wg;             // rows per workgroup: a multiple of Bo dividing m
  float mult;
  int wg0;                 // first workgroup of this layer: (m / rows_wg) x b of them
};
// The layer bounds of a grouped launch, passed as the kernel's first eight
// arguments: the build preloads them into SGPRs at wave launch (kernarg
// preloading), so a workgroup finds its layer without a memory round trip
// and reads that layer's fields in one.  w[0] = the layer count, w[i] =
// the first workgroup of layer i (INT_MAX for i >= the count).
struct LayerBounds {
  int w[GEMV_GROUP_MAX];
};
#define QDEC_BOUNDS_PARAMS int nl_, int w1_, int w2_, int w3_, int w4_, int w5_, int w6_, int w7_
#define QDEC_BOUNDS_ARGS(b) (b).w[0], (b).w[1], (b).w[2], (b).w[3], (b).w[4], (b).w[5], (b).w[6], (b).w[7]
// the layer of workgroup bx: the count of layers 1 .. 7 starting at or below it
#define QDEC_LAYER_OF(bx)                                                                        \
  ((int)((bx) >= w1_) + (int)((bx) >= w2_) + (int)((bx) >= w3_) + (int)((bx) >= w4_) +           \
   (int)((bx) >= w5_) + (int)((bx) >= w6_) + (int)((bx) >= w7_))

struct FinishArgs {
  int nl;
  FinishLayer lay[GEMV_GROUP_MAX];
};

// The MFMA GEMV of one batch column (gemv_mma_kernel): one 16-wave
// workgroup per CU.  A unit of work is one 128-row panel x one range of KR
// input columns; the 16 waves are 4 row groups (32 rows) x 4 quarters of
// the range.  Each workgroup works on one layer of the launch: x' (of the
// whole row, or of the one range all its units share) and the layer's
// table stay in LDS while it walks its units.
struct MmaLayer {
  LayerArgs L;             // one row part of a layer
  const uint16_t* x;       // [n] fp16
  float* z;                // slice r of the layer at z + r * slice_stride (layer rows)
  int64_t slice_stride;
  int64_t row0;            // first row of the part in the layer
  int nr, KR;              // K ranges of KR columns (the last may be ragged)
  int wg0, nwg;            // workgroups [wg0, wg0 + nwg) of the launch work on this layer
  int units;               // (m / 128) x nr
  int xmode;               // x' in LDS: 0 the whole row; 1 one range per workgroup
                           // (nwg a multiple of nr; the range is whole Hadamard blocks)
};
constexpr int MMA_RED_BYTES = 2 * 4 * 128 * 4;   // two buffers: 4 quarters x 128 rows fp32
constexpr int MMA_MAX_N = 16384;                  // x' of a whole row in LDS (fp16)
struct MmaArgs {
  int nl;
  int tab_bytes;           // LDS: table (and the x transform's scratch) [0, tab_bytes)
  int xs_off;              // x' fp16 [npad] from here
  int red_off;             // the cross-wave sums from here
  int scr_off;             // the x transform's fp32 scratch, or 0: it borrows the table's area
  int lds_bytes;           // the whole carve-up
  int cshift;              // HYB: log2(4 x table copies)
  int copies;
  MmaLayer lay[GEMV_GROUP_MAX];
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

// Workspace layout of qdec_gemv: the fp16 x' [b][n] (the separate input
// transform), then the fp32 K-split slices of whichever path the call takes.
// Every slice a call reads it has written, so the contents on entry do not
// matter, and a workspace sized for a batch serves every smaller batch.
inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
constexpr int GEMV_MAX_BATCH = 8;
inline int gemv_unit_rows(int had_out) { return had_out > 128 ? had_out : 128; }
// Input-chunk width of the fused GEMV: about two (panel, chunk) workgroups
// per CU, chunks a power of two in [64, 2048].
int gemv_chunk(int64_t m, int64_t n, int64_t b);
// Bytes of slices any call of up to b columns on an m x n layer writes.
size_t gemv_slice_bytes(int64_t m, int64_t n, int64_t b);
struct GemvWs {
  size_t xr, z, total;
};
inline GemvWs gemv_ws_layout(int64_t m, int64_t n, int64_t b) {
  GemvWs l;
  l.xr = 0;
  l.z = align256((size_t)(b * n) * 2);
  l.total = l.z + align256(gemv_slice_bytes(m, n, b));
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

// A kernel's dynamic-LDS limit, raised once per device to all the LDS of a
// CU (160 KiB) that its static LDS leaves, when a launch needs more than the
// default 64 KiB.  The record is a bit per device, set atomically after the
// raise: concurrent callers may both raise it, which sets the same value
// twice (no lock, and never a lower limit after a higher one).
struct LdsLimit {
  std::atomic<uint64_t> devices{0};
};
constexpr int LDS_MAX_BYTES = 160 * 1024;
inline hipError_t ensure_dynamic_lds(const void* kernel, size_t bytes, LdsLimit* lim) {
  if (bytes <= 65536) return hipSuccess;
  if (bytes > (size_t)LDS_MAX_BYTES) return hipErrorInvalidValue;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
  if (bit && (lim->devices.load(std::memory_order_acquire) & bit)) return hipSuccess;
  hipFuncAttributes fa;
  e = hipFuncGetAttributes(&fa, kernel);
  if (e != hipSuccess) return e;
  const int avail = LDS_MAX_BYTES - (int)fa.sharedSizeBytes;
  if ((int)bytes > avail) return hipErrorInvalidValue;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, avail);
  if (e == hipSuccess && bit) lim->devices.fetch_or(bit, std::memory_order_release);
  return e;
}

// Kernel launchers (return hipSuccess or the launch error).
// launch_gemv: the decode-and-multiply kernel of one part (adds into z);
// launch_gemv_finish: the output side over the whole layer.
hipError_t launch_gemv(const GemvArgs& a, hipStream_t stream);
hipError_t launch_gemv_finish(const FinishArgs& a, hipStream_t stream);
// the MFMA GEMV of one batch column: all layers of `a` share the code and kV
hipError_t launch_gemv_mma(const MmaArgs& a, int code, int kv, hipStream_t stream);
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
