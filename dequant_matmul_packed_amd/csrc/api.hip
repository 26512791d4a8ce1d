// C ABI of the qdec library: argument validation, workspace sizing, kernel
// selection and launch on the caller's stream.  Everything a call can reject
// is rejected here, on the host, before any device work is queued.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "qdec.h"
#include "qdec_device.hpp"
#include "qdec_internal.hpp"

namespace qdec {
hipError_t launch_gemv_hyb(const GemvArgs& a, hipStream_t stream);
hipError_t launch_gemv_mad1(const GemvArgs& a, hipStream_t stream);
hipError_t launch_gemv_inst3(const GemvArgs& a, hipStream_t stream);
hipError_t launch_gemv_nuq(const GemvArgs& a, hipStream_t stream);
hipError_t launch_gemv_vq(const GemvArgs& a, hipStream_t stream);
hipError_t launch_gemv_hyb1(const GemvArgs& a, hipStream_t stream);
hipError_t launch_gemv_lut(const GemvArgs& a, hipStream_t stream);

hipError_t launch_gemv(const GemvArgs& a, hipStream_t stream) {
  switch (a.L.code) {
    case HYB: return launch_gemv_hyb(a, stream);
    case MAD1: return launch_gemv_mad1(a, stream);
    case INST3: return launch_gemv_inst3(a, stream);
    case NUQ: return launch_gemv_nuq(a, stream);
    case VQ: return launch_gemv_vq(a, stream);
    case HYB1: return launch_gemv_hyb1(a, stream);
    case LUT: return launch_gemv_lut(a, stream);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace qdec

using namespace qdec;

namespace {

constexpr int kMaxHadamard = 16384;

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool is_trellis(int code) {
  return code == QDEC_CODE_HYB || code == QDEC_CODE_1MAD || code == QDEC_CODE_3INST || code == QDEC_CODE_LUT;
}

// Format-level validation; EUNSUPPORTED for valid combinations not built.
// On success *out describes the whole layer with the first part's width and
// *parts the row parts (one, or two for half-TCQ).
int check_layer(const qdec_layer* L, LayerArgs* out, LayerParts* parts = nullptr) {
  if (!L || L->abi_version != QDEC_ABI_VERSION) return QDEC_EINVAL;
  if (L->m <= 0 || L->n <= 0 || (L->m % 128) || (L->n % 16)) return QDEC_EINVAL;
  if (L->kv == 0) {
    if (L->k < 1 || L->k > 8) return QDEC_EINVAL;
  } else if (L->k != 0 || !is_trellis(L->code)) {
    return QDEC_EINVAL;
  }
  if (L->m_a) {
    if (!is_trellis(L->code) || L->m_a < 0 || L->m_a >= L->m || (L->m_a % 128) || L->kv_b < 1)
      return QDEC_EINVAL;
  } else if (L->kv_b) {
    return QDEC_EINVAL;
  }
  const int kv_a = L->kv ? L->kv : L->k * L->V;
  const int kv_b = L->m_a ? L->kv_b : kv_a;
  if (kv_a < 1 || kv_b < 1 || kv_a > L->L || kv_b > L->L) return QDEC_EINVAL;
  if (!L->codes || !aligned(L->codes, 16)) return QDEC_EINVAL;
  if (!is_pow2(L->had_in) || L->n % L->had_in) return QDEC_EINVAL;
  if (!is_pow2(L->had_out) || L->m % L->had_out) return QDEC_EINVAL;
  if (!isfinite(L->layer_scale)) return QDEC_EINVAL;
  switch (L->code) {
    case QDEC_CODE_HYB:
      if (L->L != 16 || (L->V != 1 && L->V != 2) || L->Q < 1 || L->Q > 15 || !L->lut) return QDEC_EINVAL;
      if (L->Q > 11) return QDEC_EUNSUPPORTED;   // LDS table would exceed the budget
      break;
    case QDEC_CODE_LUT:
      if (L->L != 16 || L->V != 1 || !L->lut) return QDEC_EINVAL;
      break;
    case QDEC_CODE_1MAD:
    case QDEC_CODE_3INST:
      if (L->L != 16 || L->V != 1) return QDEC_EINVAL;
      break;
    case QDEC_CODE_NUQ:
      if (L->V != 1 || L->L != L->k || !L->lut || !L->group_scale) return QDEC_EINVAL;
      if (L->group < 16 || L->group % 16 || L->n % L->group) return QDEC_EINVAL;
      break;
    case QDEC_CODE_VQ:
      if (L->V != 2 || L->L != 2 * L->k || !L->lut) return QDEC_EINVAL;
      break;
    default:
      return QDEC_EINVAL;
  }
  const int kcode = (L->code == QDEC_CODE_HYB && L->V == 1) ? HYB1 : L->code;
  if (!kv_built(kcode, kv_a) || !kv_built(kcode, kv_b)) return QDEC_EUNSUPPORTED;
  if (L->had_in > kMaxHadamard || L->had_out > kMaxHadamard) return QDEC_EUNSUPPORTED;
  if (out) {
    out->codes = L->codes;
    out->lut = L->lut;
    out->gscale = L->group_scale;
    out->sign_in = L->sign_in;
    out->sign_out = L->sign_out;
    out->m = L->m;
    out->n = L->n;
    out->code = kcode;
    out->kv = kv_a;
    out->Q = L->code == QDEC_CODE_HYB ? L->Q : 0;   // both V = 1 and V = 2
    out->qshift = L->code == QDEC_CODE_HYB ? 15 - L->Q : 0;
    out->group = L->code == QDEC_CODE_NUQ ? L->group : 1;
    out->had_in = L->had_in;
    out->had_out = L->had_out;
    out->scale = L->layer_scale;
    if (parts) {
      // a tile holds (256/V) steps of kV bits: 8 kV / V words
      const int64_t m_a = L->m_a ? L->m_a : L->m;
      parts->count = L->m_a ? 2 : 1;
      parts->part[0] = *out;
      parts->part[0].m = m_a;
      parts->row0[0] = 0;
      parts->tile0[0] = 0;
      if (L->m_a) {
        const int64_t tiles_a = (m_a / 16) * (L->n / 16);
        parts->part[1] = *out;
        parts->part[1].m = L->m - m_a;
        parts->part[1].kv = kv_b;
        parts->part[1].codes = L->codes + tiles_a * (8 * kv_a / L->V);
        parts->row0[1] = m_a;
        parts->tile0[1] = tiles_a;
      }
    }
  }
  return QDEC_OK;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

// The current device must be a gfx950 part; checked once per device.
int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return QDEC_ENODEV;
  }
  static int state[64];   // 0 unknown, 1 ok, -1 not gfx950
  if (dev < 64 && state[dev]) return state[dev] > 0 ? QDEC_OK : QDEC_ENODEV;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return QDEC_ENODEV;
  }
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) state[dev] = ok ? 1 : -1;
  return ok ? QDEC_OK : QDEC_ENODEV;
}

thread_local char g_last_error[256] = "no error";

int status_of(hipError_t e) {
  if (e == hipSuccess) return QDEC_OK;
  snprintf(g_last_error, sizeof g_last_error, "%s (%d)", hipGetErrorString(e), (int)e);
  return QDEC_EHIP;
}

}  // namespace

namespace qdec {
// Batch columns per workgroup of the batched path: 16 up to 16 columns (a
// quarter of the X' staging, B-fragment reads and MFMAs of a 64-column
// tile), else 64.  Tuning override QDEC_GEMM_NBT = 16 / 64.
int gemm_batch_tile(int64_t b) {
  static int forced = -1;
  if (forced < 0) {
    const char* ev = getenv("QDEC_GEMM_NBT");
    forced = ev ? atoi(ev) : 0;
    if (forced != 16 && forced != 64) forced = 0;
  }
  if (forced) return forced;
  return b <= 16 ? 16 : 64;
}

// K halves per workgroup of the batched path: 2 (a 16-wave workgroup, one
// per CU, adding its halves in LDS: half as many K-split slices to write and
// to sum) where the panel pairs alone come near filling the chip -- at least
// 32 per batch tile -- and each half still gets 8 steps of 64 columns; else
// 1 (8-wave workgroups, two per CU).  Only the 64-column tile is built with
// two halves.  Tuning override QDEC_GEMM_KSUB = 1 / 2.
int gemm_ksub(int64_t m, int64_t n, int64_t b) {
  static int forced = -1;
  if (forced < 0) {
    const char* ev = getenv("QDEC_GEMM_KSUB");
    forced = ev ? atoi(ev) : 0;
    if (forced != 1 && forced != 2) forced = 0;
  }
  const int64_t tile = gemm_batch_tile(b);
  if (tile != 64) return 1;
  if (forced) return forced;
  const int64_t groups = (m / 128 + GEMM_PANELS - 1) / GEMM_PANELS, nbt = (b + tile - 1) / tile;
  const int64_t niter = (n / 16 + 3) / 4;
  return (groups * nbt >= 32 && niter >= 16) ? 2 : 1;
}

// K-split factor of the batched path: at most as many workgroups as the
// CUs hold at once (two 8-wave or one 16-wave workgroup each).
int gemm_ksplit(int64_t m, int64_t n, int64_t b) {
  static int forced = -1;
  if (forced < 0) {
    // tuning override for measurements: QDEC_GEMM_KSPLIT = 1 .. 16
    const char* ev = getenv("QDEC_GEMM_KSPLIT");
    forced = ev ? atoi(ev) : 0;
    if (forced > 16) forced = 16;
  }
  const int64_t tile = gemm_batch_tile(b);
  const int64_t groups = (m / 128 + GEMM_PANELS - 1) / GEMM_PANELS, nbt = (b + tile - 1) / tile;
  const int64_t niter = (n / 16 + 3) / 4;
  const int ksub = gemm_ksub(m, n, b);
  const int64_t slots = 256 * (ksub == 2 ? 1 : GEMM_WG_PER_CU);
  int64_t ks = forced > 0 ? forced : slots / (groups * nbt);
  const int64_t most = ksub == 2 ? niter / 8 : niter;   // a half keeps at least 4 steps
  if (ks > most) ks = most;
  if (ks > 16) ks = 16;
  if (ks < 1) ks = 1;
  return (int)ks;
}

// Whether qdec_gemv runs a product of 2 to 8 columns on the batched MFMA
// path (input RHT, gemm_kernel with 16-column tiles, output RHT) instead of
// the fused GEMV.  The GEMV's time grows with its batch-column template NB
// (the batch rounded up to 2, 4 or 8: one v_dot2 per weight pair and
// column), the batched path's hardly at all up to 16 columns; measured over
// the Llama-8B shapes at b = 2 .. 8, the batched path wins where
// NB * m * n >= 4e8: 14336x4096 and 4096x14336 from 5 columns, 28672x4096
// from 3, 6144x4096 and 4096x4096 never.  Tuning override
// QDEC_GEMV_MFMA = 0 / 1 (1: every call of 2 or more columns).
bool gemv_via_gemm(int64_t m, int64_t n, int64_t b) {
  static int forced = -2;
  if (forced == -2) {
    const char* e = getenv("QDEC_GEMV_MFMA");
    forced = e ? (atoi(e) != 0) : -1;
  }
  if (b < 2) return false;
  if (forced >= 0) return forced != 0;
  const int64_t nb = b <= 2 ? 2 : b <= 4 ? 4 : 8;   // the GEMV's column template
  return (double)nb * (double)m * (double)n >= 4e8;
}

// Workspace of qdec_gemv: the GEMV's accumulator and x' slot, then (on the
// MFMA path) the K-split slices, after the accumulator so that it stays
// zero for later calls of other batches on the same workspace.
size_t gemv_ws_bytes(int64_t m, int64_t n, int64_t b) {
  const size_t base = gemv_ws_layout(m, n, b).total;
  if (!gemv_via_gemm(m, n, b)) return base;
  return base + align256((size_t)(gemm_ksplit(m, n, b) * b * m) * 4);
}

// Whether a one-column GEMV takes the separate input transform: every
// workgroup of the fused path transforms its own chunk, reading all B_in
// values of x for it.  Tuning override QDEC_GEMV_XR = 0 / 1.
bool gemv_separate_rht(int64_t m, int64_t n, int64_t b, int had_in) {
  static int forced = -2;
  if (forced == -2) {
    const char* e = getenv("QDEC_GEMV_XR");
    forced = e ? (atoi(e) != 0) : -1;
  }
  if (b > 1) return true;
  if (forced >= 0) return forced != 0;
  (void)m; (void)n; (void)had_in;
  return false;
}

int gemv_chunk(int64_t m, int64_t n, int64_t b) {
  static int forced = -1;
  if (forced < 0) {
    // tuning override for measurements: QDEC_GEMV_KC = 64 .. 2048
    const char* e = getenv("QDEC_GEMV_KC");
    const int v = e ? atoi(e) : 0;
    forced = (v >= 64 && v <= 2048 && (v & (v - 1)) == 0) ? v : 0;
  }
  if (forced > 0) {
    int kc = forced;
    while (kc > 64 && kc * b > 4096) kc /= 2;
    return kc;
  }
  // about two resident (panel, chunk) workgroups per CU; a chunk's x' slice
  // (b x Kc fp32) must fit the LDS scratch: Kc * b <= 4096.  With one batch
  // column every workgroup transforms its own chunk of x, which costs B_in
  // loads whatever the chunk width: chunks start at 256 columns there (the
  // widest that takes the wave-level transform).
  const int64_t npanels = m / 128;
  int kc = b == 1 ? 256 : 64;
  while (kc < 2048 && kc * 2 * b <= 4096 && npanels * ((n + 2 * kc - 1) / (2 * kc)) >= 448) kc *= 2;
  return kc;
}
}  // namespace qdec

extern "C" {

uint32_t qdec_abi_version(void) { return QDEC_ABI_VERSION; }

const char* qdec_last_error(void) { return g_last_error; }

const char* qdec_status_string(int status) {
  switch (status) {
    case QDEC_OK: return "ok";
    case QDEC_EINVAL: return "invalid argument";
    case QDEC_EUNSUPPORTED: return "unsupported configuration";
    case QDEC_EWORKSPACE: return "workspace missing, misaligned or too small";
    case QDEC_EHIP: return "HIP runtime error";
    case QDEC_ENODEV: return "no gfx950 device";
    default: return "unknown status";
  }
}

size_t qdec_workspace_bytes(const qdec_layer* layer, int64_t batch, int32_t op) {
  LayerArgs L;
  if (check_layer(layer, &L) != QDEC_OK) return 0;
  if (op == QDEC_OP_GEMV) {
    if (batch < 1 || batch > 8) return 0;
    return gemv_ws_bytes(L.m, L.n, batch);
  }
  if (op == QDEC_OP_GEMM) {
    if (batch < 1 || batch > 256) return 0;
    return gemm_ws_bytes(L.m, L.n, batch);
  }
  if (op == QDEC_OP_ENCODE) {
    if (batch != 1) return 0;
    if (L.code != HYB && L.code != HYB1 && L.code != MAD1 && L.code != INST3) return 0;
    return encode_ws_bytes(code_V(L.code));
  }
  return 0;
}

int qdec_rht(const void* in, int32_t in_dtype, void* out, int32_t out_dtype, int64_t rows,
             int64_t n, int32_t block, const uint32_t* signs, int32_t mode, float scale,
             void* stream) {
  if (!in || !out || rows < 0 || n <= 0) return QDEC_EINVAL;
  if ((in_dtype != 0 && in_dtype != 1) || (out_dtype != 0 && out_dtype != 1)) return QDEC_EINVAL;
  if (mode != 0 && mode != 1) return QDEC_EINVAL;
  if (!is_pow2(block) || n % block) return QDEC_EINVAL;
  if (!isfinite(scale)) return QDEC_EINVAL;
  if (block > kMaxHadamard) return QDEC_EUNSUPPORTED;
  const size_t ib = (size_t)(rows * n) * (in_dtype ? 4 : 2);
  const size_t ob = (size_t)(rows * n) * (out_dtype ? 4 : 2);
  if (in != out && overlap(in, ib, out, ob)) return QDEC_EINVAL;
  if (in == out && in_dtype != out_dtype) return QDEC_EINVAL;
  const int d = check_device();
  if (d) return d;
  RhtArgs a;
  a.in = in;
  a.out = out;
  a.in_f32 = in_dtype;
  a.out_f32 = out_dtype;
  a.rows = rows;
  a.n = n;
  a.block = block;
  a.signs = signs;
  a.mode = mode;
  a.mult = (float)((double)scale / sqrt((double)block));
  return status_of(launch_rht(a, (hipStream_t)stream));
}

static int run_batched(const LayerArgs& L, const LayerParts& parts, const uint16_t* x, uint16_t* y,
                       int64_t batch, uint16_t* xr, float* z, hipStream_t s);

int qdec_gemv(const qdec_layer* layer, const uint16_t* x, uint16_t* y, int64_t batch, void* ws,
              size_t ws_bytes, void* stream) {
  LayerArgs L;
  LayerParts parts;
  int st = check_layer(layer, &L, &parts);
  if (st) return st;
  if (!x || !y || !aligned(x, 16) || !aligned(y, 4)) return QDEC_EINVAL;
  if (batch < 1) return QDEC_EINVAL;
  if (batch > 8) return QDEC_EUNSUPPORTED;
  if (overlap(x, (size_t)(batch * L.n) * 2, y, (size_t)(batch * L.m) * 2)) return QDEC_EINVAL;
  const int Kc = gemv_chunk(L.m, L.n, batch);
  const GemvWs wl = gemv_ws_layout(L.m, L.n, batch);
  const size_t need = gemv_ws_bytes(L.m, L.n, batch);
  if (!ws || !aligned(ws, 256) || ws_bytes < need) return QDEC_EWORKSPACE;
  if (overlap(ws, need, x, (size_t)(batch * L.n) * 2) || overlap(ws, need, y, (size_t)(batch * L.m) * 2))
    return QDEC_EINVAL;
  const int d = check_device();
  if (d) return d;
  if (gemv_via_gemm(L.m, L.n, batch))
    return run_batched(L, parts, x, y, batch, (uint16_t*)((char*)ws + wl.xr),
                       (float*)((char*)ws + wl.total), (hipStream_t)stream);
  GemvArgs a;
  a.L = L;
  a.x = x;
  a.y = y;
  a.b = (int)batch;
  a.z = (float*)((char*)ws + wl.z);
  a.row0 = 0;
  a.mz = L.m;
  a.xr = nullptr;
  a.Kc = Kc;
  a.nchunks = (int)((L.n + a.Kc - 1) / a.Kc);
  a.U = gemv_unit_rows(L.had_out);
  const double factor = L.code == QDEC_CODE_1MAD ? 1.0 / sqrt(21845.0) : 1.0;
  // the 1MAD matmul path multiplies by the fp32 normaliser, as the decode does
  const double f32norm = (double)(float)factor;
  a.out_mult = (float)((double)L.scale * f32norm / sqrt((double)L.had_out));
  if (gemv_separate_rht(L.m, L.n, batch, L.had_in)) {
    // x' = RHT_in(x) once, by the RHT kernel into the workspace, then the
    // GEMV loads its slices (otherwise, with one batch column, the GEMV's
    // workgroups transform their own chunks: no extra launch)
    uint16_t* xr = (uint16_t*)((char*)ws + wl.xr);
    RhtArgs r;
    r.in = x;
    r.out = xr;
    r.in_f32 = 0;
    r.out_f32 = 0;
    r.rows = batch;
    r.n = L.n;
    r.block = L.had_in;
    r.signs = L.sign_in;
    r.mode = 0;
    r.mult = (float)(1.0 / sqrt((double)L.had_in));
    const hipError_t e = launch_rht(r, (hipStream_t)stream);
    if (e != hipSuccess) return status_of(e);
    a.xr = xr;
  }
  // the decode-and-multiply kernel per row part (each adds into z), or both
  // parts of a half-TCQ layer in one launch where that pair is built, then
  // the output side over the whole layer
  if (parts.count == 2 && !a.xr && L.code == HYB) {
    GemvArgs ah = a;
    ah.L = parts.part[0];
    ah.row0 = parts.row0[0];
    ah.codes_b = parts.part[1].codes;
    ah.m_b = parts.part[1].m;
    ah.row0_b = parts.row0[1];
    ah.grid_a = (int)((parts.part[0].m / 128) * a.nchunks);
    const hipError_t e = launch_gemv_hyb_two_parts(ah, parts.part[1].kv, (hipStream_t)stream);
    if (e == hipSuccess) return status_of(launch_gemv_finish(a, (hipStream_t)stream));
    if (e != hipErrorNotSupported) return status_of(e);
  }
  for (int p = 0; p < parts.count; ++p) {
    GemvArgs ap = a;
    ap.L = parts.part[p];
    ap.row0 = parts.row0[p];
    const hipError_t e = launch_gemv(ap, (hipStream_t)stream);
    if (e != hipSuccess) return status_of(e);
  }
  return status_of(launch_gemv_finish(a, (hipStream_t)stream));
}

int qdec_gemm(const qdec_layer* layer, const uint16_t* x, uint16_t* y, int64_t batch, void* ws,
              size_t ws_bytes, void* stream) {
  LayerArgs L;
  LayerParts parts;
  int st = check_layer(layer, &L, &parts);
  if (st) return st;
  if (!x || !y || !aligned(x, 16) || !aligned(y, 4)) return QDEC_EINVAL;
  if (batch < 1) return QDEC_EINVAL;
  if (batch > 256) return QDEC_EUNSUPPORTED;
  if (overlap(x, (size_t)(batch * L.n) * 2, y, (size_t)(batch * L.m) * 2)) return QDEC_EINVAL;
  const size_t need = gemm_ws_bytes(L.m, L.n, batch);
  if (!ws || !aligned(ws, 256) || ws_bytes < need) return QDEC_EWORKSPACE;
  if (overlap(ws, need, x, (size_t)(batch * L.n) * 2) || overlap(ws, need, y, (size_t)(batch * L.m) * 2))
    return QDEC_EINVAL;
  const int d = check_device();
  if (d) return d;
  return run_batched(L, parts, x, y, batch, (uint16_t*)ws,
                     (float*)((char*)ws + align256((size_t)(batch * L.n) * 2)), (hipStream_t)stream);
}

// The batched path: X' = RHT_in(X) into xr, the K-split partial sums into
// z, then Y = RHT_out(sum of the slices).
static int run_batched(const LayerArgs& L, const LayerParts& parts, const uint16_t* x, uint16_t* y,
                       int64_t batch, uint16_t* xr, float* z, hipStream_t s) {
  // 1. X' = RHT_in(X), fp16
  RhtArgs r;
  r.in = x;
  r.out = xr;
  r.in_f32 = 0;
  r.out_f32 = 0;
  r.rows = batch;
  r.n = L.n;
  r.block = L.had_in;
  r.signs = L.sign_in;
  r.mode = 0;
  r.mult = (float)(1.0 / sqrt((double)L.had_in));
  hipError_t e = launch_rht(r, s);
  if (e != hipSuccess) return status_of(e);
  // 2. Z[split] = W_hat X'^T over each K split (fp32 slices, plain stores)
  GemmArgs g;
  g.xr = xr;
  g.z = z;
  g.mz = L.m;
  g.b = (int)batch;
  const int64_t ks = gemm_ksplit(L.m, L.n, batch);
  g.ksplit = (int)ks;
  g.ksub = gemm_ksub(L.m, L.n, batch);
  g.nbt = gemm_batch_tile(batch);
  for (int p = 0; p < parts.count; ++p) {   // each row part writes its rows of every slice
    g.L = parts.part[p];
    g.row0 = parts.row0[p];
    e = launch_gemm(g, s);
    if (e != hipSuccess) return status_of(e);
  }
  // 3. Y = s_out .* (scale/sqrt(B) H sum_split Z[split]), fp16
  e = launch_rht_out_f32(z, g.ksplit, y, batch, L.m, L.had_out, L.sign_out,
                         (float)((double)L.scale / sqrt((double)L.had_out)), s);
  return status_of(e);
}

int qdec_encode(const qdec_layer* layer, const float* w, uint32_t* codes, void* ws, size_t ws_bytes,
                void* stream) {
  LayerArgs L;
  LayerParts parts;
  int st = check_layer(layer, &L, &parts);
  if (st) return st;
  if (L.code != HYB && L.code != HYB1 && L.code != MAD1 && L.code != INST3) return QDEC_EUNSUPPORTED;
  if (!w || !codes || !aligned(w, 4) || !aligned(codes, 16)) return QDEC_EINVAL;
  const int V = code_V(L.code);
  const size_t wbytes = (size_t)(L.m * L.n) * 4;
  const int64_t last = parts.count - 1;
  const size_t cbytes = (size_t)((parts.part[last].codes - L.codes) +
                                 (parts.part[last].m / 16) * (L.n / 16) * (8 * parts.part[last].kv / V)) * 4;
  if (overlap(w, wbytes, codes, cbytes)) return QDEC_EINVAL;
  const size_t need = encode_ws_bytes(V);
  if (!ws || !aligned(ws, 256) || ws_bytes < need) return QDEC_EWORKSPACE;
  if (overlap(ws, need, w, wbytes) || overlap(ws, need, codes, cbytes)) return QDEC_EINVAL;
  const int d = check_device();
  if (d) return d;
  for (int p = 0; p < parts.count; ++p) {
    EncodeArgs a;
    a.L = parts.part[p];
    a.w = w;
    a.row0 = parts.row0[p];
    a.codes = codes + (parts.part[p].codes - L.codes);
    a.bp = (uint32_t*)ws;
    a.ntiles = (parts.part[p].m / 16) * (L.n / 16);
    const hipError_t e = launch_encode(a, (hipStream_t)stream);
    if (e != hipSuccess) return status_of(e);
  }
  return QDEC_OK;
}

int qdec_decode_tile(const qdec_layer* layer, int64_t first_tile, int64_t n_tiles, uint16_t* out,
                     void* stream) {
  LayerArgs L;
  LayerParts parts;
  int st = check_layer(layer, &L, &parts);
  if (st) return st;
  const int64_t total = (L.m / 16) * (L.n / 16);
  if (first_tile < 0 || n_tiles < 0 || first_tile + n_tiles > total) return QDEC_EINVAL;
  if (n_tiles > 0 && (!out || !aligned(out, 16))) return QDEC_EINVAL;
  if (n_tiles == 0) return QDEC_OK;
  const int d = check_device();
  if (d) return d;
  // the requested storage range, cut at the part boundary
  for (int p = 0; p < parts.count; ++p) {
    const int64_t t0 = parts.tile0[p];
    const int64_t t1 = t0 + (parts.part[p].m / 16) * (L.n / 16);
    const int64_t lo = first_tile > t0 ? first_tile : t0;
    const int64_t hi = first_tile + n_tiles < t1 ? first_tile + n_tiles : t1;
    if (lo >= hi) continue;
    DecodeArgs a;
    a.L = parts.part[p];
    a.first = lo - t0;
    a.count = hi - lo;
    a.out = out + (lo - first_tile) * 256;
    const hipError_t e = launch_decode_tile(a, (hipStream_t)stream);
    if (e != hipSuccess) return status_of(e);
  }
  return QDEC_OK;
}

}  // extern "C"
