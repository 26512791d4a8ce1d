// C ABI of the qdec library: argument validation, workspace sizing, kernel
// selection and launch on the caller's stream.  Everything a call can reject
// is rejected here, on the host, before any device work is queued.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

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

hipError_t launch_gemv_mma_hyb(const MmaArgs& a, int kv, hipStream_t stream);
hipError_t launch_gemv_mma_other(const MmaArgs& a, int code, int kv, hipStream_t stream);

hipError_t launch_gemv_mma(const MmaArgs& a, int code, int kv, hipStream_t stream) {
  if (code == HYB) return launch_gemv_mma_hyb(a, kv, stream);
  return launch_gemv_mma_other(a, code, kv, stream);
}

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
// Largest dimension and code size a layer may have: every kernel addresses a
// layer's codes, and a call's slices, through 32-bit buffer offsets.
constexpr int64_t kMaxDim = (int64_t)1 << 20;
constexpr int64_t kMaxCodeBytes = (int64_t)1 << 31;

// Tuning overrides for measurements, compiled in only with -DQDEC_TUNING: the
// product build reads no environment variable on any path.
int tuning(const char* name) {
#ifdef QDEC_TUNING
  const char* e = getenv(name);
  return e ? atoi(e) : -1;
#else
  (void)name;
  return -1;
#endif
}

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
  if (L->m > kMaxDim || L->n > kMaxDim) return QDEC_EUNSUPPORTED;
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
  // code bytes of the whole layer (both parts) below 2 GiB
  {
    const int64_t m_a = L->m_a ? L->m_a : L->m;
    const int64_t bits = m_a * L->n * kv_a / L->V + (L->m - m_a) * L->n * kv_b / L->V;
    if (bits / 8 >= kMaxCodeBytes) return QDEC_EUNSUPPORTED;
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
// Test hook (qdec_debug_fail_launches): calls that reach the launch stage
// while it is positive take one from it and return QDEC_EHIP, launching
// nothing.
std::atomic<int> g_fail_launches{0};
int injected_failure();

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return QDEC_ENODEV;
  }
  // 0 unknown, 1 ok, -1 not gfx950; concurrent first calls may both query
  // the properties and store the same answer
  static std::atomic<int> state[64];
  if (dev < 64) {
    const int st = state[dev].load(std::memory_order_relaxed);
    if (st) return st > 0 ? injected_failure() : QDEC_ENODEV;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return QDEC_ENODEV;
  }
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) state[dev].store(ok ? 1 : -1, std::memory_order_relaxed);
  return ok ? injected_failure() : QDEC_ENODEV;
}

thread_local char g_last_error[256] = "no error";

int injected_failure() {
  int n = g_fail_launches.load(std::memory_order_relaxed);
  while (n > 0) {
    if (g_fail_launches.compare_exchange_weak(n, n - 1, std::memory_order_relaxed)) {
      snprintf(g_last_error, sizeof g_last_error, "injected launch failure (qdec_debug_fail_launches)");
      return QDEC_EHIP;
    }
  }
  return QDEC_OK;
}

int status_of(hipError_t e) {
  if (e == hipSuccess) return QDEC_OK;
  snprintf(g_last_error, sizeof g_last_error, "%s (%d)", hipGetErrorString(e), (int)e);
  return QDEC_EHIP;
}

}  // namespace

namespace qdec {
// Batch columns per workgroup of the batched path: 16 up to 16 columns (a
// quarter of the X' staging, B-fragment reads and MFMAs of a 64-column
// tile), else 64.
int gemm_batch_tile(int64_t b) {
  const int forced = tuning("QDEC_GEMM_NBT");
  if (forced == 16 || forced == 64) return forced;
  return b <= 16 ? 16 : 64;
}

// K halves per workgroup of the batched path: 2 (a 16-wave workgroup, one
// per CU, adding its halves in LDS: half as many K-split slices to write and
// to sum) where the panel pairs alone come near filling the chip -- at least
// 32 per batch tile -- and each half still gets 8 steps of 64 columns; else
// 1 (8-wave workgroups, two per CU).  Only the 64-column tile is built with
// two halves.
int gemm_ksub(int64_t m, int64_t n, int64_t b) {
  const int64_t tile = gemm_batch_tile(b);
  if (tile != 64) return 1;
  const int forced = tuning("QDEC_GEMM_KSUB");
  if (forced == 1 || forced == 2) return forced;
  const int64_t groups = (m / 128 + GEMM_PANELS - 1) / GEMM_PANELS, nbt = (b + tile - 1) / tile;
  const int64_t niter = (n / 16 + 3) / 4;
  return (groups * nbt >= 32 && niter >= 16) ? 2 : 1;
}

// K-split factor of the batched path: at most as many workgroups as the
// CUs hold at once (two 8-wave or one 16-wave workgroup each).
int gemm_ksplit(int64_t m, int64_t n, int64_t b) {
  int forced = tuning("QDEC_GEMM_KSPLIT");
  if (forced > 16) forced = 16;
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
// the dot-product GEMV.  The GEMV's time grows with its batch-column
// template NB (the batch rounded up to 2, 4 or 8: one v_dot2 per weight pair
// and column), the batched path's hardly at all up to 16 columns; measured
// over the Llama-8B shapes at b = 2 .. 8, the batched path wins where
// NB * m * n >= 4e8: 14336x4096 and 4096x14336 from 5 columns, 28672x4096
// from 3, 6144x4096 and 4096x4096 never.
bool gemv_via_gemm(int64_t m, int64_t n, int64_t b) {
  if (b < 2) return false;
  const int forced = tuning("QDEC_GEMV_MFMA");
  if (forced >= 0) return forced != 0;
  const int64_t nb = b <= 2 ? 2 : b <= 4 ? 4 : 8;   // the GEMV's column template
  return (double)nb * (double)m * (double)n >= 4e8;
}

// Whether a one-column GEMV on the dot-product kernel takes the separate
// input transform: every workgroup of the fused path transforms its own
// chunk, reading all B_in values of x for it.
bool gemv_separate_rht(int64_t b) {
  if (b > 1) return true;
  return tuning("QDEC_GEMV_XR") == 1;
}

int gemv_chunk(int64_t m, int64_t n, int64_t b) {
  const int forced = tuning("QDEC_GEMV_KC");
  if (forced >= 64 && forced <= 2048 && (forced & (forced - 1)) == 0) {
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

// ---------------------------------------------------------------------------
// The one-column MFMA GEMV (gemv_mma_kernel): planning on the host.

// Workgroups of one round: one per CU of an MI355X.  A fixed number, so that
// workspace sizes do not depend on the device (fewer CUs only mean more
// rounds).
constexpr int MMA_CUS = 256;

// Input-column range of a unit for a set of row parts (one K range for all
// of a call's parts, so that the two parts of a half-TCQ layer write the
// same slices): KR is 512, 1024 or a multiple of 2048 (the steps of a
// quarter, KR / 256, are then 2, 4 or a multiple of 8, which the kernel's
// code ring divides).  Chosen to minimise the rounds of units times the
// steps of a unit plus one (the cost of a unit's reduction, about a step).
int mma_krange(const int64_t* m, const int64_t* n, int count) {
  const int forced = tuning("QDEC_MMA_KR");
  if (forced == 512 || forced == 1024 || (forced >= 2048 && forced % 2048 == 0)) return forced;
  int64_t nmax = 0;
  for (int i = 0; i < count; ++i) nmax = n[i] > nmax ? n[i] : nmax;
  int best = 512;
  int64_t best_cost = -1;
  for (int KR = 512; KR <= 2048 * ((nmax + 2047) / 2048); KR = KR < 2048 ? 2 * KR : KR + 2048) {
    int64_t U = 0;
    for (int i = 0; i < count; ++i) U += (m[i] / 128) * ((n[i] + KR - 1) / KR);
    const int64_t cost = ((U + MMA_CUS - 1) / MMA_CUS) * (KR / 256 + 1);
    if (best_cost < 0 || cost < best_cost) {
      best = KR;
      best_cost = cost;
    }
  }
  return best;
}

// LDS carve-up of one launch: the table (or, before it is built, the x
// transform's fp32 scratch), x' (xs_elems fp16: the widest row padded to
// whole ranges, or one range), and the cross-wave sums; the scratch holds
// scr_elems fp32.  HYB takes 32 table copies where they fit, else fewer, but
// at least 2^(13 - Q) (and 4) for the decode's table addresses (more than
// 32 below Q = 8: a 64 KiB table).  false if nothing fits.
bool mma_lds(int code, int kv, int Qmin, int Qmax, int64_t xs_elems, int64_t scr_elems, MmaArgs* a) {
  if (xs_elems > MMA_MAX_N || scr_elems > MMA_MAX_N) return false;
  const size_t xs = (size_t)xs_elems * 2;
  const size_t scratch = ((size_t)padded_words((int)scr_elems) * 4 + 15) & ~(size_t)15;
  const size_t red = (size_t)MMA_RED_BYTES;
  // the transform's scratch gets an area of its own where it fits (the
  // table is then built while x is in flight), else it borrows the table's
  auto fits = [&](size_t table) -> bool {
    table = (table + 15) & ~(size_t)15;
    if (table + xs + red + scratch <= (size_t)LDS_MAX_BYTES && table > 0) {
      a->tab_bytes = (int)table;
      a->xs_off = (int)table;
      a->red_off = (int)(table + xs);
      a->scr_off = (int)(table + xs + red);
      a->lds_bytes = (int)(table + xs + red + scratch);
      return true;
    }
    const size_t tab = table > scratch ? table : scratch;
    if (tab + xs + red > (size_t)LDS_MAX_BYTES) return false;
    a->tab_bytes = (int)tab;
    a->xs_off = (int)tab;
    a->red_off = (int)(tab + xs);
    a->scr_off = 0;
    a->lds_bytes = (int)(tab + xs + red);
    return true;
  };
  if (code == HYB) {
    // at least 2^(13 - Q) copies for every layer: entry stride 4 c >= 2^(15 - Q),
    // the decode's table address being the masked hash times 4 c / 2^(15 - Q)
    const int cmin = Qmin >= 11 ? 4 : 1 << (13 - Qmin);
    for (int c = cmin > 32 ? cmin : 32; c >= 4 && c >= cmin; c /= 2) {
      if (fits((size_t)c * (2u << Qmax) * 4)) {
        a->copies = c;
        a->cshift = 31 - __builtin_clz((unsigned)(4 * c));
        return true;
      }
    }
    return false;
  }
  a->copies = 1;
  a->cshift = 2;
  size_t table = 0;
  if (code == HYB1) table = (size_t)8 * (2u << Qmax) * 4;
  if (code == VQ) table = (size_t)8 * (1u << kv) * 4;
  if (code == NUQ) table = (size_t)(1u << kv) * 4;
  if (code == LUT) table = (size_t)1 << 17;
  return fits(table);
}

// A call of the MFMA GEMV: its launches (row parts grouped by code and
// width) and the finisher over its layers.
struct MmaCall {
  int nlaunch = 0;
  MmaArgs launch[2 * GEMV_GROUP_MAX];
  int code[2 * GEMV_GROUP_MAX], kv[2 * GEMV_GROUP_MAX];
  FinishArgs fin;
};

// Slices of layer l of a call start at slice_off[l] bytes: ceil(n / KR)
// slices of m fp32 each.
size_t mma_slice_bytes(int64_t m, int64_t n, int KR) {
  return align256((size_t)((n + KR - 1) / KR) * (size_t)m * 4);
}

// Plan the MFMA GEMV over `count` layers (each one or two row parts); false
// when a launch's LDS would not fit (the caller takes another path).
bool plan_mma(const LayerArgs* L, const LayerParts* P, int count, const uint16_t* const* x,
              uint16_t* const* y, char* slices, MmaCall* c) {
  int64_t pm[2 * GEMV_GROUP_MAX], pn[2 * GEMV_GROUP_MAX];
  int np = 0;
  for (int l = 0; l < count; ++l)
    for (int p = 0; p < P[l].count; ++p) {
      pm[np] = P[l].part[p].m;
      pn[np] = P[l].part[p].n;
      ++np;
    }
  const int KR = mma_krange(pm, pn, np);
  // slices per layer, and the finisher entries
  size_t off = 0;
  float* zl[GEMV_GROUP_MAX];
  c->fin.nl = count;
  int fwg = 0;
  for (int l = 0; l < count; ++l) {
    zl[l] = reinterpret_cast<float*>(slices + off);
    off += mma_slice_bytes(L[l].m, L[l].n, KR);
    FinishLayer& f = c->fin.lay[l];
    f.z = zl[l];
    f.slice_stride = L[l].m;
    f.m = L[l].m;
    f.y = y[l];
    f.sign_out = L[l].sign_out;
    f.nslices = (int)((L[l].n + KR - 1) / KR);
    f.Bo = L[l].had_out;
    f.b = 1;
    int64_t p2 = L[l].m & -L[l].m;                  // largest power of two dividing m
    int64_t R = p2 < 1024 ? p2 : 1024;
    if (R < f.Bo) R = f.Bo;
    f.rows_wg = (int)R;
    const double norm = L[l].code == MAD1 ? (double)(float)(1.0 / sqrt(21845.0)) : 1.0;
    f.mult = (float)((double)L[l].scale * norm / sqrt((double)L[l].had_out));
    f.wg0 = fwg;
    fwg += (int)(L[l].m / R);
  }
  // launches: parts of one (code, kv), at most GEMV_GROUP_MAX each
  c->nlaunch = 0;
  bool used[GEMV_GROUP_MAX][2] = {};
  for (int l0 = 0; l0 < count; ++l0)
    for (int p0 = 0; p0 < P[l0].count; ++p0) {
      if (used[l0][p0]) continue;
      // one launch per (code, width, Q): a HYB launch's table copies must
      // suit every Q in it (mma_lds)
      const int code = P[l0].part[p0].code, kv = P[l0].part[p0].kv, Q0 = P[l0].part[p0].Q;
      MmaArgs& a = c->launch[c->nlaunch];
      a.nl = 0;
      int Qmax = 0, Qmin = 16;
      int64_t xs_elems = 0, scr_elems = 0;
      for (int l = l0; l < count; ++l)
        for (int p = 0; p < P[l].count; ++p) {
          if (used[l][p] || P[l].part[p].code != code || P[l].part[p].kv != kv || P[l].part[p].Q != Q0 ||
              a.nl == GEMV_GROUP_MAX)
            continue;
          used[l][p] = true;
          MmaLayer& ml = a.lay[a.nl++];
          ml.L = P[l].part[p];
          ml.x = x[l];
          ml.z = zl[l];
          ml.slice_stride = L[l].m;
          ml.row0 = P[l].row0[p];
          ml.nr = (int)((ml.L.n + KR - 1) / KR);
          ml.KR = KR;
          ml.units = (int)(ml.L.m / 128) * ml.nr;
          // x' of one range per workgroup where the range is whole
          // Hadamard blocks: each workgroup transforms KR values, not n
          ml.xmode = ml.nr > 1 && KR % ml.L.had_in == 0 ? 1 : 0;
          const int64_t xe = ml.xmode ? KR : (int64_t)ml.nr * KR, se = ml.xmode ? KR : ml.L.n;
          if (ml.L.Q > Qmax) Qmax = ml.L.Q;
          if (ml.L.Q < Qmin) Qmin = ml.L.Q;
          if (xe > xs_elems) xs_elems = xe;
          if (se > scr_elems) scr_elems = se;
        }
      if (!mma_lds(code, kv, Qmin, Qmax, xs_elems, scr_elems, &a)) return false;
      // workgroups: one per unit when they fit one round, else shared out
      // in proportion to the units (at least one per part; a multiple of
      // the ranges where each workgroup keeps one range)
      int64_t U = 0;
      for (int i = 0; i < a.nl; ++i) U += a.lay[i].units;
      int wg = 0;
      if (U <= MMA_CUS) {
        for (int i = 0; i < a.nl; ++i) {
          a.lay[i].wg0 = wg;
          a.lay[i].nwg = a.lay[i].units;
          wg += a.lay[i].units;
        }
      } else {
        int nw[GEMV_GROUP_MAX], tot = 0;
        for (int i = 0; i < a.nl; ++i) {
          const int g = a.lay[i].xmode ? a.lay[i].nr : 1;
          nw[i] = (int)((int64_t)MMA_CUS * a.lay[i].units / U);
          nw[i] -= nw[i] % g;
          if (nw[i] < g) nw[i] = g;
          if (nw[i] > a.lay[i].units) nw[i] = a.lay[i].units;
          tot += nw[i];
        }
        while (tot < MMA_CUS) {   // the spare workgroups to the part with the most rounds
          int bi = -1;
          int64_t br = 0;
          for (int i = 0; i < a.nl; ++i) {
            const int g = a.lay[i].xmode ? a.lay[i].nr : 1;
            const int64_t r = (a.lay[i].units + nw[i] - 1) / nw[i];
            if (nw[i] + g <= a.lay[i].units && tot + g <= MMA_CUS && r > br) { br = r; bi = i; }
          }
          if (bi < 0) break;
          const int g = a.lay[bi].xmode ? a.lay[bi].nr : 1;
          nw[bi] += g;
          tot += g;
        }
        for (int i = 0; i < a.nl; ++i) {
          a.lay[i].wg0 = wg;
          a.lay[i].nwg = nw[i];
          wg += nw[i];
        }
      }
      c->code[c->nlaunch] = code;
      c->kv[c->nlaunch] = kv;
      ++c->nlaunch;
    }
  return true;
}

// Whether a one-column qdec_gemv takes the MFMA GEMV.  Its workgroups pay a
// fixed start (the x transform, a 128 KiB table) that the dot-product
// kernel's smaller workgroups do not, and win it back on layers from about
// 4096x4096 up: measured at 2 bits per weight (us per call, MFMA / dot
// product) 4096x4096 12.1 / 12.3, 4096x14336 15.9 / 20.4, 14336x4096
// 17.6 / 19.1, 28672x4096 22.4 / 26.2, 28672x8192 33.6 / 40.1.  Tuning
// override QDEC_GEMV_MMA = 0 / 1.
// The other codes stay on the dot-product kernel, whose decoders are cheaper
// there (NUQ and VQ look up a weight pair in one read of a small table; the
// MFMA operands need each weight as an exact fp16 value): 4096x14336 NUQ
// 3-bit 29.6 / 21.7, VQ 4-bit 22.6 / 16.3.
bool gemv_use_mma(int code, int64_t m, int64_t n) {
  const int forced = tuning("QDEC_GEMV_MMA");
  if (forced >= 0) return forced != 0;
  return code == HYB && (double)m * (double)n >= 1.6e7;
}

// Bytes of slices any call of up to b columns on an m x n layer writes: the
// MFMA GEMV's ranges (one column), the dot-product GEMV's chunks, or the
// batched path's K splits.
size_t gemv_slice_bytes(int64_t m, int64_t n, int64_t b) {
  size_t most = 0;
  for (int64_t bb = 1; bb <= b; ++bb) {
    size_t s;
    if (gemv_via_gemm(m, n, bb)) {
      s = (size_t)(gemm_ksplit(m, n, bb) * bb * m) * 4;
    } else {
      const int64_t kc = gemv_chunk(m, n, bb);
      s = (size_t)(((n + kc - 1) / kc) * bb * m) * 4;
    }
    if (s > most) most = s;
  }
  const int64_t mm[1] = {m}, nn[1] = {n};
  const size_t mma = mma_slice_bytes(m, n, mma_krange(mm, nn, 1));
  return most > mma ? most : mma;
}

size_t gemv_ws_bytes(int64_t m, int64_t n, int64_t b) { return gemv_ws_layout(m, n, b).total; }
}  // namespace qdec

extern "C" {

uint32_t qdec_abi_version(void) { return QDEC_ABI_VERSION; }

int qdec_debug_fail_launches(int32_t count) {
  if (count < 0) return QDEC_EINVAL;
  g_fail_launches.store(count, std::memory_order_relaxed);
  return QDEC_OK;
}

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
  if (n > kMaxDim || rows > kMaxDim || rows * n * 4 >= ((int64_t)1 << 32)) return QDEC_EUNSUPPORTED;
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

// Launch a planned MFMA GEMV call: its launches, then the finisher.
static int run_mma(const MmaCall& c, hipStream_t s) {
  for (int i = 0; i < c.nlaunch; ++i) {
    const hipError_t e = launch_gemv_mma(c.launch[i], c.code[i], c.kv[i], s);
    if (e != hipSuccess) return status_of(e);
  }
  return status_of(launch_gemv_finish(c.fin, s));
}

int qdec_gemv(const qdec_layer* layer, const uint16_t* x, uint16_t* y, int64_t batch, void* ws,
              size_t ws_bytes, void* stream) {
  LayerArgs L;
  LayerParts parts;
  int st = check_layer(layer, &L, &parts);
  if (st) return st;
  if (!x || !y || !aligned(x, 16) || !aligned(y, 8)) return QDEC_EINVAL;
  if (batch < 1) return QDEC_EINVAL;
  if (batch > 8) return QDEC_EUNSUPPORTED;
  if (overlap(x, (size_t)(batch * L.n) * 2, y, (size_t)(batch * L.m) * 2)) return QDEC_EINVAL;
  const GemvWs wl = gemv_ws_layout(L.m, L.n, batch);
  const size_t need = wl.total;
  if (!ws || !aligned(ws, 256) || ws_bytes < need) return QDEC_EWORKSPACE;
  if (overlap(ws, need, x, (size_t)(batch * L.n) * 2) || overlap(ws, need, y, (size_t)(batch * L.m) * 2))
    return QDEC_EINVAL;
  const int d = check_device();
  if (d) return d;
  uint16_t* xr = (uint16_t*)((char*)ws + wl.xr);
  float* z = (float*)((char*)ws + wl.z);
  const hipStream_t s = (hipStream_t)stream;
  if (batch == 1 && gemv_use_mma(L.code, L.m, L.n)) {
    thread_local MmaCall call;
    if (plan_mma(&L, &parts, 1, &x, &y, (char*)z, &call)) return run_mma(call, s);
  }
  if (gemv_via_gemm(L.m, L.n, batch)) return run_batched(L, parts, x, y, batch, xr, z, s);
  // the dot-product GEMV: one slice per input chunk
  GemvArgs a;
  a.L = L;
  a.x = x;
  a.y = y;
  a.b = (int)batch;
  a.z = z;
  a.row0 = 0;
  a.mz = L.m;
  a.xr = nullptr;
  a.Kc = gemv_chunk(L.m, L.n, batch);
  a.nchunks = (int)((L.n + a.Kc - 1) / a.Kc);
  a.U = gemv_unit_rows(L.had_out);
  const double norm = L.code == MAD1 ? (double)(float)(1.0 / sqrt(21845.0)) : 1.0;
  a.out_mult = (float)((double)L.scale * norm / sqrt((double)L.had_out));
  if (gemv_separate_rht(batch)) {
    // x' = RHT_in(x) once, by the RHT kernel into the workspace, then the
    // GEMV loads its slices (otherwise, with one batch column, the GEMV's
    // workgroups transform their own chunks: no extra launch)
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
    const hipError_t e = launch_rht(r, s);
    if (e != hipSuccess) return status_of(e);
    a.xr = xr;
  }
  FinishArgs f;
  f.nl = 1;
  f.lay[0].z = z;
  f.lay[0].slice_stride = batch * L.m;
  f.lay[0].m = L.m;
  f.lay[0].y = y;
  f.lay[0].sign_out = L.sign_out;
  f.lay[0].nslices = a.nchunks;
  f.lay[0].Bo = L.had_out;
  f.lay[0].b = (int)batch;
  {
    int64_t p2 = L.m & -L.m;
    int64_t R = p2 < 1024 ? p2 : 1024;
    if (R < L.had_out) R = L.had_out;
    f.lay[0].rows_wg = (int)R;
  }
  f.lay[0].mult = a.out_mult;
  f.lay[0].wg0 = 0;
  // the decode-and-multiply kernel per row part (each writes its rows of
  // every chunk's slice), or both parts of a half-TCQ layer in one launch
  // where that pair is built, then the output side
  if (parts.count == 2 && !a.xr && L.code == HYB) {
    GemvArgs ah = a;
    ah.L = parts.part[0];
    ah.row0 = parts.row0[0];
    ah.codes_b = parts.part[1].codes;
    ah.m_b = parts.part[1].m;
    ah.row0_b = parts.row0[1];
    ah.grid_a = (int)((parts.part[0].m / 128) * a.nchunks);
    const hipError_t e = launch_gemv_hyb_two_parts(ah, parts.part[1].kv, s);
    if (e == hipSuccess) return status_of(launch_gemv_finish(f, s));
    if (e != hipErrorNotSupported) return status_of(e);
  }
  for (int p = 0; p < parts.count; ++p) {
    GemvArgs ap = a;
    ap.L = parts.part[p];
    ap.row0 = parts.row0[p];
    const hipError_t e = launch_gemv(ap, s);
    if (e != hipSuccess) return status_of(e);
  }
  return status_of(launch_gemv_finish(f, s));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// qdec_gemv_noalloc: qdec_gemv with its workspace in a static device array of
// this file, for callers that cannot allocate.  Each device the library runs
// on holds its own copy of the array until the process ends; its address on
// a device is looked up once (hipGetSymbolAddress, with that device current)
// and kept per device.  Host code never passes the array's name itself to a
// kernel or a copy: on the host that name is only a stand-in, not a device
// address.
namespace {
constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
std::atomic<void*> g_scratch_ptr[64];

// The device address of this device's scratch, or nullptr (status in *st).
void* scratch_address(int* st) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    *st = QDEC_ENODEV;
    return nullptr;
  }
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) {
    *st = status_of(e != hipSuccess ? e : hipErrorInvalidSymbol);
    return nullptr;
  }
  // concurrent first calls store the same address
  g_scratch_ptr[dev].store(p, std::memory_order_release);
  return p;
}
}  // namespace

extern "C" {

size_t qdec_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

int qdec_gemv_noalloc(const qdec_layer* layer, const uint16_t* x, uint16_t* y, int64_t batch, void* stream) {
  LayerArgs L;
  const int st = check_layer(layer, &L);
  if (st) return st;
  if (batch < 1) return QDEC_EINVAL;
  if (batch > 8) return QDEC_EUNSUPPORTED;
  if (gemv_ws_bytes(L.m, L.n, batch) > kNoAllocScratchBytes) return QDEC_EWORKSPACE;
  const int d = check_device();
  if (d) return d;
  int ast = QDEC_OK;
  void* ws = scratch_address(&ast);
  if (!ws) return ast;
  return qdec_gemv(layer, x, y, batch, ws, kNoAllocScratchBytes, stream);
}

size_t qdec_gemv_group_workspace_bytes(const qdec_layer* const* layers, int32_t count) {
  if (!layers || count < 1 || count > GEMV_GROUP_MAX) return 0;
  int64_t pm[2 * GEMV_GROUP_MAX], pn[2 * GEMV_GROUP_MAX];
  LayerArgs L[GEMV_GROUP_MAX];
  LayerParts P[GEMV_GROUP_MAX];
  int np = 0;
  for (int l = 0; l < count; ++l) {
    if (check_layer(layers[l], &L[l], &P[l]) != QDEC_OK) return 0;
    for (int p = 0; p < P[l].count; ++p) {
      pm[np] = P[l].part[p].m;
      pn[np] = P[l].part[p].n;
      ++np;
    }
  }
  const int KR = mma_krange(pm, pn, np);
  size_t total = 0;
  for (int l = 0; l < count; ++l) total += mma_slice_bytes(L[l].m, L[l].n, KR);
  return total;
}

int qdec_gemv_group(const qdec_layer* const* layers, int32_t count, const uint16_t* const* x,
                    uint16_t* const* y, void* ws, size_t ws_bytes, void* stream) {
  if (!layers || !x || !y || count < 1) return QDEC_EINVAL;
  if (count > GEMV_GROUP_MAX) return QDEC_EUNSUPPORTED;
  LayerArgs L[GEMV_GROUP_MAX];
  LayerParts P[GEMV_GROUP_MAX];
  for (int l = 0; l < count; ++l) {
    const int st = check_layer(layers[l], &L[l], &P[l]);
    if (st) return st;
    if (!x[l] || !y[l] || !aligned(x[l], 16) || !aligned(y[l], 8)) return QDEC_EINVAL;
  }
  // no output may overlap an input or another output
  for (int l = 0; l < count; ++l)
    for (int j = 0; j < count; ++j) {
      if (overlap(x[j], (size_t)L[j].n * 2, y[l], (size_t)L[l].m * 2)) return QDEC_EINVAL;
      if (j != l && overlap(y[j], (size_t)L[j].m * 2, y[l], (size_t)L[l].m * 2)) return QDEC_EINVAL;
    }
  const size_t need = qdec_gemv_group_workspace_bytes(layers, count);
  if (!ws || !aligned(ws, 256) || ws_bytes < need) return QDEC_EWORKSPACE;
  for (int l = 0; l < count; ++l)
    if (overlap(ws, need, x[l], (size_t)L[l].n * 2) || overlap(ws, need, y[l], (size_t)L[l].m * 2))
      return QDEC_EINVAL;
  const int d = check_device();
  if (d) return d;
  thread_local MmaCall call;
  if (!plan_mma(L, P, count, x, y, (char*)ws, &call)) return QDEC_EUNSUPPORTED;
  return run_mma(call, (hipStream_t)stream);
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
