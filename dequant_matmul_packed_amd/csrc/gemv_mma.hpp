// Decode-and-multiply of one batch column on the matrix cores (qdec_gemv at
// b = 1, and every launch of qdec_gemv_group).
//
// Small-batch inference is memory bound, so the codes are streamed from HBM
// once and decoded on chip ("QTIP: Quantization with Trellises and
// Incoherence Processing", "QTIP's contribution (W1)").  On gfx950 the decode
// of a HYB weight pair is a handful of VALU instructions and one random LDS
// read, and at 2 bits per weight the LDS would have to serve one read per two
// weights at more than half its peak to keep up with HBM: the table layout
// and the issue slots decide the speed, not the multiply.  So this kernel
//  - keeps 32 copies of the signed HYB table (128 KiB at Q = 9), lane l
//    reading copy l % 32: every bank serves exactly two lanes of a wave, the
//    least a 64-lane read can cost;
//  - hands the multiply to the matrix cores: a lane's decoded weights are
//    directly the A operands of v_mfma_f32_16x16x32_f16 (the layout of the
//    batched kernel), and x' is the B operand; only column 0 of each 16x16
//    product is used, which costs matrix-core time the VALU does not pay;
//  - runs one 16-wave workgroup per CU that computes x' = RHT_in(x) once
//    (of the whole row, or, where all its units share one K range, of that
//    range only) and builds the table once, then walks its units of work,
//    so that those fixed costs are paid once per CU and layer instead of once
//    per (panel, chunk) as in the dot-product kernel.
//
// Work decomposition.  A unit is one panel of 128 output rows x one range of
// KR input columns.  Wave w takes row group rg = w % 4 (tile rows 2rg, 2rg+1
// of the panel: 32 rows) and quarter ks = w / 4 of the range (KR/4 columns,
// S = KR/256 steps of 64 columns).  Lane q of tile t = lane / 8 decodes the
// 32 weights of its tile (rows 2q, 2q+1) at tile (row tr = t % 2, column
// tc = t / 2) of the step, which makes lanes l, l+16, l+32, l+48 hold one
// weight row at four column offsets: the MFMA A-operand shape under a fixed
// row permutation.  Code words stream through a PF-deep register ring that
// runs on across unit boundaries.  At the end of a unit the four quarters'
// sums meet in LDS (double buffered by unit), the output-Hadamard stages
// inside the panel are applied, and the panel's 128 sums are stored (plain
// stores) into the range's fp32 slice; gemv_finish_kernel adds the slices
// in range order.
//
// A launch may hold several layers of one code, width and Q (a grouped call):
// workgroups [wg0, wg0 + nwg) take the units of layer l, unit u = local
// workgroup + i * nwg.  Every wave of a workgroup runs the same number of
// steps and meets every barrier; every global load is a buffer load issued
// unconditionally (switched off by its offset), and the unit stores are
// buffer stores switched off the same way, so no branch holds a memory
// operation.
#pragma once

#include "gemv_impl.hpp"
#include "qdec_device.hpp"
#include "qdec_internal.hpp"

namespace qdec {

constexpr int MMA_THREADS = 1024;

// Table copies of the codes other than HYB (HYB takes MmaArgs::copies).
template <int CODE>
struct MmaTable {
  static constexpr int COPIES = (CODE == VQ || CODE == HYB1) ? 8 : 1;
};

// HYB at V = 2 with the table at a run-time stride: entry e of the lane's
// copy at byte e << cshift of the table, which starts at LDS address 0
// (gemv_mma_kernel has no static LDS, so its dynamic block starts there);
// lb is the lane's copy, 4 (lane mod copies) bytes.  The signed index is
// h >> qshift of the 16-bit hash h, and cshift >= qshift (the host keeps at
// least 2^(qshift - 2) copies), so the address is (h & mask) * 2^(cshift -
// qshift) + lb: one v_mad_u32_u16 of the masked hash.  Where kV divides 16,
// steps t and t + 16/kV share one 32-bit window and one packed hash, both
// halves are masked by one v_and_b32, and the two mads take the high and
// the low half (op_sel).  Four VALU per two states besides the window.
typedef __attribute__((address_space(3))) const uint32_t lds_cu32;
template <int KV>
__device__ __forceinline__ void hyb_pairs_strided(const uint32_t* w, uint32_t lb, uint32_t mul, uint32_t mask2,
                                                  uint32_t* out) {
  auto rd = [&](uint32_t addr) { return *reinterpret_cast<lds_cu32*>((uintptr_t)addr); };
  if constexpr (16 % KV == 0) {
    constexpr int D = 16 / KV;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      if ((t / D) & 1) continue;
      uint32_t h2, a_first, a_second;
      asm("v_pk_mad_u16 %0, %1, %1, %1" : "=v"(h2) : "v"(window_raw<32>(w, t * KV)));
      const uint32_t hm = h2 & mask2;
      asm("v_mad_u32_u16 %0, %1, %2, %3 op_sel:[1,0,0,0]" : "=v"(a_first) : "v"(hm), "s"(mul), "v"(lb));
      asm("v_mad_u32_u16 %0, %1, %2, %3" : "=v"(a_second) : "v"(hm), "s"(mul), "v"(lb));
      out[t] = rd(a_first);
      out[t + D] = rd(a_second);
    }
  } else {
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      uint32_t a;
      const uint32_t hm = hyb_hash(window_raw<16>(w, t * KV)) & mask2;
      asm("v_mad_u32_u16 %0, %1, %2, %3" : "=v"(a) : "v"(hm), "s"(mul), "v"(lb));
      out[t] = rd(a);
    }
  }
}

// 1MAD on the matrix cores: the byte sum sigma of each state's LCG output is
// formed as the fp16 number 1024 + sigma (exponent 10 holds the integers
// exactly), and one packed fp16 subtraction of 1534 gives sigma - 510 exactly
// for two states.  The fp32 normaliser 1/sqrt(21845) multiplies the finished
// sums (in the finisher), so the weights differ from the decoded values only
// by the fp16 rounding of each product, as in the dot-product kernel.
template <int KV>
__device__ __forceinline__ void mad1_pairs_centred(const uint32_t* w, uint32_t* out) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t v0 = __builtin_amdgcn_sad_u8(mad1_lcg(window_at<16>(w, (2 * i) * KV)), 0u, 0x6400u);
    const uint32_t v1 = __builtin_amdgcn_sad_u8(mad1_lcg(window_at<16>(w, (2 * i + 1) * KV)), 0u, 0x6400u);
    const half2v c = as_h2(v0 | (v1 << 16)) - half2v{(_Float16)1534.0f, (_Float16)1534.0f};
    out[i] = __builtin_bit_cast(uint32_t, c);
  }
}

// The kernel body for layer li of the launch.  X0: a launch of one layer
// whose x' is the whole row, with the table, x, the input signs, n and Q
// passed as leading (preloaded) arguments, so that the x and table loads
// issue before the layer's other fields have been read from memory.
template <int CODE, int KV, int PF, bool X0>
__device__ __forceinline__ void gemv_mma_body(int li, const uint32_t* lut_p, const uint16_t* x_p,
                                              const uint32_t* sgin_p, int n_p, int Q_p, int xmode_p, int xb_p,
                                              int NL_p, int xs_off_, int red_off_, int scr_off_, int cshift_,
                                              int copies_, const MmaArgs& a) {
  using G = LaneGeom<CODE, KV>;
  constexpr int NW = G::NW;
  constexpr int CW = CODE == NUQ ? NW + 2 : NW;          // ring words per slot (+ NUQ scales)
  constexpr uint32_t TB = 4u * G::TILE_WORDS;            // bytes per tile
  extern __shared__ __align__(16) uint32_t smem[];
  char* lds = reinterpret_cast<char*>(smem);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave & 3, ks = wave >> 2;
  const int q = lane & 7, t8 = lane >> 3, tr = t8 & 1, tc = t8 >> 1;

  // x in 8-value chunks: local chunk c = tid + 1024 j of the row or the
  // range (at most 16384 values: 2 per thread)
  uint4 xv[2];
  uint32_t sw[2];
  auto issue_x = [&](const uint16_t* xg_, const uint32_t* sg_, int n_, int xbase_, int NL_) {
    const int nch8_ = n_ >> 3;
    const auto xrs = make_rsrc(xg_, (uint32_t)n_ * 2u);
    const auto srs = make_rsrc(sg_, sg_ ? (uint32_t)(((n_ + 31) >> 5) * 4) : 0u);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = tid + MMA_THREADS * j;
      const int gc = (xbase_ >> 3) + c;
      const bool ok = c < (NL_ >> 3) && gc < nch8_;
      xv[j] = buf_load_u4(xrs, ok ? (uint32_t)gc * 16u : BUF_OFF);
      sw[j] = buf_load_u32(srs, ok ? (uint32_t)((8 * gc) >> 5) * 4u : BUF_OFF);
    }
  };
  // HYB: the LUT word of each 16-byte run of the table this thread writes
  // (run w4 = tid + 1024 k holds 4 copies of signed entry (4 w4) / copies;
  // K8 = W4 / 1024 <= 8 runs per thread: at most 128 KiB), requested with x.
  // The host keeps copies * 2^Q >= 8192, so W4 is a multiple of 1024 and
  // run k's entry is e0 + step k with e0 = 4 tid / copies < step = 4096 /
  // copies <= 2^Q: its LUT word is e0 + (step k mod 2^Q), and whether it is
  // a sign-flipped entry (bit Q) does not depend on the thread.  One vector
  // offset and scalar offsets: no per-run address arithmetic.
  uint32_t lw[8];
  auto issue_lut = [&](const uint32_t* lut_, int Q_) {
    const int nlut_ = CODE == HYB ? (1 << Q_) : 0;
    const int lc_ = 31 - __builtin_clz((unsigned)copies_);
    const int step_ = 4096 >> lc_;
    const auto lrs = make_rsrc(lut_, (uint32_t)nlut_ * 4u);
    const uint32_t vo = (uint32_t)((tid << 2) >> lc_) * 4u;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      lw[k] = __builtin_amdgcn_raw_buffer_load_b32(lrs, vo, (uint32_t)((step_ * k) & (nlut_ - 1)) * 4u, 0);
  };
  if constexpr (X0) {
    issue_x(x_p, sgin_p, n_p, xb_p, NL_p);
    issue_lut(lut_p, Q_p);
  }

  // ---- this workgroup's layer (workgroup-uniform) ---------------------------
  const uint32_t* codes = a.lay[li].L.codes;
  const uint32_t* lut = X0 ? lut_p : a.lay[li].L.lut;
  const uint16_t* gscale = a.lay[li].L.gscale;
  const uint32_t* sign_in = X0 ? sgin_p : a.lay[li].L.sign_in;
  const int64_t mpart = a.lay[li].L.m;
  const int n = X0 ? n_p : (int)a.lay[li].L.n;
  const int qshift = a.lay[li].L.qshift, Q = X0 ? Q_p : a.lay[li].L.Q, group = a.lay[li].L.group;
  const int Bi = a.lay[li].L.had_in, Bo = a.lay[li].L.had_out;
  const uint16_t* xg = X0 ? x_p : a.lay[li].x;
  float* zl = a.lay[li].z;
  const int64_t sstride = a.lay[li].slice_stride, row0 = a.lay[li].row0;
  const int nr = a.lay[li].nr, KR = a.lay[li].KR;
  const int bl = (int)blockIdx.x - a.lay[li].wg0, nwg = a.lay[li].nwg, units = a.lay[li].units;

  const int xmode = X0 ? xmode_p : a.lay[li].xmode;
  // the layer's fields in one round of scalar loads (the compiler would
  // otherwise issue some only where they are first used, after the first
  // round has returned); the launch's LDS carve-up and table geometry come
  // preloaded with the layer bounds
  asm volatile("" ::"s"(codes), "s"(lut), "s"(gscale), "s"(sign_in), "s"(mpart), "s"(n), "s"(qshift), "s"(Q),
               "s"(group), "s"(Bi), "s"(Bo), "s"(xg), "s"(zl), "s"(sstride), "s"(row0), "s"(nr), "s"(KR), "s"(bl),
               "s"(nwg), "s"(units), "s"(xmode));
  const int ntc = n >> 4;                 // tile columns
  const int npanels = (int)(mpart >> 7);
  const int Kw = KR >> 2, S = Kw >> 6;    // columns and steps of a quarter
  // the units: with the whole row in LDS, unit u = bl + i nwg (panel u %
  // npanels, range u / npanels); with one range per workgroup (xmode 1; nwg
  // a multiple of nr), range bl % nr and panels bl / nr + i (nwg / nr)
  int my_units, dp, dr, cp0, cr0;
  if (xmode == 0) {
    my_units = bl < units ? (units - bl + nwg - 1) / nwg : 0;
    dp = nwg % npanels;
    dr = nwg / npanels;
    cp0 = bl % npanels;
    cr0 = bl / npanels;
  } else {
    dp = nwg / nr;
    dr = 0;
    cp0 = bl / nr;
    cr0 = bl % nr;
    my_units = cp0 < npanels ? (npanels - cp0 + dp - 1) / dp : 0;
  }
  const int T = my_units * S;             // steps of every wave (a multiple of PF)
  // x' in LDS: the whole row (xmode 0) or the workgroup's range only, local
  // column 0 being column xbase of the row
  const int xbase = xmode == 0 ? 0 : cr0 * KR;
  const int NL = xmode == 0 ? n : KR;     // x' values kept (zero past n)

  // ---- 0. every global load the set-up needs, and the first PF code steps ----
  if constexpr (!X0) {
    issue_x(xg, sign_in, n, xbase, NL);
    issue_lut(lut, Q);
  }
  const int nch8 = n >> 3;
  const int lc = 31 - __builtin_clz((unsigned)copies_);
  const int W4 = CODE == HYB ? (copies_ << (Q + 1)) >> 2 : 0;
  const int K8 = W4 >> 10;
  const int step = 4096 >> lc;
  // codes of the whole part through one resource (format sizes below 4 GiB)
  const auto crs = make_rsrc(codes, (uint32_t)((mpart >> 4) * ntc * (int64_t)TB));
  const uint32_t lane_part = (uint32_t)(tc * 8 + 2 * rg + tr) * TB + 4u * G::lane_word(q);
  // NUQ group scales of the lane's rows 2q, 2q+1 (fp16 [rows of the layer][n / group])
  const int gstride = CODE == NUQ ? n / group : 0;
  const auto grs = make_rsrc(gscale, CODE == NUQ ? (uint32_t)((row0 + mpart) * gstride * 2) : 0u);
  const int64_t grow_l = row0 + (2 * rg + tr) * 16 + 2 * q;   // + panel * 128

  // the prefetch pointer: unit k of this workgroup, step s in it, its panel
  // and range (scalar, advanced one step at a time)
  int pk = 0, ps = 0, pp = cp0, pr = cr0;
  auto load_step = [&](uint32_t* slot) {
    const int cbase = ((pr * KR + ks * Kw) >> 4) + 4 * ps;   // tile column of tc = 0
    const bool ok = pk < my_units && cbase + tc < ntc;
    const uint32_t off = (uint32_t)((pp * ntc + cbase) * 8) * TB + lane_part;
    buf_load_words<NW>(crs, ok ? off : BUF_OFF, slot);
    if constexpr (CODE == NUQ) {
      const int64_t gr = grow_l + (int64_t)pp * 128;
      const int g = ((cbase + tc) * 16) / group;
      slot[NW] = buf_load_u16(grs, ok ? (uint32_t)((gr * gstride + g) * 2) : BUF_OFF);
      slot[NW + 1] = buf_load_u16(grs, ok ? (uint32_t)(((gr + 1) * gstride + g) * 2) : BUF_OFF);
    }
    if (++ps == S) {
      ps = 0;
      ++pk;
      pp += dp;
      pr += dr;
      if (pp >= npanels) { pp -= npanels; ++pr; }
    }
  };
  uint32_t ring[PF][CW];
#pragma unroll
  for (int j = 0; j < PF; ++j) load_step(ring[j]);
  __builtin_amdgcn_sched_barrier(0);   // all requests out before any wait

  // ---- 1. the lookup table ---------------------------------------------------
  auto build_table = [&]() {
    if constexpr (CODE == HYB) {
      // every thread writes its 16-byte runs of consecutive copies
      // (conflict-free writes) from the LUT words it loaded at the start;
      // entries 2^Q and up are the sign-flipped ones
      uint4* tab4 = reinterpret_cast<uint4*>(lds) + tid;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (k < K8) {                              // workgroup-uniform
          const uint32_t v = lw[k] ^ ((((step * k) >> Q) & 1) ? 0x80008000u : 0u);
          tab4[MMA_THREADS * k] = make_uint4(v, v, v, v);
        }
      }
    } else {
      constexpr int C = MmaTable<CODE>::COPIES;
      uint32_t* tab = smem;
      if constexpr (CODE == HYB1) fill_signed_table<C, 0x8000u>(tab, lut, Q, tid, MMA_THREADS);
      if constexpr (CODE == LUT) fill_plain_table<1>(tab, lut, 1 << 15, tid, MMA_THREADS);
      if constexpr (CODE == VQ) fill_plain_table<C>(tab, lut, 1 << KV, tid, MMA_THREADS);
      if constexpr (CODE == NUQ) fill_plain_table<1>(tab, lut, 1 << KV, tid, MMA_THREADS);
    }
  };

  // ---- 2. x' = RHT_in(x) of the row or of the range, fp16 in LDS -----------
  // Chunks of 8 consecutive values: the butterfly stages inside a chunk in
  // registers, the rest in padded LDS in passes of 3 index bits (512 groups of
  // 8 values on a 4096-value row: every thread busy).
  _Float16* xs = reinterpret_cast<_Float16*>(lds + xs_off_);
  auto x_transform = [&](float* scr) {
    const int hb_in = 31 - __builtin_clz((unsigned)Bi);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = tid + MMA_THREADS * j;          // local chunk
      const int gc = (xbase >> 3) + c;
      if (c < (NL >> 3) && gc < nch8) {
        const uint32_t r[4] = {xv[j].x, xv[j].y, xv[j].z, xv[j].w};
        const uint32_t sg = sw[j] >> ((8 * gc) & 31);
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float f = h2f((uint16_t)(r[e >> 1] >> (16 * (e & 1))));
          v[e] = ((sg >> e) & 1u) ? -f : f;
        }
#pragma unroll
        for (int h = 1; h < 8; h <<= 1) {
          if (h < Bi) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              if (!(e & h)) {
                const float x0 = v[e], x1 = v[e + h];
                v[e] = x0 + x1;
                v[e + h] = x0 - x1;
              }
            }
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) scr[pad_index(8 * c + e)] = v[e];
      }
    }
    __syncthreads();
    if (hb_in > 3) fwht_bits<3>(scr, NL, 3, hb_in, tid, MMA_THREADS);   // ends with a barrier
    const float rs = 1.0f / sqrtf((float)Bi);
    // x' is zero past n, to the end of the last range
    const int npad8 = (xmode == 0 ? nr * KR : KR) >> 3;
    const int nval8 = (n - xbase < NL ? n - xbase : NL) >> 3;
    for (int c = tid; c < npad8; c += MMA_THREADS) {
      uint32_t p[4] = {0u, 0u, 0u, 0u};
      if (c < nval8) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          p[e] = f2h_bits(scr[pad_index(8 * c + 2 * e)] * rs) |
                 ((uint32_t)f2h_bits(scr[pad_index(8 * c + 2 * e + 1)] * rs) << 16);
      }
      *reinterpret_cast<uint4*>(xs + 8 * c) = make_uint4(p[0], p[1], p[2], p[3]);
    }
  };

  // NL = 1024, 2048 or 4096 values (the whole row of such a layer, or such
  // a range): threads t < NL / 8 hold chunks of 8, index 8 t + e.  Index
  // bits 0-2 are in registers, bits 3-8 are lane bits 0-5 (butterflies
  // between lanes: DPP quad permutes for lanes ^1 and ^2, ds_swizzle for ^4,
  // ^8, ^16, ds_bpermute for ^32), then one exchange through LDS gives thread
  // a < 512 the indices a + 512 k, k < NL / 512, whose bits 9 and up are
  // again in registers; the results go to x' as fp16.  Two barriers instead
  // of five.
  auto x_transform_fast = [&](float* scr) {
    const int hb_in = 31 - __builtin_clz((unsigned)Bi);
    const int c = tid;                             // local chunk (threads < NL / 8)
    const int gc = (xbase >> 3) + c;
    const int KK = NL >> 9;                        // values per thread after the exchange
    float v[8];
    if (c < (NL >> 3)) {                           // whole waves
      const bool ok = gc < nch8;
      const uint32_t r[4] = {xv[0].x, xv[0].y, xv[0].z, xv[0].w};
      const uint32_t sg = sw[0] >> ((8 * gc) & 31);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float f = ok ? h2f((uint16_t)(r[e >> 1] >> (16 * (e & 1)))) : 0.f;
        v[e] = ((sg >> e) & 1u) ? -f : f;
      }
#pragma unroll
      for (int h = 1; h < 8; h <<= 1) {
        if (h < Bi) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            if (!(e & h)) {
              const float x0 = v[e], x1 = v[e + h];
              v[e] = x0 + x1;
              v[e + h] = x0 - x1;
            }
          }
        }
      }
      // bits 3-8 between lanes: the lower lane keeps the sum, the upper
      // one the difference
      auto stage = [&](int hbit, auto&& partner) {
        if (hb_in > hbit) {                        // workgroup-uniform
          const float sgn = (lane >> (hbit - 3)) & 1 ? -1.f : 1.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = __builtin_fmaf(v[e], sgn, partner(v[e]));
        }
      };
      stage(3, [](float x) { return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true)); });
      stage(4, [](float x) { return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, true)); });
      stage(5, [](float x) { return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x1F | (4 << 10))); });
      stage(6, [](float x) { return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x1F | (8 << 10))); });
      stage(7, [](float x) { return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x1F | (16 << 10))); });
      stage(8, [](float x) { return __shfl_xor(x, 32, 64); });
#pragma unroll
      for (int e = 0; e < 8; ++e) scr[pad_index(8 * c + e)] = v[e];
    }
    __syncthreads();
    if (c < 512) {
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = k < KK ? scr[pad_index(c + 512 * k)] : 0.f;
#pragma unroll
      for (int h = 1; h < 8; h <<= 1) {
        if ((h << 9) < Bi && h < KK) {
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            if (!(k & h)) {
              const float x0 = v[k], x1 = v[k + h];
              v[k] = x0 + x1;
              v[k + h] = x0 - x1;
            }
          }
        }
      }
      const float rs = 1.0f / sqrtf((float)Bi);
      const int nval = n - xbase < NL ? n - xbase : NL;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int i = c + 512 * k;
        if (k < KK) xs[i] = i < nval ? (_Float16)(v[k] * rs) : (_Float16)0.f;
      }
    }
    // x' is zero past the NL values, to the end of the last range
    const int npad8 = (xmode == 0 ? nr * KR : KR) >> 3;
    for (int c8 = (NL >> 3) + tid; c8 < npad8; c8 += MMA_THREADS)
      *reinterpret_cast<uint4*>(xs + 8 * c8) = make_uint4(0u, 0u, 0u, 0u);
  };

  // Where LDS allows, the transform has a scratch area of its own and the
  // table is built first, while x is still on its way; otherwise the
  // transform borrows the table's area and the table follows it.
  if (scr_off_ && (NL == 1024 || NL == 2048 || NL == 4096)) {   // workgroup-uniform
    build_table();
    x_transform_fast(reinterpret_cast<float*>(lds + scr_off_));
  } else if (scr_off_) {
    build_table();
    x_transform(reinterpret_cast<float*>(lds + scr_off_));
  } else {
    x_transform(reinterpret_cast<float*>(lds));
    __syncthreads();                      // the scratch is read; the table overwrites it
    build_table();
  }
  __syncthreads();

  // ---- 3. the units ----------------------------------------------------------
  const int cshift = cshift_;
  // HYB: the lane's copy, the stride factor and the index mask (both halves)
  const uint32_t hlb = 4u * (uint32_t)(lane & (copies_ - 1));
  const uint32_t hmul = 1u << (cshift - qshift);
  const uint32_t hmask = (0xFFFFu & ~((1u << qshift) - 1u)) * 0x10001u;
  const uint32_t* tabc = smem + (lane & (MmaTable<CODE>::COPIES - 1));          // other codes
  const auto zrs = make_rsrc(zl, (uint32_t)(nr * sstride * 4));
  const int hbits = Bo >= 128 ? 7 : 31 - __builtin_clz((unsigned)Bo);
  float4v acc[2] = {float4v{0.f, 0.f, 0.f, 0.f}, float4v{0.f, 0.f, 0.f, 0.f}};
  half8v b0 = {}, b1 = {};   // the B operands (x'), set in lanes 0, 16, 32, 48 each step
  // the current step: unit ck (panel cp, range cr), step cs in it
  int ck = 0, cs = 0, cp = cp0, cr = cr0;

  auto compute = [&](const uint32_t* wc) {
    uint32_t w[NW + 1];
#pragma unroll
    for (int i = 0; i < NW; ++i) w[i] = wc[i];
    lane_words_ready<CODE, KV>(w, lane);
    uint32_t out[16];
    if constexpr (CODE == HYB) {
      hyb_pairs_strided<KV>(w, hlb, hmul, hmask, out);
    } else if constexpr (CODE == MAD1) {
      mad1_pairs_centred<KV>(w, out);
    } else {
      float gs[2] = {0.f, 0.f};
      if constexpr (CODE == NUQ) {
        gs[0] = h2f((uint16_t)wc[NW]);
        gs[1] = h2f((uint16_t)wc[NW + 1]);
      }
      lane_decode_exact<CODE, KV, MmaTable<CODE>::COPIES>(w, tabc, qshift, gs, out);
    }
    const int col = cr * KR + ks * Kw + 64 * cs;   // first input column of the step
    if (col + 64 > n) {                              // wave-uniform: a ragged step
      const bool live = col + 16 * tc < n;
#pragma unroll
      for (int i = 0; i < 16; ++i) out[i] = live ? out[i] : 0u;
    }
    // only column 0 of the products is used: only lanes 0, 16, 32, 48 (the
    // B operand's column 0) read x' -- a sixteenth of the LDS return traffic;
    // the other lanes keep zeros
    if ((lane & 15) == 0) {
      const _Float16* xb = xs + (col - xbase) + 16 * (lane >> 4);
      b0 = *reinterpret_cast<const half8v*>(xb);
      b1 = *reinterpret_cast<const half8v*>(xb + 8);
    }
#pragma unroll
    for (int ra = 0; ra < 2; ++ra) {
      const half8v a0 = __builtin_bit_cast(half8v, make_uint4(out[8 * ra], out[8 * ra + 1], out[8 * ra + 2], out[8 * ra + 3]));
      const half8v a1 =
          __builtin_bit_cast(half8v, make_uint4(out[8 * ra + 4], out[8 * ra + 5], out[8 * ra + 6], out[8 * ra + 7]));
      acc[ra] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, b0, acc[ra], 0, 0, 0);
      acc[ra] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, b1, acc[ra], 0, 0, 0);
    }
  };

  // The end of a unit: lanes 0, 16, 32, 48 hold column 0 of the products,
  // D[i][0] for i = 4 (lane / 16) + e, MFMA row i being row
  // 16 (i / 8) + 2 (i % 8) + ra of the wave's 32.  Wave 0 then adds the
  // four quarters of the panel (quarter order), applies the in-panel
  // Hadamard stages (row bit 0 in registers, bits 1-6 between lanes: DPP
  // quad permutes, ds_swizzle, one ds_bpermute; the upper lane of a pair
  // keeps the difference, fma(v, -1, o) = o - v exactly) and stores the
  // panel; the other waves go on to their next unit.
  auto unit_end = [&]() {
    float* red = reinterpret_cast<float*>(lds + red_off_) + (ck & 1) * 512;
    if ((lane & 15) == 0) {
#pragma unroll
      for (int ra = 0; ra < 2; ++ra)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * (lane >> 4) + e;
          red[ks * 128 + 32 * rg + 16 * (i >> 3) + 2 * (i & 7) + ra] = acc[ra][e];
        }
    }
    acc[0] = float4v{0.f, 0.f, 0.f, 0.f};
    acc[1] = float4v{0.f, 0.f, 0.f, 0.f};
    __syncthreads();
    if (wave == 0) {
      float v0 = 0.f, v1 = 0.f;
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        const float2 p = *reinterpret_cast<const float2*>(red + k4 * 128 + 2 * lane);
        v0 += p.x;
        v1 += p.y;
      }
      if (hbits > 0) {
        const float s = v0 + v1;
        v1 = v0 - v1;
        v0 = s;
      }
      // row bit b (b >= 1) is lane bit b - 1
      auto stage = [&](int b, auto&& partner) {
        if (hbits > b) {                          // workgroup-uniform
          const float sg = (lane >> (b - 1)) & 1 ? -1.f : 1.f;
          v0 = __builtin_fmaf(v0, sg, partner(v0));
          v1 = __builtin_fmaf(v1, sg, partner(v1));
        }
      };
      stage(1, [](float x) { return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true)); });
      stage(2, [](float x) { return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, true)); });
      stage(3, [](float x) { return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x1F | (4 << 10))); });
      stage(4, [](float x) { return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x1F | (8 << 10))); });
      stage(5, [](float x) { return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x1F | (16 << 10))); });
      stage(6, [](float x) { return __shfl_xor(x, 32, 64); });
      const uint32_t off = (uint32_t)(((int64_t)cr * sstride + row0 + (int64_t)cp * 128 + 2 * lane) * 4);
      __builtin_amdgcn_raw_buffer_store_b64(
          __builtin_bit_cast(__attribute__((ext_vector_type(2))) uint32_t,
                             make_uint2(__builtin_bit_cast(uint32_t, v0), __builtin_bit_cast(uint32_t, v1))),
          zrs, off, 0, 0);
    }
    ++ck;
    cs = 0;
    cp += dp;
    cr += dr;
    if (cp >= npanels) { cp -= npanels; ++cr; }
  };

  // PF divides S, so a unit ends only after the last step of a group of PF.
  // A slot is refilled (with the step PF ahead, switched off past the end)
  // right after its step has read it, into the same registers: refilling
  // first would give the new words other registers and make the compiler
  // rotate the ring at the loop's back edge, after waiting for every load.
  for (int j0 = 0; j0 < T; j0 += PF) {
#pragma unroll
    for (int jj = 0; jj < PF; ++jj) {
      compute(ring[jj]);
      load_step(ring[jj]);
      ++cs;
    }
    if (cs == S) unit_end();
  }
}

template <int CODE, int KV, int PF>
__global__ __launch_bounds__(MMA_THREADS, 1) void gemv_mma_kernel(QDEC_BOUNDS_PARAMS, int xs_off_, int red_off_,
                                                                 int scr_off_, int cshift_, int copies_, MmaArgs a) {
  (void)nl_;
  gemv_mma_body<CODE, KV, PF, false>(QDEC_LAYER_OF((int)blockIdx.x), nullptr, nullptr, nullptr, 0, 0, 0, 0, 0,
                                     xs_off_, red_off_, scr_off_, cshift_, copies_, a);
}

// One layer whose x' is the whole row: the first loads' pointers and sizes
// lead the arguments (13 preloaded SGPRs with the LDS carve-up).
template <int CODE, int KV, int PF>
__global__ __launch_bounds__(MMA_THREADS, 1) void gemv_mma1_kernel(const uint32_t* lut_, const uint16_t* x_,
                                                                  const uint32_t* sgin_, int n_, int Q_, int xs_off_,
                                                                  int red_off_, int scr_off_, int cshift_,
                                                                  int copies_, MmaArgs a) {
  gemv_mma_body<CODE, KV, PF, true>(0, lut_, x_, sgin_, n_, Q_, 0, 0, n_, xs_off_, red_off_, scr_off_, cshift_,
                                    copies_, a);
}

// One layer with one K range per workgroup (x' of the range only): the
// table, x and the input signs, then n with Q, the LDS carve-up (offsets in
// 16-byte units) with the table shift and the copies, and the ranges (x'
// mode, count, KR / 512), packed in four words (10 preloaded SGPRs).
template <int CODE, int KV, int PF>
__global__ __launch_bounds__(MMA_THREADS, 1) void gemv_mma1r_kernel(const uint32_t* lut_, const uint16_t* x_,
                                                                   const uint32_t* sgin_, uint32_t nq_,
                                                                   uint32_t off0_, uint32_t off1_, uint32_t rk_,
                                                                   MmaArgs a) {
  const int n = (int)(nq_ & 0xFFFFFFu), nr = (int)((rk_ >> 1) & 0x7FFFu), KR = (int)(rk_ >> 16) << 9;
  const int xb = ((int)blockIdx.x % nr) * KR;   // one layer: range blockIdx mod nr
  gemv_mma_body<CODE, KV, PF, true>(0, lut_, x_, sgin_, n, (int)(nq_ >> 24), 1, xb, KR,
                                    (int)((off0_ & 0xFFFFu) << 4), (int)((off0_ >> 16) << 4),
                                    (int)((off1_ & 0xFFFFu) << 4), (int)((off1_ >> 16) & 0xFFu), (int)(off1_ >> 24),
                                    a);
}

// Two layers with one x (the same n and Q), both x' the whole row: both
// tables, both sign vectors, x, the second layer's first workgroup and, in
// three packed words, n and Q, the LDS carve-up (offsets in 16-byte units),
// the table shift and the copies lead the arguments (14 preloaded SGPRs).
template <int CODE, int KV, int PF>
__global__ __launch_bounds__(MMA_THREADS, 1) void gemv_mma2_kernel(const uint32_t* lut0_, const uint32_t* lut1_,
                                                                  const uint32_t* sg0_, const uint32_t* sg1_,
                                                                  const uint16_t* x_, int w1_, uint32_t nq_,
                                                                  uint32_t off0_, uint32_t off1_, MmaArgs a) {
  const int li = (int)blockIdx.x >= w1_ ? 1 : 0;
  gemv_mma_body<CODE, KV, PF, true>(li, li ? lut1_ : lut0_, x_, li ? sg1_ : sg0_, (int)(nq_ & 0xFFFFFFu),
                                    (int)(nq_ >> 24), 0, 0, (int)(nq_ & 0xFFFFFFu), (int)((off0_ & 0xFFFFu) << 4),
                                    (int)((off0_ >> 16) << 4),
                                    (int)((off1_ & 0xFFFFu) << 4), (int)((off1_ >> 16) & 0xFFu), (int)(off1_ >> 24),
                                    a);
}

// Three layers with one x (q, k, v: the same n and Q), x' the whole row:
// layer 0's table and sign vector, x, the byte offsets of layers 1 and 2's
// tables and sign vectors from layer 0's, both layer boundaries (16 bits
// each) and the three packed words of gemv_mma2_kernel (14 preloaded SGPRs).
template <int CODE, int KV, int PF>
__global__ __launch_bounds__(MMA_THREADS, 1) void gemv_mma3_kernel(const uint32_t* lut0_, const uint32_t* sg0_,
                                                                  const uint16_t* x_, int dl1_, int dl2_, int ds1_,
                                                                  int ds2_, uint32_t w12_, uint32_t nq_,
                                                                  uint32_t off0_, uint32_t off1_, MmaArgs a) {
  const int bid = (int)blockIdx.x;
  const int li = (int)(bid >= (int)(w12_ & 0xFFFFu)) + (int)(bid >= (int)(w12_ >> 16));
  const int64_t dl = li == 0 ? 0 : li == 1 ? dl1_ : dl2_;
  const int64_t ds = li == 0 ? 0 : li == 1 ? ds1_ : ds2_;
  const uint32_t* lut = reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(lut0_) + dl);
  const uint32_t* sg = sg0_ ? reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(sg0_) + ds) : nullptr;
  gemv_mma_body<CODE, KV, PF, true>(li, lut, x_, sg, (int)(nq_ & 0xFFFFFFu), (int)(nq_ >> 24), 0, 0,
                                    (int)(nq_ & 0xFFFFFFu), (int)((off0_ & 0xFFFFu) << 4), (int)((off0_ >> 16) << 4),
                                    (int)((off1_ & 0xFFFFu) << 4), (int)((off1_ >> 16) & 0xFFu), (int)(off1_ >> 24),
                                    a);
}

// PF = min(S, 8): the ring depth divides the steps of a unit (S is 2, 4 or a
// multiple of 8: KR is 512, 1024 or a multiple of 2048).
template <int CODE, int KV, int PF>
hipError_t launch_gemv_mma_p(const MmaArgs& a, unsigned grid, size_t lds, hipStream_t stream) {
  static LdsLimit have;
  const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&gemv_mma_kernel<CODE, KV, PF>), lds, &have);
  if (e != hipSuccess) return e;
  if constexpr (CODE == HYB) {
    if (a.nl == 1 && a.lay[0].xmode == 0) {
      static LdsLimit have1;
      const hipError_t e1 = ensure_dynamic_lds(reinterpret_cast<const void*>(&gemv_mma1_kernel<CODE, KV, PF>), lds,
                                               &have1);
      if (e1 != hipSuccess) return e1;
      const MmaLayer& l0 = a.lay[0];
      hipLaunchKernelGGL((gemv_mma1_kernel<CODE, KV, PF>), dim3(grid), dim3(MMA_THREADS), lds, stream, l0.L.lut, l0.x,
                         l0.L.sign_in, (int)l0.L.n, l0.L.Q, a.xs_off, a.red_off, a.scr_off, a.cshift, a.copies, a);
      return hipGetLastError();
    }
    const MmaLayer& l0 = a.lay[0];
    const MmaLayer& l1 = a.lay[1];
    const bool packs = ((a.xs_off | a.red_off | a.scr_off) & 15) == 0 && a.xs_off < (1 << 20) &&
                       a.red_off < (1 << 20) && a.scr_off < (1 << 20) && a.cshift < 256 && a.copies < 256 &&
                       l0.L.n < (1 << 24) && l0.L.Q < 256;
    const uint32_t nq = (uint32_t)l0.L.n | ((uint32_t)l0.L.Q << 24);
    const uint32_t off0 = ((uint32_t)a.xs_off >> 4) | (((uint32_t)a.red_off >> 4) << 16);
    const uint32_t off1 = ((uint32_t)a.scr_off >> 4) | ((uint32_t)a.cshift << 16) | ((uint32_t)a.copies << 24);
    if (a.nl == 1 && packs && l0.xmode == 1 && l0.nr >= 1 && l0.nr < (1 << 15) && l0.KR % 512 == 0 &&
        (l0.KR >> 9) < (1 << 16)) {
      static LdsLimit have1r;
      const hipError_t e1 = ensure_dynamic_lds(reinterpret_cast<const void*>(&gemv_mma1r_kernel<CODE, KV, PF>), lds,
                                               &have1r);
      if (e1 != hipSuccess) return e1;
      const uint32_t rk = 1u | ((uint32_t)l0.nr << 1) | ((uint32_t)(l0.KR >> 9) << 16);
      hipLaunchKernelGGL((gemv_mma1r_kernel<CODE, KV, PF>), dim3(grid), dim3(MMA_THREADS), lds, stream, l0.L.lut,
                         l0.x, l0.L.sign_in, nq, off0, off1, rk, a);
      return hipGetLastError();
    }
    if (a.nl == 3 && packs) {
      const MmaLayer& l2 = a.lay[2];
      auto delta = [](const void* p, const void* q, int64_t* d) {
        *d = (int64_t)((intptr_t)p - (intptr_t)q);
        return *d >= INT32_MIN && *d <= INT32_MAX;
      };
      int64_t dl1, dl2, ds1 = 0, ds2 = 0;
      const bool signs = l0.L.sign_in && l1.L.sign_in && l2.L.sign_in;
      const bool nosigns = !l0.L.sign_in && !l1.L.sign_in && !l2.L.sign_in;
      if (l0.xmode == 0 && l1.xmode == 0 && l2.xmode == 0 && l0.x == l1.x && l0.x == l2.x &&
          l0.L.n == l1.L.n && l0.L.n == l2.L.n && l0.L.Q == l1.L.Q && l0.L.Q == l2.L.Q && l1.wg0 < (1 << 16) &&
          l2.wg0 < (1 << 16) && (signs || nosigns) && delta(l1.L.lut, l0.L.lut, &dl1) &&
          delta(l2.L.lut, l0.L.lut, &dl2) &&
          (nosigns || (delta(l1.L.sign_in, l0.L.sign_in, &ds1) && delta(l2.L.sign_in, l0.L.sign_in, &ds2)))) {
        static LdsLimit have3;
        const hipError_t e3 = ensure_dynamic_lds(reinterpret_cast<const void*>(&gemv_mma3_kernel<CODE, KV, PF>), lds,
                                                 &have3);
        if (e3 != hipSuccess) return e3;
        const uint32_t w12 = (uint32_t)l1.wg0 | ((uint32_t)l2.wg0 << 16);
        hipLaunchKernelGGL((gemv_mma3_kernel<CODE, KV, PF>), dim3(grid), dim3(MMA_THREADS), lds, stream, l0.L.lut,
                           l0.L.sign_in, l0.x, (int)dl1, (int)dl2, (int)ds1, (int)ds2, w12, nq, off0, off1, a);
        return hipGetLastError();
      }
    }
    if (a.nl == 2 && packs && l0.xmode == 0 && l1.xmode == 0 && l0.x == l1.x && l0.L.n == l1.L.n &&
        l0.L.Q == l1.L.Q) {
      static LdsLimit have2;
      const hipError_t e2 = ensure_dynamic_lds(reinterpret_cast<const void*>(&gemv_mma2_kernel<CODE, KV, PF>), lds,
                                               &have2);
      if (e2 != hipSuccess) return e2;
      hipLaunchKernelGGL((gemv_mma2_kernel<CODE, KV, PF>), dim3(grid), dim3(MMA_THREADS), lds, stream, l0.L.lut,
                         l1.L.lut, l0.L.sign_in, l1.L.sign_in, l0.x, l1.wg0, nq, off0, off1, a);
      return hipGetLastError();
    }
  }
  LayerBounds b;
  b.w[0] = a.nl;
  for (int i = 1; i < GEMV_GROUP_MAX; ++i) b.w[i] = i < a.nl ? a.lay[i].wg0 : INT_MAX;
  hipLaunchKernelGGL((gemv_mma_kernel<CODE, KV, PF>), dim3(grid), dim3(MMA_THREADS), lds, stream,
                     QDEC_BOUNDS_ARGS(b), a.xs_off, a.red_off, a.scr_off, a.cshift, a.copies, a);
  return hipGetLastError();
}

template <int CODE, int KV>
hipError_t launch_gemv_mma_k(const MmaArgs& a, hipStream_t stream) {
  unsigned grid = 0;
  int S = 1 << 30;
  for (int l = 0; l < a.nl; ++l) {
    if (a.lay[l].wg0 != (int)grid) return hipErrorInvalidValue;
    grid += (unsigned)a.lay[l].nwg;
    const int s = a.lay[l].KR >> 8;
    if (s < S) S = s;
  }
  if (grid == 0) return hipSuccess;
  const size_t lds = (size_t)a.lds_bytes;
  if (lds < (size_t)a.red_off + MMA_RED_BYTES || lds > (size_t)LDS_MAX_BYTES) return hipErrorInvalidValue;
  if (S == 2) return launch_gemv_mma_p<CODE, KV, 2>(a, grid, lds, stream);
  if (S == 4) return launch_gemv_mma_p<CODE, KV, 4>(a, grid, lds, stream);
  return launch_gemv_mma_p<CODE, KV, 8>(a, grid, lds, stream);
}

template <int CODE>
hipError_t launch_gemv_mma_code(const MmaArgs& a, int kv, hipStream_t stream) {
#define QDEC_MMA_KV(KV)                                                              \
  case KV:                                                                           \
    if constexpr (kv_built(CODE, KV)) return launch_gemv_mma_k<CODE, KV>(a, stream); \
    break;
  switch (kv) {
    QDEC_MMA_KV(2) QDEC_MMA_KV(3) QDEC_MMA_KV(4) QDEC_MMA_KV(5)
    QDEC_MMA_KV(6) QDEC_MMA_KV(7) QDEC_MMA_KV(8)
    default: break;
  }
#undef QDEC_MMA_KV
  return hipErrorInvalidValue;
}

}  // namespace qdec
