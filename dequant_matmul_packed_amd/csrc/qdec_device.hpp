// Device-side building blocks shared by the qdec kernels (gfx950, wave64).
//
// Packed format, lane layout and code rules are those of include/qdec.h:
// a 16x16 tile is a stream of 256/V steps of kV bits; 8 consecutive lanes
// handle one tile and lane q of the group decodes weights 32q .. 32q+31 (tile
// rows 2q and 2q+1), the steps whose windows start in stream bits
// [q*LB, (q+1)*LB), LB = (32/V)*kV.  The state of a step is an L-bit window
// that may run past the lane's own bits into the next lane's first word (the
// last lane wraps to the first: the tail-biting stream), which a cross-lane
// permute supplies ("QTIP: Quantization with Trellises and Incoherence
// Processing", "Figure 2 (Q4)": the bitshift trellis decodes any step from
// its own window, so all lanes decode in parallel).  Every kernel takes kV,
// the bits per trellis step, as its width parameter: k = kV/V bits per
// weight, 2.5 at V = 2 and kV = 5 (the fractional widths of the "Q-Palette"
// summary).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qdec {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

// Code kinds of the kernels: the public codes, with HYB split by V (HYB is
// V = 2, HYB1 is V = 1, an internal number) and LUT the pure lookup.
enum { HYB = 1, MAD1 = 2, INST3 = 3, NUQ = 4, VQ = 5, LUT = 6, HYB1 = 7 };

__host__ __device__ constexpr int code_V(int code) { return (code == HYB || code == VQ) ? 2 : 1; }
// State bits: kV for the scalar and vector quantizers (L = kV: plain
// indices), 16 for the trellis codes.
__host__ __device__ constexpr int code_L(int code, int kv) {
  return (code == NUQ || code == VQ) ? kv : 16;
}
// The (code, kV) pairs the kernels are built for: HYB at V = 2 takes kV 4 to
// 8 (2 to 4 bits per weight in half-bit steps), VQ 4, 6, 8 (k = 2, 3, 4),
// the V = 1 codes 2 to 4.
__host__ __device__ constexpr bool kv_built(int code, int kv) {
  return code == HYB ? (kv >= 4 && kv <= 8)
       : code == VQ ? (kv == 4 || kv == 6 || kv == 8)
       : (kv >= 2 && kv <= 4);
}

// Where a lane's bits sit for a code with KV bits per step: LANE_BITS =
// (32/V)*KV stream bits per lane (its 32 weights), loaded as NW words from
// word lane_word(q) of the tile; TILE_WORDS per tile.  When LANE_BITS is an
// odd multiple of 16 (V = 2 and odd KV), odd lanes start 16 bits into their
// first word (HALF).
template <int CODE, int KV>
struct LaneGeom {
  static constexpr int V = code_V(CODE);
  static constexpr int L = code_L(CODE, KV);
  static constexpr int LANE_BITS = (32 / V) * KV;
  static constexpr int NW = (LANE_BITS + 31) / 32;
  static constexpr int TILE_WORDS = LANE_BITS / 4;
  static constexpr bool HALF = (LANE_BITS % 32) != 0;
  static_assert(LANE_BITS % 16 == 0, "lane segments start on 16-bit boundaries");
  // every window of the lane (the last one starts at bit LANE_BITS - KV)
  // ends within its NW words plus one more
  static_assert(LANE_BITS - KV + L <= 32 * (NW + 1), "windows reach one word past the lane");
  // shifted odd lanes have no valid word past their own NW
  static_assert(!HALF || LANE_BITS - KV + L <= 32 * NW, "half-word lanes stay within NW words");
  __host__ __device__ static constexpr uint32_t lane_word(int q) { return (uint32_t)(q * LANE_BITS) >> 5; }
};

// Computed-code constants (this library's own; the pages give none).
constexpr uint32_t MAD1_A = 0x00EA4F79u, MAD1_C = 0xC2AA9973u;
constexpr uint32_t INST3_A = 0x00E77B2Bu, INST3_C = 0xEACB81D7u;
constexpr uint32_t INST3_MASK = 0x8FFF8FFFu, INST3_PATTERN = 0x30003000u;
// fp32(1/sqrt(21845)): unit variance for a centred sum of four uniform bytes.
constexpr uint32_t MAD1_NORM_BITS = 0x3BDDB446u;
// 1MAD in the matmul paths: the byte sum sigma is formed as the fp16 number
// 1024 + sigma (exponent 10 makes integers exact); the mean 1024 + 510 is
// removed once per chunk through the sum of the activations.
constexpr float MAD1_BIAS = 1534.0f;

__device__ __forceinline__ float mad1_norm() { return __builtin_bit_cast(float, MAD1_NORM_BITS); }

__device__ __forceinline__ uint16_t f2h_bits(float v) {
  return __builtin_bit_cast(uint16_t, (_Float16)v);
}
__device__ __forceinline__ float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
__device__ __forceinline__ half2v as_h2(uint32_t v) { return __builtin_bit_cast(half2v, v); }

// L-bit window starting at bit offset o of the lane's word array (MSB first).
// o and L are compile-time constants after unrolling, so this folds to one
// shift/mask or one funnel shift (v_alignbit_b32) plus a mask.
template <int L>
__device__ __forceinline__ uint32_t window_at(const uint32_t* w, int o) {
  const int i = o >> 5, r = o & 31;
  const uint32_t mask = (L == 32) ? 0xFFFFFFFFu : ((1u << L) - 1u);
  if (r + L <= 32) return (w[i] >> (32 - r - L)) & mask;
  return __builtin_amdgcn_alignbit(w[i], w[i + 1], 64 - r - L) & mask;
}

// The same window with the stream bits that precede it left above bit L
// (not masked off): for the HYB hash, whose 16 used bits depend only on the
// window's low 16 bits (see hyb_hash).
template <int L>
__device__ __forceinline__ uint32_t window_raw(const uint32_t* w, int o) {
  const int i = o >> 5, r = o & 31;
  if (r + L <= 32) return w[i] >> (32 - r - L);
  return __builtin_amdgcn_alignbit(w[i], w[i + 1], 64 - r - L);
}

// ---------------------------------------------------------------------------
// Raw buffer loads.  A buffer resource covers `bytes` bytes from a
// wave-uniform base; a load whose byte offset lies at or beyond that size
// returns zero and touches no memory.  Every load can therefore be issued
// unconditionally and switched off through its offset: no branch around it,
// so the compiler keeps exact counts of the loads in flight and waits only
// for the one it needs (a load inside a branch ends in a wait for all of
// them at the join).
constexpr uint32_t BUF_OFF = 0x80000000u;   // an offset beyond every resource here
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
template <int K>
__device__ __forceinline__ void buf_load_words(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t* w) {
  if constexpr (K == 1) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  } else if constexpr (K == 2) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    w[0] = v[0]; w[1] = v[1];
  } else if constexpr (K == 3) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, 0);
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2];
  } else if constexpr (K == 4) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
  } else {
#pragma unroll
    for (int i = 0; i < K; ++i) w[i] = __builtin_amdgcn_raw_buffer_load_b32(r, off + 4 * i, 0, 0);
  }
}
__device__ __forceinline__ uint4 buf_load_u4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint32_t buf_load_u32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load_u16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

// First word of the next lane of the same 8-lane tile group (lane 7 wraps to
// lane 0: the tail-biting stream).
__device__ __forceinline__ uint32_t next_lane_word(uint32_t v, int lane) {
  const int src = (lane & ~7) | ((lane + 1) & 7);
  return (uint32_t)__builtin_amdgcn_ds_bpermute(src << 2, (int)v);
}

// Completes a lane's word array w[0..NW] for window extraction: w[NW] is the
// next lane's first word, and with HALF the odd lanes, whose words were
// loaded from 16 bits before their segment, shift them into place (the next
// lane is even there, so its first word starts exactly where the lane's
// segment ends).  Called by all lanes (the permute reads every lane).
template <int CODE, int KV>
__device__ __forceinline__ void lane_words_ready(uint32_t* w, int lane) {
  using G = LaneGeom<CODE, KV>;
  w[G::NW] = next_lane_word(w[0], lane);
  if constexpr (G::HALF) {
    const bool odd = lane & 1;
#pragma unroll
    for (int i = 0; i < G::NW; ++i) {
      const uint32_t sh = __builtin_amdgcn_alignbit(w[i], w[i + 1], 16);
      w[i] = odd ? sh : w[i];
    }
  }
}

// HYB hash: h = s*s + s (mod 2^16); the signed table index is h >> (15 - Q)
// (Q index bits plus the sign bit 15).
// Only bits below 16 of h are used, and they depend only on the low 16 bits
// of s, so the 24-bit multiply-add (full rate) is exact here whatever the
// bits of s above 16.  It is written as the instruction itself: from the
// plain expression the compiler forms a 64-bit multiply-add when it knows
// the high bits of s are zero, a slower instruction.
__device__ __forceinline__ uint32_t hyb_hash(uint32_t s) {
  uint32_t h;
  asm("v_mad_u32_u24 %0, %1, %1, %1" : "=v"(h) : "v"(s));
  return h;
}
__device__ __forceinline__ uint32_t hyb_signed_index(uint32_t s, int qshift) {
  return (hyb_hash(s) & 0xFFFFu) >> qshift;
}

// Two states 16 bits apart in the stream (steps t and t + 16/kV when kV
// divides 16) are the two halves of one 32-bit window: the high half is the
// state at the window's first bit, the low half the one 16 bits later.  The
// packed 16-bit multiply-add then hashes both at once, each half of its
// result being (s*s + s) mod 2^16 of its state, which is all the index uses.
__device__ __forceinline__ void hyb_index_pair(uint32_t win32, int qshift, uint32_t& idx_first,
                                               uint32_t& idx_second) {
  uint32_t h2;
  asm("v_pk_mad_u16 %0, %1, %1, %1" : "=v"(h2) : "v"(win32));
  idx_first = h2 >> (16 + qshift);
  idx_second = (h2 & 0xFFFFu) >> qshift;
}

// 1MAD: LCG output for a state.
__device__ __forceinline__ uint32_t mad1_lcg(uint32_t s) { return s * MAD1_A + MAD1_C; }
// 3INST: LCG, then force the high exponent bits of both halves.
// The pattern is held in a register so that the mask-and-insert is one
// v_and_or_b32 (an instruction here takes at most one literal constant).
__device__ __forceinline__ uint32_t inst3_bits(uint32_t s) {
  uint32_t pat = INST3_PATTERN;
  asm("" : "+v"(pat));
  return ((s * INST3_A + INST3_C) & INST3_MASK) | pat;
}

// Exact fp16 value of 1MAD: fp16(fp32((sigma - 510) * fp32(1/sqrt(21845)))).
__device__ __forceinline__ uint16_t mad1_value_bits(uint32_t s) {
#pragma clang fp contract(off)   // the fp32 product is rounded before the fp16 conversion
  const int sigma = (int)__builtin_amdgcn_sad_u8(mad1_lcg(s), 0u, 0u);
  return f2h_bits((float)(sigma - 510) * mad1_norm());
}
// Exact fp16 value of 3INST: the fp16 sum of the two halves (one rounding).
__device__ __forceinline__ uint16_t inst3_value_bits(uint32_t s) {
  const uint32_t u = inst3_bits(s);
  const _Float16 lo = __builtin_bit_cast(_Float16, (uint16_t)(u & 0xFFFFu));
  const _Float16 hi = __builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
  return __builtin_bit_cast(uint16_t, (_Float16)(lo + hi));
}

// ---------------------------------------------------------------------------
// LDS lookup tables.  HYB: the 2^Q-entry LUT expanded by the sign bit into
// 2^(Q+1) signed entries (the sign flips both halves), replicated COPIES
// times with entry e of copy c at word e*COPIES + c, so lanes that use
// different copies fall in different banks.  VQ: 2^(2k) pairs, replicated
// the same way.  NUQ: 2^k fp16 levels (one copy, broadcast reads).
// FLIP is the sign flip of an entry: both halves (V = 2) or the low one
// (V = 1, whose words carry one fp16 value in the low half).
template <int COPIES, uint32_t FLIP = 0x80008000u>
__device__ __forceinline__ void fill_signed_table(uint32_t* tab, const uint32_t* __restrict__ lut,
                                                  int Q, int tid, int nthreads) {
  const int E = 2 << Q;
  for (int e = tid; e < E; e += nthreads) {
    uint32_t v = lut[e & ((1 << Q) - 1)];
    if (e >> Q) v ^= FLIP;
#pragma unroll
    for (int c = 0; c < COPIES; ++c) tab[e * COPIES + c] = v;
  }
}

template <int COPIES>
__device__ __forceinline__ void fill_plain_table(uint32_t* tab, const uint32_t* __restrict__ lut,
                                                 int entries, int tid, int nthreads) {
  for (int e = tid; e < entries; e += nthreads) {
    const uint32_t v = lut[e];
#pragma unroll
    for (int c = 0; c < COPIES; ++c) tab[e * COPIES + c] = v;
  }
}

// ---------------------------------------------------------------------------
// Exact decode of a lane's 32 weights into 16 fp16 pairs:
// out[i] = (weight 32q + 2i, weight 32q + 2i + 1), i.e. tile row 2q + (i >> 3),
// columns 2(i & 7) and 2(i & 7) + 1.  w[0..NW] are the lane's words as
// lane_words_ready leaves them.  tabc points at this lane's copy of the table
// (HYB/VQ) or at the NUQ levels; gs[r] is the NUQ group scale of the lane's
// row 2q + r (unused otherwise).
// HYB at V = 2: the lane's 16 table pairs, out[t] for step t.  Where kV
// divides 16, steps t and t + 16/kV come from one window and one packed hash.
template <int KV, int COPIES>
__device__ __forceinline__ void hyb_lane_pairs(const uint32_t* w, const uint32_t* tabc, int qshift,
                                               uint32_t* out) {
  if constexpr (16 % KV == 0) {
    constexpr int D = 16 / KV;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      if ((t / D) & 1) continue;                       // the second of a pair
      uint32_t i0, i1;
      hyb_index_pair(window_raw<32>(w, t * KV), qshift, i0, i1);
      out[t] = tabc[i0 * COPIES];
      out[t + D] = tabc[i1 * COPIES];
    }
  } else {
#pragma unroll
    for (int t = 0; t < 16; ++t) out[t] = tabc[hyb_signed_index(window_raw<16>(w, t * KV), qshift) * COPIES];
  }
}

template <int CODE, int KV, int COPIES>
__device__ __forceinline__ void lane_decode_exact(const uint32_t* w, const uint32_t* tabc,
                                                  int qshift, const float* gs, uint32_t* out) {
  constexpr int V = code_V(CODE);
  constexpr int L = code_L(CODE, KV);
  if constexpr (CODE == HYB) {
    static_assert(V == 2 && L == 16, "HYB: two weights per step, 16-bit states");
    hyb_lane_pairs<KV, COPIES>(w, tabc, qshift, out);
  } else if constexpr (V == 2) {
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      out[t] = tabc[window_at<L>(w, t * KV) * COPIES];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      uint32_t v[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int t = 2 * i + h;
        const uint32_t s = window_at<L>(w, t * KV);
        if constexpr (CODE == MAD1) v[h] = mad1_value_bits(s);
        else if constexpr (CODE == INST3) v[h] = inst3_value_bits(s);
        else if constexpr (CODE == HYB1) v[h] = tabc[hyb_signed_index(s, qshift) * COPIES] & 0xFFFFu;
        else if constexpr (CODE == LUT) v[h] = reinterpret_cast<const uint16_t*>(tabc)[s];
        else {  // NUQ: fp16(level * group scale); the fp32 product is exact
          const uint16_t lvl = (uint16_t)tabc[s];
          v[h] = f2h_bits(h2f(lvl) * gs[i >> 3]);
        }
      }
      out[i] = v[0] | (v[1] << 16);
    }
  }
}

}  // namespace qdec

namespace qdec {

// ---------------------------------------------------------------------------
// Fast Walsh-Hadamard transform on an LDS float array, in place and
// unnormalised: every segment of S consecutive entries (S a power of two,
// `total` a multiple of S) is multiplied by the Sylvester-ordered H_S.  The
// radix-2 stages act on distinct index bits and commute, so they run in
// passes of up to 4 bits, 16 values per thread held in registers.  Entry i
// lives at word pad_index(i) = i + i/32: with one spare word per 32 the
// strided accesses of every pass fall in distinct banks.  All threads of
// the block must call these; they end with a barrier.
__device__ __forceinline__ int pad_index(int i) { return i + (i >> 5); }
__host__ __device__ constexpr int padded_words(int n) { return n + (n >> 5) + 1; }

template <int E>
__device__ __forceinline__ void fwht_pass(float* buf, int total, int b0, int tid, int nthreads) {
  constexpr int G = 1 << E;
  const int ngroups = total >> E;
  for (int g = tid; g < ngroups; g += nthreads) {
    const int lo = g & ((1 << b0) - 1);
    const int hi = g >> b0;
    const int base = (hi << (b0 + E)) | lo;
    float v[G];
#pragma unroll
    for (int i = 0; i < G; ++i) v[i] = buf[pad_index(base + (i << b0))];
#pragma unroll
    for (int h = 1; h < G; h <<= 1) {
#pragma unroll
      for (int i = 0; i < G; ++i) {
        if (!(i & h)) {
          const float a = v[i], b = v[i + h];
          v[i] = a + b;
          v[i + h] = a - b;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < G; ++i) buf[pad_index(base + (i << b0))] = v[i];
  }
}

// Stages on index bits [bit_lo, bit_hi) only; `total` a multiple of 2^bit_hi.
// Passes of up to R bits: R = 4 (16 values per thread) suits 256-thread
// blocks; 1024-thread blocks take R = 3, which keeps all their threads busy
// on a 4096-value transform (512 groups of 8 instead of 256 of 16).
template <int R = 4>
__device__ inline void fwht_bits(float* buf, int total, int bit_lo, int bit_hi, int tid, int nthreads) {
  for (int b0 = bit_lo; b0 < bit_hi; b0 += R) {
    const int e = (bit_hi - b0) < R ? (bit_hi - b0) : R;
    switch (e) {
      case 1: fwht_pass<1>(buf, total, b0, tid, nthreads); break;
      case 2: fwht_pass<2>(buf, total, b0, tid, nthreads); break;
      case 3: fwht_pass<3>(buf, total, b0, tid, nthreads); break;
      default: fwht_pass<R < 4 ? R : 4>(buf, total, b0, tid, nthreads); break;
    }
    __syncthreads();
  }
}

__device__ inline void fwht_segments(float* buf, int total, int S, int tid, int nthreads) {
  fwht_bits(buf, total, 0, 31 - __builtin_clz((unsigned)S), tid, nthreads);
}

// In-register FWHT of P values (P a power of two).
template <int P>
__device__ __forceinline__ void fwht_regs(float* v) {
#pragma unroll
  for (int h = 1; h < P; h <<= 1) {
#pragma unroll
    for (int i = 0; i < P; ++i) {
      if (!(i & h)) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
}

// Sign of entry j of a packed sign vector (bit set = -1); NULL = all +1.
__device__ __forceinline__ float sign_of(const uint32_t* __restrict__ s, int64_t j) {
  if (!s) return 1.0f;
  return ((s[j >> 5] >> (j & 31)) & 1u) ? -1.0f : 1.0f;
}

}  // namespace qdec
