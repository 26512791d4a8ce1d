/*
 * qdec CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct CPU implementation of the weight-only
 * quantized matmul y = W_hat x with incoherence processing, used to check the
 * HIP library.  Only the tests, the smoke check and the bench's CPU-baseline
 * leg may load it; the product path never calls it.  It shares no source with
 * the HIP library: it has its own descriptor, its own fp16 rounding, its own
 * bit reader and its own Hadamard (by definition, O(B^2)).
 *
 * Sources (web pages; sections named as they appear there):
 *  - "QTIP: Quantization with Trellises and Incoherence Processing"
 *    (OpenReview discussion):
 *      "Figure 2 (Q4)"  -- the bitshift trellis: a state is its predecessor
 *        shifted by kV bits with kV fresh bits at the low end (the two share
 *        L-kV bits), so only kV new bits are stored
 *        per step; the worked example 0010110 -> 00,01,10,01,11,10.
 *      "Ablations and fast inference (W1 and W2)" -- L = kV makes the trellis
 *        plain k-bit V-dim VQ; the bitshift trellis needs no stored graph and
 *        decodes in parallel.
 *      untitled ALU-op comment at the top of the discussion, "HYB Uniqueness
 *        (Q2)", "Bit Accounting (Q2)" -- HYB: Q=9, V=2, a 512 x 32-bit LUT of
 *        fp16 pairs expanded by a sign to 1024 entries; RHT sign vectors of
 *        n+m bits.
 *      computed-codes reply and "LCG citation (O2)" -- 1MAD/3INST: a
 *        deterministic, fixed-instruction-count map from the L-bit state to
 *        a pseudo-Gaussian value, built on an LCG.
 *      "Incoherence Processing (W2)" -- the random Hadamard transform (RHT)
 *        on both sides, invertible up to rounding.
 *      "Other hardware (e.g. ARM) (W3)" -- HYB with a one-dimensional
 *        codebook (Q = 6, V = 1).
 *      "Ablations and fast inference (W1 and W2)", Table A -- the pure-lookup
 *        codebook of 2^L values (L = 16, V = 1: 16 * 2^L bits).
 *  - "Q-Palette" blog summary -- fractional bit widths (2.5 bits and the
 *    like) and half-TCQ, two trellis bit widths in one layer (2.5 and 3 bits
 *    giving 2.75).  Here a trellis step may take any whole number kV of bits,
 *    so V = 2 gives k = kV/2 (2.5 bits at kV = 5), and the rows of a layer
 *    may be cut at a panel boundary into two parts of different kV.
 *  - "Q-Palette" blog summary -- non-uniform scalar (NUQ) and vector (VQ)
 *    quantizers alongside TCQ.
 *  - QuIP# (arXiv 2402.04396) abstract and Fig. 2 -- RHT incoherence
 *    processing.
 *
 * Readings where the pages are silent (each is also a format rule the HIP
 * library implements independently):
 *  - tail-biting per 256-weight tile: the state window wraps around the end of
 *    the tile's (256/V)*kV-bit stream, so storage is exactly kV/V bits per
 *    weight;
 *  - half-TCQ: rows [0, m_a) at kv, rows [m_a, m) at kv_b, m_a a multiple of
 *    128; the tiles of the first part are stored first (panel layout over its
 *    own rows), then those of the second part;
 *  - stream bits are MSB-first in little-endian u32 words;
 *  - 16x16 tiles, weight j of a tile at (row j>>4, col j&15), step t covering
 *    weights tV..tV+V-1; tiles stored in panels of 8 tile-rows, column-major
 *    inside a panel;
 *  - HYB hash h = s*s+s mod 2^16, index = bits [15-Q, 15) of h, sign = bit 15
 *    of h flipping both halves of the LUT pair (V = 2) or the one value
 *    (V = 1: the fp16 value is the low half of the LUT word);
 *  - pure lookup: entry s of 2^L fp16 values packed two per LUT word (entry
 *    e in the low half of word e/2 when e is even, the high half when odd);
 *  - 1MAD / 3INST constants are this library's own (not on the pages);
 *  - Sylvester-ordered Hadamard, 1/sqrt(B) normalisation, signs before H on
 *    the input and after H on the output, sign bit set means -1;
 *  - the encoder (the step before the path) minimises the squared error of a
 *    tile over all tail-biting streams with the Viterbi algorithm on the
 *    bitshift trellis ("Figure 2 (Q4)": the trellis lives in the state
 *    numbering; "Why does TCQ work? (Q5)": TCQ searches a 2^(kV)-sized part
 *    of the 2^L-state space at every step).  The pages do not say how the
 *    wrap of a tail-biting stream is chosen; here a first pass over the
 *    sequence rotated by half its length picks the L-kV wrap bits (the top
 *    bits of the first state), and a second pass is the exact Viterbi
 *    given them.  Path costs are accumulated in fp32 in a fixed order (no
 *    fused multiply-add), ties going to the smaller index, so that a GPU
 *    encoder with the same arithmetic takes the same decisions.
 *
 * Floating point: fp64 throughout; conversion to fp16 by this file's own
 * round-to-nearest-even (orc_f16_from_double).  Build with -ffp-contract=off
 * and without fast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Code kinds (same numbering as the library's public header, restated).     */
enum { ORC_HYB = 1, ORC_1MAD = 2, ORC_3INST = 3, ORC_NUQ = 4, ORC_VQ = 5, ORC_LUT = 6 };

/* Constants of the computed codes.  The pages name the codes and say they are
 * built on an LCG with a fixed instruction count; the numbers are this
 * project's own, chosen so that over all 2^16 states the values are
 * near-Gaussian and neighbouring trellis states are uncorrelated. */
#define ORC_1MAD_A 0x00EA4F79u
#define ORC_1MAD_C 0xC2AA9973u
#define ORC_3INST_A 0x00E77B2Bu
#define ORC_3INST_C 0xEACB81D7u
#define ORC_3INST_MASK 0x8FFF8FFFu
#define ORC_3INST_PATTERN 0x30003000u

typedef struct {
  int32_t code, L, k, V, Q;
  int32_t kv;              /* bits per trellis step of rows [0, m_a); 0 = k*V */
  int32_t kv_b;            /* bits per step of rows [m_a, m); 0 = one part */
  int64_t m_a;             /* rows of the first part; 0 = all rows        */
  int64_t m, n;
  const uint32_t *codes;   /* packed tile streams                         */
  const uint32_t *lut;     /* HYB: 2^Q pairs; NUQ: 2^k levels; VQ: 2^(kV) */
  const uint16_t *gscale;  /* NUQ: fp16 [m][n/group], else NULL            */
  int32_t group;           /* NUQ group length along a row                */
  float scale;             /* per-layer scale                             */
  const uint32_t *sign_in; /* n bits, NULL = all +1                       */
  const uint32_t *sign_out;/* m bits, NULL = all +1                       */
  int32_t had_in, had_out; /* Hadamard block sizes                        */
} orc_layer;

/* ------------------------------------------------------------------------ */
/* fp16 <-> fp64, round to nearest, ties to even, subnormals kept.           */

double orc_f16_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int f = h & 1023;
  double v;
  if (e == 31)
    v = f ? NAN : INFINITY;
  else if (e == 0)
    v = ldexp((double)f, -24);
  else
    v = ldexp((double)(1024 + f), e - 25);
  return sign ? -v : v;
}

uint16_t orc_f16_from_double(double v) {
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (isnan(v)) return 0x7E00;
  if (isinf(a)) return sign | 0x7C00;
  if (a == 0.0) return sign;
  int e2;
  frexp(a, &e2);            /* a = mant * 2^e2, mant in [0.5, 1) */
  int e = e2 - 1;           /* a in [2^e, 2^(e+1))               */
  int q;                    /* exponent of the unit in the last place */
  if (e < -14) q = -24;     /* subnormal range: fixed quantum 2^-24 */
  else q = e - 10;
  double mq = ldexp(a, -q); /* exact: a scaled by a power of two  */
  double f = floor(mq);
  double frac = mq - f;     /* exact in fp64                       */
  if (frac > 0.5 || (frac == 0.5 && fmod(f, 2.0) == 1.0)) f += 1.0;
  /* f is the significand in units of 2^q */
  if (q == -24) {
    /* subnormal (or rounds up to the smallest normal, f == 1024) */
    return sign | (uint16_t)f;
  }
  if (f >= 2048.0) { f = 1024.0; e += 1; }
  if (e > 15) return sign | 0x7C00;
  return sign | (uint16_t)((e + 15) << 10) | (uint16_t)((int)f - 1024);
}

/* The same rounding over an array of fp32 values (each converts to fp64
   exactly), for exhaustive checks over whole binades. */
void orc_f16_from_float_array(const float* v, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f16_from_double((double)v[i]);
}

/* Round fp64 to fp32 (C's conversion rounds to nearest-even by default).   */
static double orc_round_f32(double v) { return (double)(float)v; }

/* ------------------------------------------------------------------------ */
/* Bit stream and trellis walk ("Figure 2 (Q4)").                            */

/* Stream bit p of a tile: word p>>5, MSB-first inside the word.            */
static int orc_bit(const uint32_t *words, int64_t p) {
  return (int)((words[p >> 5] >> (31 - (p & 31))) & 1u);
}

/* Bit-serial shift-register walk over an explicit bit array.
 * The first state is the first L bits; every later state shifts the register
 * left by kV and brings in the next kV bits.  With tailbiting, bit positions
 * wrap modulo nbits (the reading used for tiles); otherwise the stream must
 * hold L + (nsteps-1)*kV bits.  Returns 0 on success, -1 on a short stream. */
int orc_walk_bits(const uint8_t *bits, int64_t nbits, int L, int kV,
                  int64_t nsteps, int tailbiting, uint32_t *states) {
  if (L < 1 || L > 31 || kV < 1 || kV > L || nsteps < 0) return -1;
  if (!tailbiting && nsteps > 0 && L + (nsteps - 1) * kV > nbits) return -1;
  if (nbits <= 0 && nsteps > 0) return -1;
  uint32_t mask = (L == 32) ? 0xFFFFFFFFu : ((1u << L) - 1u);
  uint32_t r = 0;
  int64_t pos = 0;
  for (int i = 0; i < L; i++) {
    r = (r << 1) | (bits[pos % nbits] & 1u);
    pos++;
  }
  if (nsteps > 0) states[0] = r & mask;
  for (int64_t t = 1; t < nsteps; t++) {
    for (int i = 0; i < kV; i++) {
      r = ((r << 1) | (bits[pos % nbits] & 1u)) & mask;
      pos++;
    }
    states[t] = r;
  }
  return 0;
}

/* Random-access form of the same walk: state t is the L-bit window that
 * starts at stream bit t*kV (mod nbits), read MSB-first.                    */
uint32_t orc_window_state(const uint8_t *bits, int64_t nbits, int L, int kV,
                          int64_t t) {
  uint32_t r = 0;
  for (int i = 0; i < L; i++) r = (r << 1) | (bits[(t * kV + i) % nbits] & 1u);
  return r;
}

/* ------------------------------------------------------------------------ */
/* State -> value maps.                                                      */

/* HYB ("HYB Uniqueness (Q2)", "Bit Accounting (Q2)", ALU-op comment):
 * hash the state, take Q index bits into a 2^Q-entry LUT of fp16 pairs, and
 * let one more hash bit flip the sign of both halves.                       */
static void orc_value_hyb(uint32_t s, int Q, const uint32_t *lut,
                          uint16_t out[2]) {
  uint32_t h = (s * s + s) & 0xFFFFu;
  uint32_t idx = (h >> (15 - Q)) & ((1u << Q) - 1u);
  uint32_t neg = (h >> 15) & 1u;
  uint32_t e = lut[idx];
  uint16_t lo = (uint16_t)(e & 0xFFFFu), hi = (uint16_t)(e >> 16);
  if (neg) { lo ^= 0x8000; hi ^= 0x8000; }
  out[0] = lo;
  out[1] = hi;
}

/* HYB at V = 1: the same hash and index; the value is the fp16 in the low
 * half of the LUT word, its sign flipped by hash bit 15.                     */
static uint16_t orc_value_hyb1(uint32_t s, int Q, const uint32_t *lut) {
  uint32_t h = (s * s + s) & 0xFFFFu;
  uint32_t idx = (h >> (15 - Q)) & ((1u << Q) - 1u);
  uint16_t v = (uint16_t)(lut[idx] & 0xFFFFu);
  return ((h >> 15) & 1u) ? (uint16_t)(v ^ 0x8000u) : v;
}

/* Pure lookup: the state itself indexes 2^L fp16 values, two per word.      */
static uint16_t orc_value_lut(uint32_t s, const uint32_t *lut) {
  uint32_t w = lut[s >> 1];
  return (uint16_t)((s & 1u) ? (w >> 16) : (w & 0xFFFFu));
}

/* 1MAD: one LCG multiply-add on the state, then the sum of the four bytes of
 * the 32-bit result (a sum of four near-uniform bytes, mean 510, variance
 * 4*(256^2-1)/12 = 21845), centred and scaled to unit variance in fp32, then
 * rounded to fp16.                                                           */
static uint16_t orc_value_1mad(uint32_t s) {
  uint32_t u = ORC_1MAD_A * s + ORC_1MAD_C; /* mod 2^32 by unsigned wrap */
  int sigma = (int)(u & 255u) + (int)((u >> 8) & 255u) +
              (int)((u >> 16) & 255u) + (int)(u >> 24);
  double c32 = orc_round_f32(1.0 / sqrt(21845.0));
  double v32 = orc_round_f32((double)(sigma - 510) * c32);
  return orc_f16_from_double(v32);
}

/* 3INST: LCG, then a bit-field insert that forces the high exponent bits of
 * both fp16 halves (keeping sign, low exponent bits and mantissa from the
 * LCG), then the fp16 sum of the two halves.                                */
static uint16_t orc_value_3inst(uint32_t s) {
  uint32_t u = ORC_3INST_A * s + ORC_3INST_C;
  u = (u & ORC_3INST_MASK) | ORC_3INST_PATTERN;
  double lo = orc_f16_to_double((uint16_t)(u & 0xFFFFu));
  double hi = orc_f16_to_double((uint16_t)(u >> 16));
  return orc_f16_from_double(lo + hi); /* fp64 sum is exact here */
}

/* ------------------------------------------------------------------------ */
/* Layer geometry.                                                           */

static int orc_is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

static int orc_is_trellis(int code) {
  return code == ORC_HYB || code == ORC_1MAD || code == ORC_3INST || code == ORC_LUT;
}

/* Bits per trellis step of the first part, of the second part, and the rows
 * of the first part (a layer with one part: m_a = m, kv_b = kv).            */
static int orc_kv_a(const orc_layer *Lr) { return Lr->kv ? Lr->kv : Lr->k * Lr->V; }
static int orc_kv_b(const orc_layer *Lr) { return Lr->m_a ? Lr->kv_b : orc_kv_a(Lr); }
static int64_t orc_m_a(const orc_layer *Lr) { return Lr->m_a ? Lr->m_a : Lr->m; }

int orc_validate(const orc_layer *Lr) {
  if (!Lr || !Lr->codes) return -1;
  if (Lr->m <= 0 || Lr->n <= 0 || Lr->m % 128 || Lr->n % 16) return -1;
  if (Lr->kv == 0) {
    if (Lr->k < 1 || Lr->k > 8) return -1;
  } else if (Lr->k != 0 || !orc_is_trellis(Lr->code)) {
    return -1;
  }
  if (Lr->m_a) {
    if (!orc_is_trellis(Lr->code) || Lr->m_a < 0 || Lr->m_a >= Lr->m || Lr->m_a % 128 ||
        Lr->kv_b < 1)
      return -1;
  } else if (Lr->kv_b) {
    return -1;
  }
  switch (Lr->code) {
  case ORC_HYB:
    if ((Lr->V != 1 && Lr->V != 2) || Lr->L != 16 || Lr->Q < 1 || Lr->Q > 15 ||
        !Lr->lut)
      return -1;
    break;
  case ORC_LUT:
    if (Lr->V != 1 || Lr->L != 16 || !Lr->lut) return -1;
    break;
  case ORC_1MAD:
  case ORC_3INST:
    if (Lr->V != 1 || Lr->L != 16) return -1;
    break;
  case ORC_NUQ:
    if (Lr->V != 1 || Lr->L != Lr->k || !Lr->lut || !Lr->gscale) return -1;
    if (Lr->group < 16 || Lr->group % 16 || Lr->n % Lr->group) return -1;
    break;
  case ORC_VQ:
    if (Lr->V != 2 || Lr->L != Lr->k * 2 || !Lr->lut) return -1;
    break;
  default:
    return -1;
  }
  if (orc_kv_a(Lr) < 1 || orc_kv_a(Lr) > Lr->L) return -1;
  if (orc_kv_b(Lr) < 1 || orc_kv_b(Lr) > Lr->L) return -1;
  if (!orc_is_pow2(Lr->had_in) || Lr->n % Lr->had_in) return -1;
  if (!orc_is_pow2(Lr->had_out) || Lr->m % Lr->had_out) return -1;
  return 0;
}

/* Storage index of tile (R, C): panels of 8 tile-rows, tiles of a panel laid
 * out column by column.                                                      */
int64_t orc_tile_index(int64_t n, int64_t R, int64_t C) {
  int64_t tiles_per_row = n / 16;
  return ((R / 8) * tiles_per_row + C) * 8 + (R % 8);
}

/* Inverse of orc_tile_index, by its definition (panel, column, row-in-panel).*/
void orc_tile_coords(int64_t n, int64_t index, int64_t *R, int64_t *C) {
  int64_t tiles_per_row = n / 16;
  int64_t r8 = index % 8;
  int64_t rest = index / 8;
  *C = rest % tiles_per_row;
  *R = (rest / tiles_per_row) * 8 + r8;
}

/* Where tile (R, C) lives: its step width kV and its first code word.  The
 * tile stream holds 256/V steps of kV bits, (256/V)*kV/32 words.  Tiles of
 * the second part (tile rows from m_a/16 on) follow all tiles of the first
 * and are indexed over the second part's own rows.                           */
static const uint32_t *orc_tile_words(const orc_layer *Lr, int64_t R, int64_t C, int *kV) {
  const int64_t Ra = orc_m_a(Lr) / 16, tpr = Lr->n / 16;
  const int64_t words_a = (256 / Lr->V) * (int64_t)orc_kv_a(Lr) / 32;
  if (R < Ra) {
    *kV = orc_kv_a(Lr);
    return Lr->codes + orc_tile_index(Lr->n, R, C) * words_a;
  }
  *kV = orc_kv_b(Lr);
  const int64_t words_b = (256 / Lr->V) * (int64_t)*kV / 32;
  return Lr->codes + Ra * tpr * words_a + orc_tile_index(Lr->n, R - Ra, C) * words_b;
}

/* Grid coordinates of the tile at storage index `index` (both parts).      */
static void orc_storage_coords(const orc_layer *Lr, int64_t index, int64_t *R, int64_t *C) {
  const int64_t Ra = orc_m_a(Lr) / 16, tiles_a = Ra * (Lr->n / 16);
  if (index < tiles_a) {
    orc_tile_coords(Lr->n, index, R, C);
  } else {
    orc_tile_coords(Lr->n, index - tiles_a, R, C);
    *R += Ra;
  }
}

/* States of tile (R, C): the stream is the tile's (256/V)*kV bits, walked
 * bit-serially with wrap-around (tail-biting); 256/V states.                */
static int orc_tile_states(const orc_layer *Lr, int64_t R, int64_t C,
                           uint32_t states[256]) {
  const int V = Lr->V, L = Lr->L;
  int kV;
  const uint32_t *words = orc_tile_words(Lr, R, C, &kV);
  const int64_t nbits = (256 / V) * (int64_t)kV;
  uint8_t bits[4096];
  if (nbits > 4096 || nbits % 32) return -1;
  for (int64_t p = 0; p < nbits; p++) bits[p] = (uint8_t)orc_bit(words, p);
  return orc_walk_bits(bits, nbits, L, kV, 256 / V, 1, states);
}

/* Value(s) of weight slot j of tile (R, C) given its state: fp16 pattern for
 * decode_tile and the exact fp64 weight (before the layer scale).  NUQ: the
 * fp16 pattern is RNE16(level * group scale); the exact weight is the fp64
 * product.                                                                   */
static int orc_tile_values(const orc_layer *Lr, int64_t R, int64_t C,
                           uint16_t out16[256], double out64[256]) {
  uint32_t states[256];
  if (orc_tile_states(Lr, R, C, states)) return -1;
  const int V = Lr->V;
  for (int64_t t = 0; t < 256 / V; t++) {
    uint32_t s = states[t];
    uint16_t v[2];
    double e[2];
    switch (Lr->code) {
    case ORC_HYB:
      if (V == 2) orc_value_hyb(s, Lr->Q, Lr->lut, v);
      else v[0] = orc_value_hyb1(s, Lr->Q, Lr->lut);
      break;
    case ORC_LUT: v[0] = orc_value_lut(s, Lr->lut); break;
    case ORC_1MAD: v[0] = orc_value_1mad(s); break;
    case ORC_3INST: v[0] = orc_value_3inst(s); break;
    case ORC_NUQ: {
      int64_t row = R * 16 + (t >> 4), col = C * 16 + (t & 15);
      double level = orc_f16_to_double((uint16_t)(Lr->lut[s] & 0xFFFFu));
      double gs = orc_f16_to_double(
          Lr->gscale[row * (Lr->n / Lr->group) + col / Lr->group]);
      e[0] = level * gs;
      v[0] = orc_f16_from_double(e[0]);
      break;
    }
    case ORC_VQ:
      v[0] = (uint16_t)(Lr->lut[s] & 0xFFFFu);
      v[1] = (uint16_t)(Lr->lut[s] >> 16);
      break;
    default: return -1;
    }
    for (int i = 0; i < V; i++) {
      if (Lr->code != ORC_NUQ) e[i] = orc_f16_to_double(v[i]);
      if (out16) out16[t * V + i] = v[i];
      if (out64) out64[t * V + i] = e[i];
    }
  }
  return 0;
}

/* Decode one tile (by grid coordinates) into 256 fp16 bit patterns in
 * tile-local row-major order.                                                */
int orc_decode_tile(const orc_layer *Lr, int64_t R, int64_t C,
                    uint16_t out[256]) {
  if (orc_validate(Lr)) return -1;
  if (R < 0 || R >= Lr->m / 16 || C < 0 || C >= Lr->n / 16) return -1;
  return orc_tile_values(Lr, R, C, out, NULL);
}

/* Decode tiles [first, first+count) in storage order (each mapped back to its
 * grid coordinates, part by part) into out[count][256].                      */
int orc_decode_storage(const orc_layer *Lr, int64_t first, int64_t count,
                       uint16_t *out) {
  if (orc_validate(Lr)) return -1;
  const int64_t total = (Lr->m / 16) * (Lr->n / 16);
  if (first < 0 || count < 0 || first + count > total) return -1;
  int bad = 0;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; i++) {
    int64_t R, C;
    orc_storage_coords(Lr, first + i, &R, &C);
    if (orc_tile_values(Lr, R, C, out + i * 256, NULL)) bad = 1;
  }
  return bad ? -1 : 0;
}

/* Rows [r0, r1) of the effective weight matrix W_hat in fp64 (row-major,
 * (r1-r0) x n): layer scale x exact code value.                              */
static int orc_decode_rows(const orc_layer *Lr, int64_t r0, int64_t r1,
                           double *W) {
  const int64_t n = Lr->n;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t R = r0 / 16; R < r1 / 16; R++) {
    double tile[256];
    for (int64_t C = 0; C < n / 16; C++) {
      if (orc_tile_values(Lr, R, C, NULL, tile)) { bad = 1; continue; }
      for (int j = 0; j < 256; j++) {
        int64_t row = R * 16 + (j >> 4), col = C * 16 + (j & 15);
        W[(row - r0) * n + col] = (double)Lr->scale * tile[j];
      }
    }
  }
  return bad ? -1 : 0;
}

int orc_decode_dense(const orc_layer *Lr, double *W) {
  if (orc_validate(Lr)) return -1;
  return orc_decode_rows(Lr, 0, Lr->m, W);
}

/* ------------------------------------------------------------------------ */
/* Hadamard by definition: H[i][j] = (-1)^popcount(i & j) (Sylvester order). */

static int orc_popcount64(uint64_t v) {
  int c = 0;
  while (v) { c += (int)(v & 1u); v >>= 1; }
  return c;
}

int orc_hadamard_entry(int64_t i, int64_t j) {
  return (orc_popcount64((uint64_t)(i & j)) & 1) ? -1 : 1;
}

static int orc_sign(const uint32_t *signs, int64_t j) {
  if (!signs) return 1;
  return ((signs[j >> 5] >> (j & 31)) & 1u) ? -1 : 1;
}

/* Block-diagonal randomized Hadamard transform of each row of x (rows x n):
 *  mode 0 (input side):  y = scale/sqrt(B) * H (s .* x)
 *  mode 1 (output side): y = s .* (scale/sqrt(B) * H x)
 * naive O(B^2) per block, fp64.                                              */
int orc_rht(const double *x, double *y, int64_t rows, int64_t n, int64_t B,
            const uint32_t *signs, int mode, double scale) {
  if (!orc_is_pow2(B) || n % B || rows < 0) return -1;
  const double norm = scale / sqrt((double)B);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; r++) {
    const double *xr = x + r * n;
    double *yr = y + r * n;
    for (int64_t b0 = 0; b0 < n; b0 += B) {
      for (int64_t i = 0; i < B; i++) {
        double acc = 0.0;
        for (int64_t j = 0; j < B; j++) {
          double xj = xr[b0 + j];
          if (mode == 0) xj *= orc_sign(signs, b0 + j);
          acc += orc_hadamard_entry(i, j) * xj;
        }
        acc *= norm;
        if (mode == 1) acc *= orc_sign(signs, b0 + i);
        yr[b0 + i] = acc;
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* The forward pass (the plain definition of what the library computes):
 *   x'  = (1/sqrt(Bin))  H_in  (s_in .* x)        per input block
 *   z   = W_hat x'                                  fp64 matvec per column
 *   y   = s_out .* ((1/sqrt(Bout)) H_out z)        per output block
 * x is b x n fp16 bit patterns; y is b x m fp64.  W is a caller buffer of
 * m*n doubles (the dense W_hat, filled here).                               */
int orc_forward(const orc_layer *Lr, const uint16_t *x, int64_t b, double *W,
                double *y) {
  if (orc_validate(Lr) || b < 0) return -1;
  const int64_t m = Lr->m, n = Lr->n;
  if (orc_decode_dense(Lr, W)) return -1;
  double *xd = (double *)malloc(sizeof(double) * (size_t)(b * n + 1));
  double *xr = (double *)malloc(sizeof(double) * (size_t)(b * n + 1));
  double *z = (double *)malloc(sizeof(double) * (size_t)(b * m + 1));
  if (!xd || !xr || !z) { free(xd); free(xr); free(z); return -1; }
  for (int64_t i = 0; i < b * n; i++) xd[i] = orc_f16_to_double(x[i]);
  orc_rht(xd, xr, b, n, Lr->had_in, Lr->sign_in, 0, 1.0);
  for (int64_t c = 0; c < b; c++) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < m; r++) {
      double acc = 0.0;
      for (int64_t j = 0; j < n; j++) acc += W[r * n + j] * xr[c * n + j];
      z[c * m + r] = acc;
    }
  }
  orc_rht(z, y, b, m, Lr->had_out, Lr->sign_out, 1, 1.0);
  free(xd); free(xr); free(z);
  return 0;
}

/* Sampled form for full-size layers: outputs y[c][rows in one output block]
 * for selected batch columns, computing only the W_hat rows of that block.
 * cols: list of nc batch column indices; block: output Hadamard block index.
 * y_out: nc x had_out doubles.                                               */
int orc_forward_block(const orc_layer *Lr, const uint16_t *x, int64_t b,
                      const int64_t *cols, int64_t nc, int64_t block,
                      double *y_out) {
  if (orc_validate(Lr) || b < 0) return -1;
  const int64_t m = Lr->m, n = Lr->n, Bo = Lr->had_out;
  if (block < 0 || block >= m / Bo) return -1;
  for (int64_t i = 0; i < nc; i++)
    if (cols[i] < 0 || cols[i] >= b) return -1;
  double *xd = (double *)malloc(sizeof(double) * (size_t)(nc * n + 1));
  double *xr = (double *)malloc(sizeof(double) * (size_t)(nc * n + 1));
  double *Wb = (double *)malloc(sizeof(double) * (size_t)(Bo * n + 1));
  double *z = (double *)malloc(sizeof(double) * (size_t)(nc * Bo + 1));
  if (!xd || !xr || !Wb || !z) { free(xd); free(xr); free(Wb); free(z); return -1; }
  for (int64_t i = 0; i < nc; i++)
    for (int64_t j = 0; j < n; j++) xd[i * n + j] = orc_f16_to_double(x[cols[i] * n + j]);
  orc_rht(xd, xr, nc, n, Lr->had_in, Lr->sign_in, 0, 1.0);
  int bad = orc_decode_rows(Lr, block * Bo, (block + 1) * Bo, Wb) ? 1 : 0;
  if (!bad) {
    for (int64_t i = 0; i < nc; i++) {
#pragma omp parallel for schedule(static)
      for (int64_t r = 0; r < Bo; r++) {
        double acc = 0.0;
        for (int64_t j = 0; j < n; j++) acc += Wb[r * n + j] * xr[i * n + j];
        z[i * Bo + r] = acc;
      }
    }
    /* signs of this block's rows start at bit block*Bo */
    for (int64_t i = 0; i < nc; i++) {
      for (int64_t r = 0; r < Bo; r++) {
        double acc = 0.0;
        for (int64_t j = 0; j < Bo; j++) acc += orc_hadamard_entry(r, j) * z[i * Bo + j];
        acc /= sqrt((double)Bo);
        acc *= orc_sign(Lr->sign_out, block * Bo + r);
        y_out[i * Bo + r] = acc;
      }
    }
  }
  free(xd); free(xr); free(Wb); free(z);
  return bad ? -1 : 0;
}

/* Per-state value for statistics tests (V values as fp16 bit patterns).     */
int orc_state_value(int code, int V, int Q, const uint32_t *lut, uint32_t s,
                    uint16_t out[2]) {
  switch (code) {
  case ORC_HYB:
    if (V == 1) { out[0] = orc_value_hyb1(s, Q, lut); return 1; }
    orc_value_hyb(s, Q, lut, out);
    return 2;
  case ORC_LUT: out[0] = orc_value_lut(s, lut); return 1;
  case ORC_1MAD: out[0] = orc_value_1mad(s); return 1;
  case ORC_3INST: out[0] = orc_value_3inst(s); return 1;
  default: return -1;
  }
}

/* Lloyd-Max quantizer for N(0,1) by plain Lloyd iteration in fp64:
 * alternate nearest-neighbour thresholds (midpoints) and centroids (the
 * conditional means of the Gaussian between thresholds), from a uniform
 * start, for `iters` rounds.  levels: nlev ascending.                        */
static double orc_phi(double t) { return exp(-0.5 * t * t) / sqrt(2.0 * M_PI); }
static double orc_Phi(double t) { return 0.5 * erfc(-t / sqrt(2.0)); }

int orc_lloyd_max_gauss(int nlev, int iters, double *levels, double *mse) {
  if (nlev < 2 || nlev > 256) return -1;
  for (int i = 0; i < nlev; i++) levels[i] = -3.0 + 6.0 * (i + 0.5) / nlev;
  double th[257];
  for (int it = 0; it < iters; it++) {
    th[0] = -INFINITY;
    th[nlev] = INFINITY;
    for (int i = 1; i < nlev; i++) th[i] = 0.5 * (levels[i - 1] + levels[i]);
    for (int i = 0; i < nlev; i++) {
      double a = th[i], b = th[i + 1];
      double pa = isinf(a) ? 0.0 : orc_phi(a), pb = isinf(b) ? 0.0 : orc_phi(b);
      double mass = orc_Phi(b) - orc_Phi(a);
      levels[i] = (pa - pb) / mass;  /* E[X | a < X < b] for N(0,1) */
    }
  }
  if (mse) {
    /* E[(X - q(X))^2] = sum over cells of  E[X^2] - 2 c E[X] + c^2 P  */
    th[0] = -INFINITY;
    th[nlev] = INFINITY;
    for (int i = 1; i < nlev; i++) th[i] = 0.5 * (levels[i - 1] + levels[i]);
    double acc = 0.0;
    for (int i = 0; i < nlev; i++) {
      double a = th[i], b = th[i + 1], c = levels[i];
      double pa = isinf(a) ? 0.0 : orc_phi(a), pb = isinf(b) ? 0.0 : orc_phi(b);
      double apa = isinf(a) ? 0.0 : a * pa, bpb = isinf(b) ? 0.0 : b * pb;
      double P = orc_Phi(b) - orc_Phi(a);
      double EX = pa - pb;
      double EX2 = P + apa - bpb;
      acc += EX2 - 2.0 * c * EX + c * c * P;
    }
    *mse = acc;
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* The encoder: Viterbi on the bitshift trellis.                              */

/* Squared error of one step: targets x[0..V) against scale * values c[0..V),
 * in fp32, products and differences rounded one by one (the build forbids
 * contraction into fused multiply-adds).                                     */
static float orc_step_dist(const float *x, const float *c, float scale, int V) {
  float d = 0.0f;
  for (int i = 0; i < V; i++) {
    float p = scale * c[i];
    float e = x[i] - p;
    float sq = e * e;
    d = (i == 0) ? sq : d + sq;
  }
  return d;
}

/* Viterbi over the bitshift trellis (L state bits, kV new bits per step) for
 * T steps of V targets: state s_t is reached from the 2^kV states whose low
 * L-kV bits are the high L-kV bits of s_t, and the path cost is the fp32
 * sum over t of the squared error of step (t + r) mod T against value(s_t)
 * (vals: 2^L x V floats).  start_P >= 0 admits only first states with high
 * L-kV bits start_P; end_P >= 0 only last states with low L-kV bits end_P.
 * Among equal costs the smaller predecessor, and the smaller last state, win.
 * Writes the best path's states; returns its cost (INFINITY if none).       */
float orc_viterbi(int L, int kV, int V, int T, const float *vals, const float *x, float scale,
                  int r, int64_t start_P, int64_t end_P, uint32_t *states) {
  if (L < 1 || L > 24 || kV < 1 || kV > L || T < 1 || (V != 1 && V != 2)) return NAN;
  const int64_t S = (int64_t)1 << L, G = (int64_t)1 << (L - kV), U = (int64_t)1 << kV;
  float *cost = (float *)malloc(sizeof(float) * (size_t)S);
  float *next = (float *)malloc(sizeof(float) * (size_t)S);
  uint8_t *bp = (uint8_t *)malloc((size_t)(T * G));
  if (!cost || !next || !bp) { free(cost); free(next); free(bp); return NAN; }
  const float *x0 = x + (size_t)(r % T) * V;
  for (int64_t st = 0; st < S; st++) {
    int ok = start_P < 0 || (st >> kV) == start_P;
    cost[st] = ok ? orc_step_dist(x0, vals + st * V, scale, V) : INFINITY;
  }
  for (int t = 1; t < T; t++) {
    const float *xt = x + (size_t)((t + r) % T) * V;
    for (int64_t g = 0; g < G; g++) {
      /* predecessors of the states g * 2^kV + v: u * G + g, u = 0 .. 2^kV-1 */
      float best = cost[g];
      int bu = 0;
      for (int64_t u = 1; u < U; u++) {
        float c = cost[u * G + g];
        if (c < best) { best = c; bu = (int)u; }
      }
      bp[(int64_t)t * G + g] = (uint8_t)bu;
      for (int64_t v = 0; v < U; v++) {
        int64_t st = g * U + v;
        next[st] = best + orc_step_dist(xt, vals + st * V, scale, V);
      }
    }
    float *tmp = cost; cost = next; next = tmp;
  }
  float best = INFINITY;
  int64_t bs = -1;
  for (int64_t st = 0; st < S; st++) {
    if (end_P >= 0 && (st & (G - 1)) != end_P) continue;
    if (bs < 0 || cost[st] < best) { best = cost[st]; bs = st; }
  }
  if (bs >= 0 && !isinf(best)) {
    states[T - 1] = (uint32_t)bs;
    for (int t = T - 1; t >= 1; t--) {
      int64_t g = states[t] >> kV;
      states[t - 1] = (uint32_t)((int64_t)bp[(int64_t)t * G + g] * G + g);
    }
  } else {
    best = INFINITY;
  }
  free(cost); free(next); free(bp);
  return best;
}

/* Tail-biting encode of T steps into a stream of T*kV bits (MSB first in
 * words): the first state's L bits, then the kV new bits of every later
 * state.  exact = 0: the wrap bits P (high L-kV bits of the first state)
 * come from a first pass over the sequence rotated by T/2, whose best path
 * passes through some state at the original step 0; exact = 1: every P is
 * tried (tiny trellises only).  The second pass is the Viterbi with the
 * first state's high bits and the last state's low bits both P, which is
 * exactly the set of tail-biting streams with those wrap bits.  Returns the
 * cost; states (T entries) receives the path.                               */
float orc_encode_stream(int L, int kV, int V, int T, const float *vals, const float *x, float scale,
                        int exact, uint32_t *words, uint32_t *states) {
  const int64_t nbits = (int64_t)T * kV;
  if (nbits < L) return NAN;
  const int64_t G = (int64_t)1 << (L - kV);
  float best;
  if (!exact) {
    const int r = T / 2;
    uint32_t *rot = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)T);
    if (!rot) return NAN;
    float c1 = orc_viterbi(L, kV, V, T, vals, x, scale, r, -1, -1, rot);
    int64_t P = (int64_t)(rot[(T - r) % T] >> kV);
    free(rot);
    if (isnan(c1)) return NAN;
    best = orc_viterbi(L, kV, V, T, vals, x, scale, 0, P, P, states);
  } else {
    uint32_t *tmp = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)T);
    if (!tmp) return NAN;
    best = INFINITY;
    for (int64_t P = 0; P < G; P++) {
      float c = orc_viterbi(L, kV, V, T, vals, x, scale, 0, P, P, tmp);
      if (c < best) { best = c; memcpy(states, tmp, sizeof(uint32_t) * (size_t)T); }
    }
    free(tmp);
  }
  if (isnan(best) || isinf(best)) return best;
  const int64_t nwords = (nbits + 31) / 32;
  memset(words, 0, sizeof(uint32_t) * (size_t)nwords);
  int64_t pos = 0;
  for (int i = L - 1; i >= 0 && pos < nbits; i--, pos++)
    if ((states[0] >> i) & 1u) words[pos >> 5] |= 1u << (31 - (pos & 31));
  for (int t = 1; t < T; t++)
    for (int i = kV - 1; i >= 0 && pos < nbits; i--, pos++)
      if ((states[t] >> i) & 1u) words[pos >> 5] |= 1u << (31 - (pos & 31));
  return best;
}

/* Encode a whole layer: W (m x n fp32, row-major) -> codes_out in the
 * layer's packed format (both parts of a half-TCQ layer), each tile
 * minimising its squared error against layer_scale x value.  The layer's
 * code, V, Q, lut and widths select the trellis; its codes pointer is not
 * read.  sse_out (optional): the sum of the tiles' path costs.              */
int orc_encode_layer(const orc_layer *Lr, const float *W, uint32_t *codes_out, int exact,
                     double *sse_out) {
  if (orc_validate(Lr) || !orc_is_trellis(Lr->code) || Lr->L != 16) return -1;
  const int V = Lr->V, T = 256 / V;
  const int64_t S = (int64_t)1 << Lr->L;
  float *vals = (float *)malloc(sizeof(float) * (size_t)(S * V));
  if (!vals) return -1;
  for (int64_t st = 0; st < S; st++) {
    uint16_t o[2];
    orc_state_value(Lr->code, V, Lr->Q, Lr->lut, (uint32_t)st, o);
    for (int i = 0; i < V; i++) vals[st * V + i] = (float)orc_f16_to_double(o[i]);
  }
  const int64_t tiles = (Lr->m / 16) * (Lr->n / 16);
  double sse = 0.0;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : sse)
  for (int64_t i = 0; i < tiles; i++) {
    int64_t R, C;
    int kV;
    orc_storage_coords(Lr, i, &R, &C);
    const uint32_t *w = orc_tile_words(Lr, R, C, &kV);
    float x[256];
    uint32_t st[256];
    for (int j = 0; j < 256; j++) x[j] = W[(R * 16 + (j >> 4)) * Lr->n + C * 16 + (j & 15)];
    float c = orc_encode_stream(Lr->L, kV, V, T, vals, x, Lr->scale, exact,
                                codes_out + (w - Lr->codes), st);
    if (isnan(c) || isinf(c)) bad = 1;
    else sse += c;
  }
  free(vals);
  if (sse_out) *sse_out = sse;
  return bad ? -1 : 0;
}

int orc_omp_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Thread count of the OpenMP loops that follow (timing the oracle on one
 * core and on all of them). */
void orc_set_threads(int n) {
#ifdef _OPENMP
  extern void omp_set_num_threads(int);
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
