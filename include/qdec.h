/*
 * qdec -- weight-only quantized matrix multiplication on AMD Instinct MI355X
 * (gfx950): y = W_hat x, with W_hat decoded on the fly from packed low-bit
 * codes and wrapped in incoherence processing.
 *
 * What is computed.  The weight matrix is stored as  W = S_out H_out W_hat
 * H_in S_in  (randomized Hadamard transform, RHT, on both sides: "QTIP:
 * Quantization with Trellises and Incoherence Processing", author response
 * "Incoherence Processing (W2)" and "Bit Accounting (Q2)"; QuIP#, Fig. 2).
 * A call computes, for every batch row x of X (fp16):
 *
 *     x' = (1/sqrt(B_in))  H_{B_in}  (s_in .* x)         block-diagonal over n
 *     z  = W_hat x'                                        fp32 accumulate
 *     y  = s_out .* ((1/sqrt(B_out)) H_{B_out} z)         block-diagonal over m
 *
 * and rounds y to fp16 (round to nearest even).  H_B is the Sylvester-ordered
 * Hadamard matrix, H[i][j] = (-1)^popcount(i & j).  Small-batch inference is
 * memory bound, so the codes are streamed from HBM once and decoded in
 * registers ("QTIP's contribution (W1)"); the problem is weight-only
 * quantized MatMul with activations kept in floating point (the quantized
 * MatMul rate-distortion abstract, "WaterSIC").
 *
 * Codes (W_hat = layer_scale x value; see the packed format below):
 *  - QDEC_CODE_HYB   bitshift trellis, L = 16, V = 2, k bits per weight; the
 *                    state is hashed, h = s*s + s mod 2^16; Q index bits
 *                    [15-Q, 15) of h pick a fp16 pair from a 2^Q-entry LUT
 *                    and bit 15 of h flips the sign of both halves
 *                    (untitled ALU-op comment, "HYB Uniqueness (Q2)").
 *                    With V = 1 the same index picks one fp16 value and bit
 *                    15 flips its sign (a one-dimensional codebook, "Other
 *                    hardware (e.g. ARM) (W3)": Q = 6, V = 1).
 *  - QDEC_CODE_1MAD  bitshift trellis, L = 16, V = 1; u = 0xEA4F79*s +
 *                    0xC2AA9973 (mod 2^32); value = fp16(fp32((b0+b1+b2+b3
 *                    - 510) * fp32(1/sqrt(21845)))), b_i the bytes of u.
 *  - QDEC_CODE_3INST bitshift trellis, L = 16, V = 1; u = 0xE77B2B*s +
 *                    0xEACB81D7; u = (u & 0x8FFF8FFF) | 0x30003000; value =
 *                    fp16(lo16(u) + hi16(u)) with both halves read as fp16.
 *                    (1MAD/3INST: computed codes with a fixed instruction
 *                    count and no LUT, built on an LCG -- computed-codes reply
 *                    and "LCG citation (O2)"; the constants are this
 *                    library's own.)
 *  - QDEC_CODE_NUQ   non-uniform scalar quantizer ("Q-Palette" summary):
 *                    L = k, V = 1, a k-bit index into a 2^k-entry fp16 level
 *                    table, times an fp16 scale per `group` weights of a row.
 *  - QDEC_CODE_VQ    2-D vector quantizer ("Q-Palette" summary): L = 2k,
 *                    V = 2, one 2k-bit index per weight pair into a 2^(2k)
 *                    table of fp16 pairs.  With L = kV the trellis reduces to
 *                    plain k-bit V-dim VQ ("Ablations and fast inference").
 *  - QDEC_CODE_LUT   pure lookup ("Ablations and fast inference (W1 and
 *                    W2)", Table A): bitshift trellis, L = 16, V = 1; the
 *                    state itself indexes a table of 2^16 fp16 values
 *                    (16 x 2^L bits = 128 KiB, held in LDS).
 *
 * Bit widths.  A trellis step (or a NUQ/VQ index) takes kV bits for V
 * weights: k = kV/V bits per weight.  The trellis codes may give kV directly
 * (field kv), which allows fractional widths at V = 2: kV = 5 is 2.5 bits
 * per weight, kV = 7 is 3.5 ("Q-Palette" summary: fractional-bit
 * quantizers).  Half-TCQ ("Q-Palette" summary: two trellis widths in one
 * layer, 2.5 and 3 bits averaging 2.75) cuts the rows at m_a, a multiple of
 * 128: rows [0, m_a) take kv, rows [m_a, m) take kv_b.
 *
 * Packed format (version 2).
 *  - W_hat is cut into 16x16 tiles; tile (R, C) covers rows 16R..16R+15 and
 *    columns 16C..16C+15; weight j of a tile sits at (j >> 4, j & 15).
 *  - Each tile is a stream of (256/V)*kV bits held in (256/V)*kV/32
 *    little-endian uint32 words; stream bit p is bit 31 - (p & 31) of word
 *    p >> 5 (MSB first).
 *  - Step t (t = 0 .. 256/V - 1) covers weights tV .. tV+V-1.  Its state is
 *    the L-bit window starting at stream bit t*kV, read MSB first, wrapping
 *    around the end of the tile's stream (tail-biting): each state is the
 *    previous one shifted left by kV bits with kV new bits appended, so two
 *    neighbours share L-kV bits ("Figure 2 (Q4)"), so every
 *    bit string is a valid walk and storage is exactly k bits per weight.
 *  - Tiles are stored in panels of 8 tile-rows (128 output rows); inside a
 *    panel, column by column: storage index of tile (R, C) is
 *      ((R / 8) * (n / 16) + C) * 8 + (R % 8).
 *    A half-TCQ layer stores the tiles of rows [0, m_a) this way, then those
 *    of rows [m_a, m), indexed as a layer of their own (R counted from m_a/16),
 *    at their own width; storage indices run on across the two parts.
 *  - HYB LUT: 2^Q uint32 words, each an fp16 pair (low half = first weight);
 *    at V = 1, each word's low half is the value (the high half is ignored).
 *    NUQ table: 2^k uint32 words, fp16 level in the low half.  VQ table:
 *    2^(2k) uint32 words, fp16 pairs.  LUT table: 2^15 uint32 words holding
 *    the 2^16 fp16 values, entry e in the low half of word e/2 when e is
 *    even, the high half when odd.  NUQ group scales: fp16 [m][n/group].
 *  - Sign vectors: bit j (bit j & 31 of word j >> 5) set means s[j] = -1;
 *    NULL means all +1.  They take n + m bits ("Bit Accounting (Q2)").
 *
 * Conventions.
 *  - Every pointer is a DEVICE pointer owned by the caller; the library never
 *    allocates, frees or synchronizes.  `stream` is a hipStream_t passed as
 *    void* (NULL = the default stream); every call is asynchronous on it.
 *  - Argument errors are found on the host before any launch and return a
 *    negative status with no device work queued.  A failed launch returns
 *    QDEC_EHIP.  No exception crosses this interface.
 *  - Workspaces: size them with qdec_workspace_bytes (or
 *    qdec_gemv_group_workspace_bytes); their contents on entry do not
 *    matter -- every part of it a call reads, the same call has written.
 *    Calls that share one workspace must be ordered (same stream).
 *  - Results are reproducible bit for bit: every split of the K dimension
 *    writes a slice of its own (plain stores, no atomics) and the slices
 *    are added in a fixed order.
 *  - x and y must not overlap.  The library is reentrant: its only state is
 *    per-device kernel attributes and device checks, set with atomic
 *    operations, and per-thread call plans.
 *  - Sizes: m, n <= 2^20 and code bytes below 2^31 per layer
 *    (QDEC_EUNSUPPORTED beyond): kernels address a layer through 32-bit
 *    buffer offsets.
 */
#ifndef QDEC_H
#define QDEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QDEC_ABI_VERSION 2u

typedef enum {
  QDEC_OK = 0,
  QDEC_EINVAL = -1,      /* bad argument or descriptor                     */
  QDEC_EUNSUPPORTED = -2,/* valid but not built (a code/k/V/batch combo)    */
  QDEC_EWORKSPACE = -3,  /* workspace missing, misaligned or too small      */
  QDEC_EHIP = -4,        /* a HIP runtime call or launch failed             */
  QDEC_ENODEV = -5       /* no usable gfx950 device                         */
} qdec_status;

typedef enum {
  QDEC_CODE_HYB = 1,
  QDEC_CODE_1MAD = 2,
  QDEC_CODE_3INST = 3,
  QDEC_CODE_NUQ = 4,
  QDEC_CODE_VQ = 5,
  QDEC_CODE_LUT = 6
} qdec_code;

/* One quantized linear layer.  Plain data; all pointers are device pointers
 * owned by the caller.  Supported combinations (kV = k*V, or kv):
 *   HYB    L = 16, V = 2, kV in {4, 5, 6, 7, 8}; or V = 1, kV in {2, 3, 4};
 *          Q in [1, 11]
 *   1MAD   L = 16, V = 1, kV in {2, 3, 4}
 *   3INST  L = 16, V = 1, kV in {2, 3, 4}
 *   NUQ    L = k,  V = 1, k in {2, 3, 4}, group a multiple of 16 dividing n
 *   VQ     L = 2k, V = 2, k in {2, 3, 4}
 *   LUT    L = 16, V = 1, kV in {2, 3, 4}
 * The trellis codes (HYB, 1MAD, 3INST, LUT) may set kv (then k = 0) and a
 * second part (m_a, kv_b), each width one of the above.
 * m % 128 == 0, n % 16 == 0; had_in (had_out) a power of two dividing n (m),
 * at most 16384; codes 16-byte aligned.                                      */
typedef struct qdec_layer {
  uint32_t abi_version;          /* QDEC_ABI_VERSION                          */
  int32_t code;                  /* qdec_code                                 */
  int32_t L, k, V, Q;            /* state bits, bits/weight, weights/step, HYB index bits */
  int32_t kv;                    /* trellis bits per step of rows [0, m_a); 0 = k*V */
  int32_t kv_b;                  /* bits per step of rows [m_a, m); 0 when m_a = 0 */
  int64_t m_a;                   /* half-TCQ: rows of the first part; 0 = one part */
  int64_t m, n;                  /* W_hat is m (out) x n (in)                 */
  const uint32_t *codes;         /* m*n*kV/(32V) words (summed over the parts) */
  const uint32_t *lut;           /* HYB / NUQ / VQ / LUT table (see format), else NULL */
  const uint16_t *group_scale;   /* NUQ: fp16 [m][n/group]; else NULL         */
  int32_t group;                 /* NUQ group length along a row; else 0      */
  float layer_scale;             /* multiplies every decoded value            */
  const uint32_t *sign_in;       /* n bits or NULL                            */
  const uint32_t *sign_out;      /* m bits or NULL                            */
  int32_t had_in, had_out;       /* RHT block sizes (1 = no Hadamard)         */
} qdec_layer;

/* Operation selector for qdec_workspace_bytes.                               */
#define QDEC_OP_GEMV 1
#define QDEC_OP_GEMM 2
#define QDEC_OP_ENCODE 3

/* Bytes of workspace qdec_gemv (op = QDEC_OP_GEMV), qdec_gemm
 * (op = QDEC_OP_GEMM) or qdec_encode (op = QDEC_OP_ENCODE, batch = 1) needs
 * for this layer at this batch.  0 on a bad argument.                        */
size_t qdec_workspace_bytes(const qdec_layer *layer, int64_t batch, int32_t op);

/* Randomized Hadamard transform of `rows` rows of length n, block-diagonal
 * with block size `block` (a power of two dividing n, at most 16384):
 *   mode 0 (input side):  out = scale/sqrt(block) * H (s .* in)
 *   mode 1 (output side): out = s .* (scale/sqrt(block) * H in)
 * in/out: row-major, dtype 0 = fp16, 1 = fp32; in-place allowed when the
 * dtypes match.  signs: n bits or NULL.  ("Incoherence Processing (W2)";
 * QuIP# abstract and Fig. 2.)                                                 */
int qdec_rht(const void *in, int32_t in_dtype, void *out, int32_t out_dtype,
             int64_t rows, int64_t n, int32_t block, const uint32_t *signs,
             int32_t mode, float scale, void *stream);

/* Fused decode-and-multiply for small batches ("QTIP's contribution (W1)":
 * small-batch inference is memory bound, so the weights are decoded on the
 * fly): Y[b][m] = layer(X[b][n]) as defined above, 1 <= batch <= 8, fp16
 * in/out, fp32 accumulation.  Two launches: one kernel decodes and
 * multiplies, the finisher adds its K slices and applies the output
 * transform.  At one batch column the decode kernel also applies the input
 * transform: for HYB codes (V = 2) on layers of at least 1.6e7 weights
 * (4096 x 4096 and up) it is the MFMA kernel (one workgroup per CU; the
 * decoded weights are MFMA operands), otherwise the dot-product kernel.  With more batch columns the input transform runs
 * first in a kernel of its own, and on large layers (NB * m * n >= 4e8,
 * NB = batch rounded up to 2, 4 or 8) the call runs the batched path of
 * qdec_gemm instead.  x 16-byte and y 8-byte aligned.
 * ws: qdec_workspace_bytes(layer, batch, QDEC_OP_GEMV) bytes, 256-byte
 * aligned; its contents on entry do not matter.  A workspace sized for a
 * batch serves every smaller batch of the same layer.                       */
int qdec_gemv(const qdec_layer *layer, const uint16_t *x, uint16_t *y,
              int64_t batch, void *ws, size_t ws_bytes, void *stream);

/* qdec_gemv without a caller-provided workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The workspace is a static device array
 * of qdec_noalloc_scratch_bytes() = 8 MiB inside the library: each device
 * holds its own copy until the process ends; the call itself allocates and
 * frees nothing.  Layers whose qdec_gemv workspace at this batch exceeds it
 * return QDEC_EWORKSPACE before any launch.  Every call on one device shares
 * that device's array: calls that overlap in time on one device (other
 * streams, other threads) race and must be ordered by the caller.  Nothing in
 * the array needs to start at zero.  Otherwise as qdec_gemv.                 */
int qdec_gemv_noalloc(const qdec_layer *layer, const uint16_t *x, uint16_t *y, int64_t batch,
                      void *stream);

/* Bytes of the static workspace of qdec_gemv_noalloc.                         */
size_t qdec_noalloc_scratch_bytes(void);

/* Several independent one-column products in one call (the projections of
 * a decoder layer that read the same activations, e.g. q, k and v, or gate
 * and up): y[l] = layers[l](x[l]) for l < count <= 8, each as qdec_gemv at
 * batch 1.  The row parts of all layers that share a code, width and Q run in
 * one launch of the one-column MFMA kernel, and one finisher launch serves
 * every layer, so a group costs two launches instead of two per layer.
 * x[l]: [n_l] fp16, 16-byte aligned; y[l]: [m_l] fp16, 8-byte aligned, no
 * y overlapping any x or another y (x may be shared).  ws:
 * qdec_gemv_group_workspace_bytes(layers, count) bytes, 256-byte aligned;
 * its contents on entry do not matter.  QDEC_EUNSUPPORTED when a layer's
 * row or lookup table does not fit the kernel's LDS (rows wider than 16384
 * columns).                                                                   */
int qdec_gemv_group(const qdec_layer *const *layers, int32_t count, const uint16_t *const *x,
                    uint16_t *const *y, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes of qdec_gemv_group for these layers (0 on a bad argument). */
size_t qdec_gemv_group_workspace_bytes(const qdec_layer *const *layers, int32_t count);

/* Batched decode-and-multiply (prefill): same result as qdec_gemv for
 * 1 <= batch <= 256; decoded weights go from registers straight into fp16
 * MFMA (the transformed activations are staged in LDS), fp32 accumulation.
 * Three launches on `stream` (input RHT, GEMM, output RHT).
 * ws: qdec_workspace_bytes(layer, batch, QDEC_OP_GEMM) bytes, 256-byte
 * aligned; its contents on entry do not matter.                             */
int qdec_gemm(const qdec_layer *layer, const uint16_t *x, uint16_t *y,
              int64_t batch, void *ws, size_t ws_bytes, void *stream);

/* Tail-biting trellis encoder, the step before the matmuls: writes into
 * `codes` (the layer's code words in the packed format, both parts of a
 * half-TCQ layer) the streams that minimise, tile by tile, the squared error
 * sum (w - layer_scale x value)^2 against w (fp32 [m][n], row-major, device;
 * finite values).  The search is the Viterbi algorithm on the bitshift
 * trellis ("Figure 2 (Q4)": the predecessors of a state are the 2^kV states
 * whose low L-kV bits are its high L-kV bits; "Why does TCQ work? (Q5)").
 * The wrap of a tail-biting stream is chosen by a first, free-ended pass
 * over the step sequence rotated by half its length (the high L-kV bits of
 * the state its best path takes at step 0); the second pass is the exact
 * Viterbi over the streams with that wrap.  Path costs are fp32 sums in a
 * fixed order, ties to the smaller predecessor and last state, so the codes
 * are a deterministic function of w.  Codes HYB (V = 1, 2), 1MAD and 3INST
 * (QDEC_EUNSUPPORTED otherwise); layer->codes is not read.  ws:
 * qdec_workspace_bytes(layer, 1, QDEC_OP_ENCODE) bytes, 256-byte aligned;
 * its contents do not matter.  codes: 16-byte aligned, not overlapping w.  */
int qdec_encode(const qdec_layer *layer, const float *w, uint32_t *codes, void *ws,
                size_t ws_bytes, void *stream);

/* Decode tiles [first_tile, first_tile + n_tiles) in storage order into
 * out[n_tiles][256] fp16, tile-local row-major.  Values are the code values
 * before the layer scale (HYB/VQ pairs, 1MAD/3INST values), and for NUQ
 * fp16(level * group scale).  Runs the same device decoders as the matmuls;
 * it is the bit-exact parity surface.                                        */
int qdec_decode_tile(const qdec_layer *layer, int64_t first_tile,
                     int64_t n_tiles, uint16_t *out, void *stream);

/* Test hook for callers' error paths: the next `count` calls (of any entry
 * point) that pass their argument checks and find a gfx950 device return
 * QDEC_EHIP without launching anything, and qdec_last_error names the hook.
 * count = 0 clears it.  QDEC_EINVAL for a negative count.  The count is
 * shared by every thread of the process.                                    */
int qdec_debug_fail_launches(int32_t count);

/* Human-readable name of a status code (static storage).                    */
const char *qdec_status_string(int status);

/* ABI version of the loaded library (QDEC_ABI_VERSION).                      */
uint32_t qdec_abi_version(void);

/* Text of the HIP error behind the calling thread's last QDEC_EHIP (static,
 * per-thread storage; "no error" if there was none).                         */
const char *qdec_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QDEC_H */
