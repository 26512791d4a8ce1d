// qdec_encode: the tail-biting trellis encoder (the step before the matmul).
//
// Each 16x16 tile is quantized to the stream of (256/V) steps of KV bits
// whose cyclic walk minimises the squared error against the tile's targets
// (Viterbi on the bitshift trellis: "QTIP: Quantization with Trellises and
// Incoherence Processing", "Figure 2 (Q4)" -- the trellis is the numbering
// of the states, the predecessors of s are the 2^KV states whose low L-KV
// bits are the high L-KV bits of s; "Why does TCQ work? (Q5)").  A tile is
// encoded in two passes: the first, free-ended, over the step sequence
// rotated by half its length, picks the L-KV wrap bits P from the state its
// best path takes at the original step 0; the second is the Viterbi whose
// first state has high bits P and whose last state has low bits P, i.e.
// exactly the tail-biting streams with that wrap.
//
// One workgroup of 1024 threads encodes one tile at a time (a persistent
// grid walks the tiles).  The 2^16 path costs live in registers, 64 per
// thread: thread t owns the states u * G + g (G = 2^(16-KV)) for its
// groups g and a range of u, so the minimum over the 2^KV predecessors of
// a group is formed in registers (and, at KV >= 7, across 2 or 4 lanes);
// the G minima go through LDS once per step, and every thread adds the
// squared error of its own states' values.  The arithmetic is fp32 in a
// fixed order with no contraction, ties going to the smaller predecessor
// and the smaller last state, so the result is that of a plain sequential
// Viterbi with the same rules.  The winning predecessor of every group and
// step goes to the workspace (one word per thread and step); the traceback
// reads it back in chunks through LDS.
#include "gemv_impl.hpp"
#include "qdec_device.hpp"
#include "qdec_internal.hpp"

namespace qdec {

constexpr int ENC_THREADS = 1024;

template <int KV>
struct EncGeom {
  static constexpr int L = 16;
  static constexpr int G = 1 << (L - KV);        // groups (predecessor sets)
  static constexpr int U = 1 << KV;              // predecessors per group
  static constexpr int UPT = U < 64 ? U : 64;    // predecessors per thread
  static constexpr int GPT = 64 / UPT;           // groups per thread
  static constexpr int TPG = U / UPT;            // threads per group (KV >= 7)
  static_assert(GPT * ENC_THREADS / TPG == G, "every group owned once");
  // LDS words of the minima / traceback area: at least 8 steps of words
  static constexpr int AREA = G > 8 * ENC_THREADS ? G : 8 * ENC_THREADS;
  static constexpr int CH = AREA / ENC_THREADS;  // traceback steps per chunk
};

// Squared error of one step (V targets against scale x the state's values),
// in fp32, rounding every product and sum on its own.
template <int V>
__device__ __forceinline__ float enc_step_dist(const float* x, const float* c, float scale) {
#pragma clang fp contract(off)
  float d = 0.0f;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const float p = scale * c[i];
    const float e = x[i] - p;
    const float sq = e * e;
    d = (i == 0) ? sq : d + sq;
  }
  return d;
}

template <int CODE>
__device__ __forceinline__ void enc_values(uint32_t s, const uint32_t* tab, int qshift, float* c) {
  if constexpr (CODE == HYB) {
    const uint32_t pr = tab[hyb_signed_index(s, qshift)];
    c[0] = h2f((uint16_t)(pr & 0xFFFFu));
    c[1] = h2f((uint16_t)(pr >> 16));
  } else if constexpr (CODE == HYB1) {
    c[0] = h2f((uint16_t)(tab[hyb_signed_index(s, qshift)] & 0xFFFFu));
  } else if constexpr (CODE == MAD1) {
    c[0] = h2f(mad1_value_bits(s));
  } else {
    c[0] = h2f(inst3_value_bits(s));
  }
}

__device__ __forceinline__ float enc_add(float a, float b) {
#pragma clang fp contract(off)
  return a + b;
}

// Lexicographic minimum of (cost, index) pairs, as a scan in index order
// with a strict comparison would find it.
__device__ __forceinline__ void enc_take_min(float& c, uint32_t& i, float c2, uint32_t i2) {
  const bool take = c2 < c || (c2 == c && i2 < i);
  c = take ? c2 : c;
  i = take ? i2 : i;
}

template <int CODE, int KV>
__global__ __launch_bounds__(ENC_THREADS) void encode_kernel(EncodeArgs a) {
  using E = EncGeom<KV>;
  constexpr int V = code_V(CODE);
  constexpr int T = 256 / V;
  constexpr int G = E::G, U = E::U, UPT = E::UPT, GPT = E::GPT, TPG = E::TPG;
  constexpr int TW = T * KV / 32;                 // stream words per tile
  extern __shared__ __align__(16) uint32_t smem[];
  float* area = reinterpret_cast<float*>(smem);   // [AREA]: group minima, or traceback chunks
  uint32_t* bpl = smem;                           // the same words, as backpointers
  float* xs = reinterpret_cast<float*>(smem + E::AREA);   // [256] targets of the tile
  uint32_t* stream = smem + E::AREA + 256;        // [TW] stream words being assembled
  __shared__ float red_c[ENC_THREADS / 64];
  __shared__ uint32_t red_i[ENC_THREADS / 64];
  __shared__ uint32_t bcast;
  uint32_t* tab = smem + E::AREA + 256 + 64;      // HYB table (2^(Q+1) signed entries)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if constexpr (CODE == HYB) fill_signed_table<1>(tab, a.L.lut, a.L.Q, tid, ENC_THREADS);
  if constexpr (CODE == HYB1) fill_signed_table<1, 0x8000u>(tab, a.L.lut, a.L.Q, tid, ENC_THREADS);

  // this thread's states: u = u0 + uu (uu < UPT), g = g0 + j (j < GPT)
  const uint32_t g0 = TPG == 1 ? (uint32_t)tid * GPT : (uint32_t)(tid / TPG);
  const uint32_t u0 = TPG == 1 ? 0u : (uint32_t)(tid % TPG) * UPT;
  uint32_t* bpw = a.bp + (size_t)blockIdx.x * T * ENC_THREADS;   // [T][1024] words
  const int64_t tpr = a.L.n >> 4;

  for (int64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
    // tile (R, C) of this part from its storage index (panel order)
    const int64_t r8 = tile & 7, rest = tile >> 3;
    const int64_t C = rest % tpr, R = (rest / tpr) * 8 + r8;
    __syncthreads();   // the previous tile's traceback is done with LDS
    if (tid < 256) {
      const int64_t row = a.row0 + R * 16 + (tid >> 4), col = C * 16 + (tid & 15);
      xs[tid] = a.w[row * a.L.n + col];
    }
    if (tid < TW) stream[tid] = 0u;

    uint32_t P = 0;
#pragma nounroll
    for (int pass = 0; pass < 2; ++pass) {
      const int r = pass == 0 ? T / 2 : 0;        // rotation of the step sequence
      float c[UPT][GPT];
      __syncthreads();                             // targets (and, first, the table) in LDS
      {
        float xv[V];
#pragma unroll
        for (int i = 0; i < V; ++i) xv[i] = xs[(r % T) * V + i];
        uint32_t sbase = u0 * G + g0;
        asm volatile("" : "+v"(sbase));   // no tile-invariant values held across tiles
#pragma unroll
        for (int uu = 0; uu < UPT; ++uu)
#pragma unroll
          for (int j = 0; j < GPT; ++j) {
            const uint32_t s = sbase + (uint32_t)(uu * G + j);
            float cv[V];
            enc_values<CODE>(s, tab, a.L.qshift, cv);
            const float d = enc_step_dist<V>(xv, cv, a.L.scale);
            c[uu][j] = (pass == 0 || (s >> KV) == P) ? d : __builtin_inff();
          }
      }
#pragma nounroll
      for (int t = 1; t < T; ++t) {
        // (A) minimum over the predecessors of each owned group
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < GPT; ++j) {
          float best = c[0][j];
          uint32_t bu = u0;
#pragma unroll
          for (int uu = 1; uu < UPT; ++uu) {
            const bool lt = c[uu][j] < best;
            best = lt ? c[uu][j] : best;
            bu = lt ? u0 + uu : bu;
          }
          if constexpr (TPG > 1) {
#pragma unroll
            for (int msk = 1; msk < TPG; msk <<= 1) {
              const float ob = __shfl_xor(best, msk, 64);
              const uint32_t ou = (uint32_t)__shfl_xor((int)bu, msk, 64);
              enc_take_min(best, bu, ob, ou);
            }
            if (tid % TPG == 0) area[g0] = best;
            word = bu;
          } else {
            area[g0 + j] = best;
            word |= bu << (KV * j);
          }
        }
        bpw[(size_t)t * ENC_THREADS + tid] = word;
        __syncthreads();
        // (B) new costs: minimum of the state's group plus its step error
        float xv[V];
#pragma unroll
        for (int i = 0; i < V; ++i) xv[i] = xs[((t + r) % T) * V + i];
        // in batches of 8 states, so that the LDS reads in flight stay few
        // (the 64 path costs already fill half of the registers); the state
        // numbers are recomputed every step (an opaque copy of the base
        // keeps the compiler from holding 64 step-invariant values live)
        uint32_t sbase = u0 * G + g0;
        asm volatile("" : "+v"(sbase));
#pragma unroll
        for (int b0 = 0; b0 < 64; b0 += 8) {
#pragma unroll
          for (int bi = 0; bi < 8; ++bi) {
            const int uu = (b0 + bi) / GPT, j = (b0 + bi) % GPT;
            const uint32_t s = sbase + (uint32_t)(uu * G + j);
            float cv[V];
            enc_values<CODE>(s, tab, a.L.qshift, cv);
            const float d = enc_step_dist<V>(xv, cv, a.L.scale);
            c[uu][j] = enc_add(area[s >> KV], d);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();   // every thread has read the minima
      }
      // best last state: smallest cost, then smallest index (pass 2: low
      // L-KV bits must be P)
      float bc = __builtin_inff();
      uint32_t bi = 0xFFFFFFFFu;
#pragma unroll
      for (int uu = 0; uu < UPT; ++uu)
#pragma unroll
        for (int j = 0; j < GPT; ++j) {
          const uint32_t s = (u0 + uu) * G + g0 + j;
          if (pass == 0 || (s & (G - 1)) == P) enc_take_min(bc, bi, c[uu][j], s);
        }
#pragma unroll
      for (int msk = 1; msk < 64; msk <<= 1) {
        const float oc = __shfl_xor(bc, msk, 64);
        const uint32_t oi = (uint32_t)__shfl_xor((int)bi, msk, 64);
        enc_take_min(bc, bi, oc, oi);
      }
      if (lane == 0) {
        red_c[wave] = bc;
        red_i[wave] = bi;
      }
      __syncthreads();
      if (tid == 0) {
        float fc = red_c[0];
        uint32_t fi = red_i[0];
        for (int w = 1; w < ENC_THREADS / 64; ++w) enc_take_min(fc, fi, red_c[w], red_i[w]);
        bcast = fi;
      }
      __syncthreads();
      uint32_t s = bcast;
      // traceback: pass 1 down to the rotated step T - r (the original step
      // 0), pass 2 to step 0, CH steps of backpointers at a time through LDS;
      // pass 2 writes each state's new bits into the stream (bits past the
      // tile's T*KV are the wrap P again and are dropped)
      const int tstop = pass == 0 ? T - r : 0;
      for (int hi = T - 1; hi > tstop; hi -= E::CH) {
        const int lo = hi - E::CH + 1 > tstop + 1 ? hi - E::CH + 1 : tstop + 1;   // steps lo .. hi
        __syncthreads();
        for (int i = tid; i < (hi - lo + 1) * ENC_THREADS; i += ENC_THREADS)
          bpl[i] = bpw[(size_t)lo * ENC_THREADS + i];
        __syncthreads();
        if (tid == 0) {
          for (int t = hi; t >= lo; --t) {
            if (pass == 1) {
              const int pos = 16 + (t - 1) * KV;       // first bit of step t's new bits
              const uint32_t nb = s & (U - 1);
#pragma unroll
              for (int i = 0; i < KV; ++i) {
                const int p = pos + i;
                if (p < T * KV && ((nb >> (KV - 1 - i)) & 1u)) stream[p >> 5] |= 1u << (31 - (p & 31));
              }
            }
            const uint32_t g = s >> KV;
            const uint32_t own = TPG == 1 ? g / GPT : g * TPG;
            const uint32_t sh = TPG == 1 ? KV * (g % GPT) : 0u;
            const uint32_t u = (bpl[(t - lo) * ENC_THREADS + own] >> sh) & (U - 1);
            s = u * G + g;
          }
        }
      }
      if (tid == 0) {
        if (pass == 0) {
          bcast = s >> KV;
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i)   // the first state's 16 bits
            if ((s >> (15 - i)) & 1u) stream[i >> 5] |= 1u << (31 - (i & 31));
        }
      }
      __syncthreads();
      P = bcast;
    }
    if (tid < TW) a.codes[tile * TW + tid] = stream[tid];
  }
}

template <int CODE, int KV>
static hipError_t launch_encode_t(const EncodeArgs& a, hipStream_t stream) {
  using E = EncGeom<KV>;
  const size_t tabw = (CODE == HYB || CODE == HYB1) ? (size_t)(2 << a.L.Q) : 0;
  const size_t lds = ((size_t)E::AREA + 256 + 64 + tabw) * 4;
  static LdsLimit have;
  const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&encode_kernel<CODE, KV>), lds, &have);
  if (e != hipSuccess) return e;
  const int64_t grid = a.ntiles < ENCODE_GRID ? a.ntiles : ENCODE_GRID;
  hipLaunchKernelGGL((encode_kernel<CODE, KV>), dim3((unsigned)grid), dim3(ENC_THREADS), lds, stream, a);
  return hipGetLastError();
}

template <int CODE>
static hipError_t launch_encode_code(const EncodeArgs& a, hipStream_t stream) {
#define QDEC_ENC_KV(KV)                                                            \
  case KV:                                                                        \
    if constexpr (kv_built(CODE, KV)) return launch_encode_t<CODE, KV>(a, stream); \
    break;
  switch (a.L.kv) {
    QDEC_ENC_KV(2) QDEC_ENC_KV(3) QDEC_ENC_KV(4) QDEC_ENC_KV(5)
    QDEC_ENC_KV(6) QDEC_ENC_KV(7) QDEC_ENC_KV(8)
    default: break;
  }
#undef QDEC_ENC_KV
  return hipErrorInvalidValue;
}

hipError_t launch_encode(const EncodeArgs& a, hipStream_t stream) {
  if (a.ntiles <= 0) return hipSuccess;
  switch (a.L.code) {
    case HYB: return launch_encode_code<HYB>(a, stream);
    case HYB1: return launch_encode_code<HYB1>(a, stream);
    case MAD1: return launch_encode_code<MAD1>(a, stream);
    case INST3: return launch_encode_code<INST3>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qdec
