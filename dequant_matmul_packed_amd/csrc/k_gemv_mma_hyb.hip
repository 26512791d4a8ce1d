// The one-column MFMA GEMV for the HYB code at V = 2 (kV = 4 .. 8).
#include "gemv_mma.hpp"

namespace qdec {
hipError_t launch_gemv_mma_hyb(const MmaArgs& a, int kv, hipStream_t stream) {
  return launch_gemv_mma_code<HYB>(a, kv, stream);
}
}  // namespace qdec
