// The one-column MFMA GEMV for the codes other than HYB at V = 2.
#include "gemv_mma.hpp"

namespace qdec {
hipError_t launch_gemv_mma_other(const MmaArgs& a, int code, int kv, hipStream_t stream) {
  switch (code) {
    case MAD1: return launch_gemv_mma_code<MAD1>(a, kv, stream);
    case INST3: return launch_gemv_mma_code<INST3>(a, kv, stream);
    case NUQ: return launch_gemv_mma_code<NUQ>(a, kv, stream);
    case VQ: return launch_gemv_mma_code<VQ>(a, kv, stream);
    case HYB1: return launch_gemv_mma_code<HYB1>(a, kv, stream);
    case LUT: return launch_gemv_mma_code<LUT>(a, kv, stream);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace qdec
