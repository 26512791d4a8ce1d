// qdec_gemv kernels for the HYB code (k = 2, 3, 4; batch tiles 1, 2, 4, 8).
#include "gemv_impl.hpp"

namespace qdec {
hipError_t launch_gemv_hyb(const GemvArgs& a, hipStream_t stream) {
  return launch_gemv_code<HYB>(a, stream);
}
}  // namespace qdec
