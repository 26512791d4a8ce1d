// qdec_gemv kernels for the MAD1 code (k = 2, 3, 4; batch tiles 1, 2, 4, 8).
#include "gemv_impl.hpp"

namespace qdec {
hipError_t launch_gemv_mad1(const GemvArgs& a, hipStream_t stream) {
  return launch_gemv_code<MAD1>(a, stream);
}
}  // namespace qdec
