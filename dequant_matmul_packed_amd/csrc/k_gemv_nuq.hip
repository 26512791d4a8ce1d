// qdec_gemv kernels for the NUQ code (k = 2, 3, 4; batch tiles 1, 2, 4, 8).
#include "gemv_impl.hpp"

namespace qdec {
hipError_t launch_gemv_nuq(const GemvArgs& a, hipStream_t stream) {
  return launch_gemv_code<NUQ>(a, stream);
}
}  // namespace qdec
