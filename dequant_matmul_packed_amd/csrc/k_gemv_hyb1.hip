// qdec_gemv kernels for HYB with a one-dimensional codebook (V = 1; k = 2, 3,
// 4; batch tiles 1, 2, 4, 8).
#include "gemv_impl.hpp"

namespace qdec {
hipError_t launch_gemv_hyb1(const GemvArgs& a, hipStream_t stream) {
  return launch_gemv_code<HYB1>(a, stream);
}
}  // namespace qdec
