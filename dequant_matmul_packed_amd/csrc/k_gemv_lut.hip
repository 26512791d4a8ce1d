// qdec_gemv kernels for the pure-lookup code (L = 16, V = 1, a 128 KiB table
// of 2^16 fp16 values in LDS; k = 2, 3, 4; batch tiles 1, 2, 4, 8).
#include "gemv_impl.hpp"

namespace qdec {
hipError_t launch_gemv_lut(const GemvArgs& a, hipStream_t stream) {
  return launch_gemv_code<LUT>(a, stream);
}
}  // namespace qdec
