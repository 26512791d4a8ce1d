// qdec_gemv kernels for half-TCQ HYB layers (V = 2) at one batch column:
// both row parts in one launch, for the width pairs one half-bit apart.
#include "gemv_impl.hpp"

namespace qdec {
hipError_t launch_gemv_hyb_two_parts(const GemvArgs& a, int kvb, hipStream_t stream) {
  return launch_gemv_two_parts<HYB>(a, kvb, stream);
}
}  // namespace qdec
