// Instantiations of the grouped product kernel for f32 MFMA operands.
#include "gemm_impl.h"

namespace dmuon {
hipError_t launch_gemm_f32(GemmKind kind, int tile, const GemmArgs& a, hipStream_t st, const char** name) {
  return launch_tile<float, float, float, false>(tile, kind, a, st, name);
}
}  // namespace dmuon
