// Instantiations of the grouped product kernel for f16 MFMA operands.
#include "gemm_impl.h"

namespace dmuon {
hipError_t launch_gemm_f16(GemmKind kind, int tile, const GemmArgs& a, hipStream_t st, const char** name) {
  return launch_tile<f16, f16, bf16_t, true>(tile, kind, a, st, name);
}
}  // namespace dmuon
