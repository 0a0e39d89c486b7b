// Instantiations of the grouped product kernel for bf16 MFMA operands.
#include "gemm_impl.h"

namespace dmuon {
hipError_t launch_gemm_bf16(GemmKind kind, int tile, const GemmArgs& a, hipStream_t st, const char** name) {
  return launch_tile<bf16_t, bf16_t, bf16_t, true>(tile, kind, a, st, name);
}
}  // namespace dmuon
