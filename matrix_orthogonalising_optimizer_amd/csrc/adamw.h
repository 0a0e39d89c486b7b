// Launch interface of the fused AdamW kernel (adamw.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace dmuon {

// Fused AdamW step over up to kMaxTab tensors (adamw.hip): parameters and
// gradients of element size esize (2: bf16, 4: f32), fp32 moments m and v,
// all updated in place.  Block b works on tensor i with blk0[i] <= b <
// blk0[i + 1], elements [(b - blk0[i]) kAdamChunk, + kAdamChunk).  Bit i of
// vec_mask: tensor i's four pointers are 16-byte aligned.
constexpr int64_t kAdamChunk = 8192;
struct AdamwArgs {
  uint64_t w[kMaxTab];
  uint64_t g[kMaxTab];
  uint64_t m[kMaxTab];
  uint64_t v[kMaxTab];
  int64_t numel[kMaxTab];
  int64_t blk0[kMaxTab + 1];
  uint64_t vec_mask;
  int32_t ntens;
  int32_t esize;
  float beta1, beta2;
  float omb1, omb2;       // 1 - beta1, 1 - beta2
  float eps;
  float decay;            // 1 - lr wd
  float step_size;        // lr / (1 - beta1^t)
  float inv_sqrt_bc2;     // 1 / sqrt(1 - beta2^t)
};
hipError_t launch_adamw(const AdamwArgs& args, hipStream_t stream, const char** name = nullptr);

}  // namespace dmuon
