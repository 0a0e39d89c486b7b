// Launch interface of the fused small-matrix kernels (small.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace dmuon {

// Fused Gram Newton-Schulz for short sides up to 128 (small.hip): the Gram
// product, the T recurrence steps and the final product with the states in
// LDS.  Matrices are bf16, rows <= cols (rows = the short side), row pitch
// cols.  X is read from x_base + i * x_stride (the workspace copy of u) or,
// when x_base is null, from tab[i] itself; the result overwrites tab[i]
// (update == 0) or is applied to it as W <- c0 W + c1 O (update == 1).
//
// One launch (SMALL_ONE) runs the whole map with one workgroup per matrix; a
// CU holds one such workgroup (the states take the whole LDS), so a launch
// takes up to kSmallMaxTab matrices and 256 of them fill the GPU.  A small
// batch leaves CUs idle, and the final product (about a quarter of the time)
// is the part that divides: the map then runs as two launches,
//   SMALL_REC   : workgroup i runs the Gram product and the recurrence, then
//                 writes Q's LDS image (rows x 2 rows bytes, rows padded to 64
//                 or 128) and two scalars (the input scale and the output
//                 factor) at split_base + i * split_stride;
//   SMALL_FINAL : workgroup (c, i) computes output columns 128 c .. 128 c +
//                 127 of matrix i from that Q and X, as the one-launch
//                 kernel's final phase does.
// (Splitting the Gram product over workgroups as well was slower: its fp32
// partial products cost more to write and read back than the split saved.)
constexpr int kSmallMaxSteps = 64;
constexpr int kSmallMaxTab = 256;
struct SmallArgs {
  uint64_t tab[kSmallMaxTab];
  const char* x_base;
  int64_t x_stride;           // bytes
  char* split_base;           // split launches: Q image and scalars per matrix
  int64_t split_stride;       // bytes per matrix of that region
  int32_t rows, cols;
  int32_t steps;              // 1 .. kSmallMaxSteps
  int32_t update;
  float a, b1, c2;            // P = a I + b1 A~ + c2 A~^2 (A~ the scaled state)
  float sscale;               // power-of-two scale s of the Gram state A~ = s A
  float eps;                  // kappa = 1 / (||X||_F + eps)
  float ofac;                 // 2^e_T, times the shape factor when updating
  float c0, c1;
  float qmul[kSmallMaxSteps]; // Q_{k+1} = P_k Q_k qmul[k] (stored Q_k = Q_k / 2^e_k)
};
enum SmallLaunch { SMALL_ONE = 0, SMALL_REC = 1, SMALL_FINAL = 2 };

// Bytes per matrix of the split region for short side `rows`: Q's LDS image
// and the two scalars.
int64_t small_split_bytes(int rows);
hipError_t launch_small_ns(const SmallArgs& args, int nmat, SmallLaunch which, hipStream_t stream,
                           const char** name = nullptr);

}  // namespace dmuon
