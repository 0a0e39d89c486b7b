// Internal launch interface between the host engine (dmuon.cpp) and the HIP
// kernels (gemm_*.hip, elementwise.hip).  Plain structs, passed by value as
// kernel arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dmuon {

// Number of caller pointers a single launch can carry inline in its kernel
// arguments.  Larger groups are split into several launches by the host.
constexpr int kMaxTab = 64;

// Per-matrix scalar slots (floats) written by the finalize kernel.
constexpr int kScalStride = 8;
constexpr int kSlotKappa = 0;   // 1 / (||X||_F + eps)
constexpr int kSlotSX = 1;      // power-of-two input scale for fp16 operands
constexpr int kSlotSyrk = 2;    // scale turning X X^T into the stored Gram state
constexpr int kSlotFinal = 3;   // scale turning Q X~ (X~ = X * input scale) into the result
constexpr int kSlotNorm = 4;    // ||X||_F (float, informational)
constexpr int kSlotSyrkX = 5;   // scale turning X~ X~^T (X~ = X * input scale) into the stored Gram state

enum class Prec : int { F16 = 0, BF16 = 1, F32 = 2 };

// Where operand / output matrix `i` of a problem lives.
//   tab != 0 : the caller pointer GemmArgs::tab[GemmProb::tab0 + i]
//   tab == 0 : base + i * stride (bytes)
// ld is the row pitch in elements.
struct MatRef {
  const void* base;
  int64_t stride;
  int64_t ld;
  int32_t tab;
  int32_t pad_;
};

// Kinds of grouped product.  "KK": both operands are row panels with K
// contiguous; "MM": both are stored with M (N) contiguous; "KM": A has K
// contiguous, B has N contiguous.
enum GemmKind : int {
  // Gram product G = X X^T from the workspace copy of the input (the caller's
  // dtype), lower tiles only, written to both triangles of the m x m state.
  KIND_SYRK_KK = 0,
  KIND_SYRK_MM = 1,
  // Symmetric m x m product of two state matrices, lower tiles, mirrored.
  KIND_SYM_KK = 2,
  // P = c0 I + pc1 D + pc2 (A B^T) (pc1, pc2 per problem), symmetric, lower
  // tiles only; A, B and D are one matrix (the launch checks it).
  KIND_POLY = 3,
  // Full output C = alpha A B^T (final product).
  KIND_OUT_KM = 4,
  KIND_OUT_KK = 5,
  // Full output W = c0 W + c1 alpha A B^T (final product fused with the update).
  KIND_UPD_KM = 6,
  KIND_UPD_KK = 7,
  // Standard-form step (16-bit operands): X' = c0 D + c1 alpha A B^T with
  // A = P' (M x M), B rows = X^T (N x M), D = X (M x N) updated in place and
  // X'^T written to C (N x M).
  KIND_AXPY_KK = 8,
};

// GemmArgs::lower bits.  A symmetric matrix "stored lower" holds only the
// lower triangle of tile x tile blocks (diagonal blocks whole); the upper
// blocks are never written or read.
constexpr int32_t kLowerA = 1;    // operand A is stored lower
constexpr int32_t kLowerB = 2;    // operand B is stored lower
constexpr int32_t kLowerOut = 4;  // a symmetric output is written lower only

// One problem of a launch: `batch` products of one shape.  A launch runs up
// to kMaxProb problems of the same kind (one kernel instance) over one grid,
// so that small groups fill the GPU together.
constexpr int kMaxProb = 4;
struct GemmProb {
  MatRef A, B, C, D;
  int32_t M, N, K;
  int32_t batch;       // matrices
  int32_t tiles;       // tiles per matrix
  int32_t tiles_n;     // tiles along N (full tilings)
  int32_t tab0;        // first GemmArgs::tab entry of this problem's caller pointers
  float alpha;         // factor of the epilogue scale
  float pc1, pc2;      // KIND_POLY: P = c0 I + pc1 D + pc2 (A B^T) (the state scale differs per bucket)
  const float* scal;   // per-matrix scalars of this problem's matrix 0 (kScalStride floats each)
};

struct GemmArgs {
  GemmProb p[kMaxProb];
  int32_t nprob;
  int32_t alpha_slot; // scalar slot of the epilogue scale, -1 for 1.0
  float c0, c1, c2;    // c0: KIND_POLY's diagonal term; c0, c1: the update and AXPY epilogues
  int32_t out_esize;  // caller output element size for full outputs: 2 (bf16) or 4 (f32)
  int32_t lower;      // kLower* bits: operands / output stored as their lower triangle of tiles
  uint64_t tab[kMaxTab];
};

// Launch one grouped GEMM.  `tile` is the square block tile (64, 128, 256).
// `name` (optional) receives the kernel instance as the profiler prints it.
hipError_t launch_gemm(Prec prec, GemmKind kind, int tile, const GemmArgs& args,
                       hipStream_t stream, const char** name = nullptr);

// Sum of squares (fp64 partials) of each input matrix and an optional copy of
// it into the workspace.  Inputs come from `tab` (caller pointers).
struct NormArgs {
  uint64_t tab[kMaxTab];
  char* copy_base;     // nullptr: no copy
  int64_t copy_stride; // bytes
  int64_t elems;       // rows * cols
  int32_t esize;       // input element size: 2 (bf16) or 4 (f32)
  int32_t copy_esize;  // copy element size: esize, or 4 to widen bf16 to f32
  int32_t nblk;        // blocks per matrix
  int32_t vec_ok;      // all pointers 16-byte aligned
  double* partial;     // [matrix][nblk]
};
hipError_t launch_norm_copy(const NormArgs& args, int nmat, hipStream_t stream);

// Muon momentum: buf <- mu buf + g, u <- g + mu buf (or buf), u stored in the
// workspace in the parameter dtype, plus fp64 partial sums of u^2.
struct MomentumArgs {
  uint64_t g[kMaxTab];
  uint64_t buf[kMaxTab];
  char* u_base;
  int64_t u_stride;
  int64_t elems;
  int32_t esize;       // gradient element size: 2 (bf16) or 4 (f32)
  int32_t u_esize;     // stored u element size: 2 (bf16) or 4 (f32)
  int32_t nblk;
  int32_t nesterov;
  int32_t vec_ok;
  float mu;
  double* partial;
};
hipError_t launch_momentum(const MomentumArgs& args, int nmat, hipStream_t stream);

// Per-matrix scalars from the partial sums.
struct FinalizeArgs {
  const double* partial;
  int32_t nblk;
  float* scal;         // [matrix][kScalStride]
  float eps;
  float state_scale;   // fixed power-of-two scale of the fp16 Gram state
  int32_t f16_inputs;  // 1: choose a power-of-two input scale for fp16
};
hipError_t launch_finalize(const FinalizeArgs& args, int nmat, hipStream_t stream);

// Operand copies for 16-bit buckets.  The Gram product reads rows of X
// (m x n) and the final product rows of X^T (n x m); the input pass leaves the
// copy in the caller's layout (X, or X^T for tall matrices), so each matrix
// gets its transpose here.  The transpose is either the same bf16 bits or fp16
// times the matrix's power-of-two input scale; the caller-layout copy can be
// converted to scaled fp16 in place.  2-byte elements throughout.
struct PrepArgs {
  char* src_base;      // caller-layout copy, rows x cols, row pitch cols
  int64_t src_stride;  // bytes per matrix
  char* t_base;        // transposed copy, cols x rows, row pitch t_ld
  int64_t t_stride;
  int64_t t_ld;        // elements
  int32_t rows, cols;
  int32_t t_f16;       // 1: transposed copy as scaled fp16, 0: bf16 bits
  int32_t s_f16;       // 1: convert the caller-layout copy to scaled fp16 in place
  const float* scal;   // per-matrix scalars (input scale in kSlotSX)
};
hipError_t launch_prep(const PrepArgs& args, int nmat, hipStream_t stream);

// Deterministic pseudo-random bf16 values in [-1, 1) (a 32-bit integer hash of
// the element index and the seed), for profiling inputs.
hipError_t launch_fill_bf16(uint16_t* p, int64_t n, uint32_t seed, hipStream_t stream);

// Zero `bytes` bytes at base + i * stride for i < nmat (a kernel, so that a
// captured graph holds no memset node).
hipError_t launch_zero_bytes(char* base, int64_t stride, int64_t bytes, int nmat, hipStream_t stream);

// out = f X (or W = c0 W + c1 f X) with f = scal[slot]: the zero-step output
// (f = kappa, source the input copy) and the standard form's last write
// (f = kappa / input scale, source the fp16 iterate).
struct ScaleOutArgs {
  uint64_t out[kMaxTab];     // caller outputs (or W)
  const char* src_base;      // workspace copy of X / u
  int64_t src_stride;
  int64_t elems;
  int32_t esize;             // workspace copy element size
  int32_t out_esize;         // caller element size
  int32_t update;
  int32_t src_f16;           // 2-byte source holds fp16 (else bf16)
  int32_t slot;              // scalar slot of the factor applied to the source
  const float* scal;
  float c0, c1;
};
hipError_t launch_scale_out(const ScaleOutArgs& args, int nmat, hipStream_t stream);

}  // namespace dmuon

namespace dmuon {
// Per-precision entry points (one translation unit each, built in parallel).
hipError_t launch_gemm_f16(GemmKind kind, int tile, const GemmArgs& a, hipStream_t st, const char** name);
hipError_t launch_gemm_bf16(GemmKind kind, int tile, const GemmArgs& a, hipStream_t st, const char** name);
hipError_t launch_gemm_f32(GemmKind kind, int tile, const GemmArgs& a, hipStream_t st, const char** name);
}  // namespace dmuon
