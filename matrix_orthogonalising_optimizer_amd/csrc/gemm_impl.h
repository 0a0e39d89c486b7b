// Grouped symmetric / full NT product kernel for gfx950 (MI355X) MFMA, plus
// the element conversions shared with the elementwise kernels.
//
// The products of the Gram Newton-Schulz recurrence (DMuon, gist.science
// technical summary section 2.2) are all written as C = A B^T with both
// operands read as row panels whose K index is contiguous:
//   * Gram product      G  = X X^T      (A = B = X, K = long side)
//   * symmetric products A A, P A, R P, P Q: every m x m operand is symmetric
//     and stored in full, so its column panel equals its row panel;
//   * final product     Q X (or X Q), one operand read MN-contiguous and
//     transposed in registers on its way to LDS.
// Symmetric outputs are computed on lower-triangle tiles only and stored to
// both triangles, which halves the MFMA work of the dominant products.
//
// Block tile BM x BN (square: 64, 128 or 256), 256 threads = 2 x 2 waves,
// wave tile (BM/2) x (BN/2) built from 32 x 32 MFMA blocks.  Each LDS row holds
// 128 bytes of K (64 fp16/bf16 or 32 fp32 values) as eight 16-byte chunks,
// XOR-swizzled by row so that the MFMA fragment reads, the row-wise writes and
// the transposed writes are all spread over the banks.  Two LDS stages; the
// next K slice is fetched from global memory into registers while the current
// one feeds the MFMAs.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace dmuon {
namespace {

typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct bf16_t {  // storage tag for bfloat16
  uint16_t x;
};

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);                       // round to nearest even
  return u >> 16;
}
__device__ __forceinline__ uint32_t f32_to_f16(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (f16)f);
}
__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(f16, (uint16_t)bits16);
}

template <class E>
struct Elt;
template <>
struct Elt<f16> {
  static constexpr int kSize = 2;
  __device__ static uint32_t enc(float f) { return f32_to_f16(f); }
  __device__ static float dec(uint32_t b) { return f16_to_f32(b); }
};
template <>
struct Elt<bf16_t> {
  static constexpr int kSize = 2;
  __device__ static uint32_t enc(float f) { return f32_to_bf16(f); }
  __device__ static float dec(uint32_t b) { return bf16_to_f32(b); }
};
template <>
struct Elt<float> {
  static constexpr int kSize = 4;
};

// ---------------------------------------------------------------- MFMA
template <class E>
struct Mfma;
template <>
struct Mfma<f16> {
  __device__ static void run(const u32x4& a, const u32x4& b, f32x16& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                               __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};
template <>
struct Mfma<bf16_t> {
  __device__ static void run(const u32x4& a, const u32x4& b, f32x16& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
template <>
struct Mfma<float> {
  // A 16-byte chunk holds four K values; each feeds one K=2 MFMA whose second K
  // index comes from the other half-wave.  The same chunk-to-K assignment is
  // used for both operands, so the sum over all chunks is the full product.
  __device__ static void run(const u32x4& a, const u32x4& b, f32x16& c) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[j]), __uint_as_float(b[j]),
                                               c, 0, 0, 0);
  }
};

// ---------------------------------------------------------------- LDS layout
__device__ __forceinline__ int lds_swz(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int r, int ch) { return (r << 7) + ((ch ^ lds_swz(r)) << 4); }

__device__ __forceinline__ const char* mat_ptr(const MatRef& r, const uint64_t* tab, int var, int mi) {
  if (r.tab) return reinterpret_cast<const char*>(tab[mi]);
  return reinterpret_cast<const char*>(r.base[var]) + (int64_t)mi * r.stride;
}

// bf16 bits -> f16 bits times a power-of-two scale (exact for in-range values).
__device__ __forceinline__ uint32_t cvt_pair_bf16_f16(uint32_t w, float s) {
  float lo = __uint_as_float(w << 16) * s;
  float hi = __uint_as_float(w & 0xffff0000u) * s;
  return f32_to_f16(lo) | (f32_to_f16(hi) << 16);
}
__device__ __forceinline__ void cvt_chunk(u32x4& v, float s) {
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = cvt_pair_bf16_f16(v[j], s);
}

// Element-wise gather of up to VEC values starting at element index `idx` of
// row-contiguous data; missing values are zero.
template <int ESIZE>
__device__ __forceinline__ u32x4 load_chunk_partial(const char* p, int64_t idx, int nvalid) {
  u32x4 v = {0u, 0u, 0u, 0u};
  if constexpr (ESIZE == 2) {
    const uint16_t* q = reinterpret_cast<const uint16_t*>(p) + idx;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (e < nvalid) v[e >> 1] |= (uint32_t)q[e] << (16 * (e & 1));
  } else {
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p) + idx;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (e < nvalid) v[e] = q[e];
  }
  return v;
}

// ---------------------------------------------------------------- tile loaders
// K-contiguous operand: tile rows are source rows, K runs along each row.
template <class E, int ROWS>
struct LoaderK {
  static constexpr int VEC = 16 / Elt<E>::kSize;
  static constexpr int CNT = (ROWS * 8 + 255) / 256;
  u32x4 r[CNT];

  __device__ __forceinline__ void load(const char* p, int64_t ld, int row0, int rows_valid, int k0,
                                       int K, bool vec_ok, int tid) {
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const int L = i * 256 + tid;
      const int row = L >> 3, ch = L & 7;
      const int grow = row0 + row, gk = k0 + ch * VEC;
      if (L < ROWS * 8 && grow < rows_valid && gk < K) {
        const int64_t idx = (int64_t)grow * ld + gk;
        if (vec_ok && gk + VEC <= K)
          r[i] = *reinterpret_cast<const u32x4*>(p + idx * Elt<E>::kSize);
        else
          r[i] = load_chunk_partial<Elt<E>::kSize>(p, idx, K - gk);
      } else {
        r[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  __device__ __forceinline__ void convert(float s) {
#pragma unroll
    for (int i = 0; i < CNT; ++i) cvt_chunk(r[i], s);
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const int L = i * 256 + tid;
      if (L < ROWS * 8) *reinterpret_cast<u32x4*>(lds + lds_off(L >> 3, L & 7)) = r[i];
    }
  }
};

// MN-contiguous operand: the source holds element (row, k) at k * ld + row.
// Each thread reads a VEC x VEC block (VEC K rows of VEC contiguous tile rows)
// and transposes it in registers.
template <class E, int ROWS>
struct LoaderM {
  static constexpr int VEC = 16 / Elt<E>::kSize;
  static constexpr int MB = ROWS / VEC;  // blocks along the tile rows
  static constexpr int NB = MB * 8;      // 8 K-blocks of VEC per 128-byte row
  static constexpr int CNT = (NB + 255) / 256;
  u32x4 r[CNT][VEC];

  __device__ __forceinline__ void load(const char* p, int64_t ld, int row0, int rows_valid, int k0,
                                       int K, bool vec_ok, int tid) {
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const int b = i * 256 + tid;
      const int mb = b % MB, kb = b / MB;
      const int gm = row0 + mb * VEC;
#pragma unroll
      for (int rr = 0; rr < VEC; ++rr) {
        const int gk = k0 + kb * VEC + rr;
        if (b < NB && gk < K && gm < rows_valid) {
          const int64_t idx = (int64_t)gk * ld + gm;
          if (vec_ok && gm + VEC <= rows_valid)
            r[i][rr] = *reinterpret_cast<const u32x4*>(p + idx * Elt<E>::kSize);
          else
            r[i][rr] = load_chunk_partial<Elt<E>::kSize>(p, idx, rows_valid - gm);
        } else {
          r[i][rr] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  }
  __device__ __forceinline__ void convert(float s) {
#pragma unroll
    for (int i = 0; i < CNT; ++i)
#pragma unroll
      for (int rr = 0; rr < VEC; ++rr) cvt_chunk(r[i][rr], s);
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const int b = i * 256 + tid;
      if (b >= NB) continue;
      const int mb = b % MB, kb = b / MB;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        u32x4 o;
        if constexpr (VEC == 8) {
          // o holds K values kb*8 .. kb*8+7 of tile row mb*8+e
          const int w = e >> 1, sh = 16 * (e & 1);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t lo = (r[i][2 * j][w] >> sh) & 0xffffu;
            const uint32_t hi = (r[i][2 * j + 1][w] >> sh) & 0xffffu;
            o[j] = lo | (hi << 16);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) o[j] = r[i][j][e];
        }
        *reinterpret_cast<u32x4*>(lds + lds_off(mb * VEC + e, kb)) = o;
      }
    }
  }
};

template <class E, int ROWS, bool MN>
struct LoaderSel {
  using T = LoaderK<E, ROWS>;
};
template <class E, int ROWS>
struct LoaderSel<E, ROWS, true> {
  using T = LoaderM<E, ROWS>;
};

constexpr int EPI_SYM = 0, EPI_POLY = 1, EPI_OUT = 2, EPI_UPD = 3;

__device__ __forceinline__ void lower_tile(int t, int& ti, int& tj) {
  int i = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  while (i * (i + 1) / 2 > t) --i;
  ti = i;
  tj = t - i * (i + 1) / 2;
}

// Store one value of the symmetric state at (r, c) and (c, r).
template <class E>
__device__ __forceinline__ void store_state(char* C, int64_t ld, int r, int c, float v) {
  if constexpr (Elt<E>::kSize == 2) {
    const uint16_t b = (uint16_t)Elt<E>::enc(v);
    reinterpret_cast<uint16_t*>(C)[(int64_t)r * ld + c] = b;
    if (r != c) reinterpret_cast<uint16_t*>(C)[(int64_t)c * ld + r] = b;
  } else {
    reinterpret_cast<float*>(C)[(int64_t)r * ld + c] = v;
    if (r != c) reinterpret_cast<float*>(C)[(int64_t)c * ld + r] = v;
  }
}

template <class E>
__device__ __forceinline__ float load_state(const char* D, int64_t ld, int r, int c) {
  if constexpr (Elt<E>::kSize == 2)
    return Elt<E>::dec(reinterpret_cast<const uint16_t*>(D)[(int64_t)r * ld + c]);
  else
    return reinterpret_cast<const float*>(D)[(int64_t)r * ld + c];
}

// Caller-facing matrices are bf16 (2 bytes) or f32 (4 bytes).
__device__ __forceinline__ float load_out(const char* p, int64_t i, bool f32) {
  if (f32) return reinterpret_cast<const float*>(p)[i];
  return bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
}
__device__ __forceinline__ void store_out(char* p, int64_t i, float v, bool f32) {
  if (f32)
    reinterpret_cast<float*>(p)[i] = v;
  else
    reinterpret_cast<uint16_t*>(p)[i] = (uint16_t)f32_to_bf16(v);
}

// ---------------------------------------------------------------- GEMM kernel
template <class E, int BT, bool A_MN, bool B_MN, int EPI>
__global__ void __launch_bounds__(256) gemm_kernel(const GemmArgs g) {
  constexpr int BM = BT, BN = BT;
  constexpr int VEC = 16 / Elt<E>::kSize;
  constexpr int BK = 8 * VEC;
  constexpr int WTM = BM / 2, WTN = BN / 2;
  constexpr int MT = WTM / 32, NT = WTN / 32;
  constexpr bool SYM = EPI <= EPI_POLY;
  constexpr int STAGE = (BM + BN) * 128;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // XCD-aware order: consecutive workgroups go round-robin over the 8 XCDs,
  // so give each XCD a contiguous range of logical tiles (shared panels stay
  // in that XCD's L2).
  const int total = g.tiles * g.batch * g.nvar;
  const int per = gridDim.x >> 3;
  const int logical = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (logical >= total) return;
  const int prob = logical / g.tiles;
  const int t = logical - prob * g.tiles;
  const int var = prob / g.batch;
  const int mi = prob - var * g.batch;
  int ti, tj;
  if constexpr (SYM) {
    lower_tile(t, ti, tj);
  } else {
    ti = t / g.tiles_n;
    tj = t - ti * g.tiles_n;
  }
  const int m0 = ti * BM, n0 = tj * BN;

  const char* pa = mat_ptr(g.A, g.tab, var, mi);
  const char* pb = mat_ptr(g.B, g.tab, var, mi);
  const bool va = ((g.A.ld % VEC) == 0) && ((reinterpret_cast<uintptr_t>(pa) & 15) == 0);
  const bool vb = ((g.B.ld % VEC) == 0) && ((reinterpret_cast<uintptr_t>(pb) & 15) == 0);
  float sa = 1.0f, sb = 1.0f;
  if constexpr (Elt<E>::kSize == 2) {
    if (g.conv_a) sa = g.scal[mi * kScalStride + kSlotSX];
    if (g.conv_b) sb = g.scal[mi * kScalStride + kSlotSX];
  }

  typename LoaderSel<E, BM, A_MN>::T la;
  typename LoaderSel<E, BN, B_MN>::T lb;

  f32x16 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = (g.K + BK - 1) / BK;

  auto fetch = [&](int kt) {
    la.load(pa, g.A.ld, m0, g.M, kt * BK, g.K, va, tid);
    lb.load(pb, g.B.ld, n0, g.N, kt * BK, g.K, vb, tid);
  };
  auto stash = [&](int stage) {
    if constexpr (Elt<E>::kSize == 2 && sizeof(E) == 2) {
      if (g.conv_a) la.convert(sa);
      if (g.conv_b) lb.convert(sb);
    }
    char* s = smem + stage * STAGE;
    la.store(s, tid);
    lb.store(s + BM * 128, tid);
  };

  fetch(0);
  stash(0);
  __syncthreads();

  const int arow = wm * WTM + (lane & 31);
  const int brow = wn * WTN + (lane & 31);
  const int half = lane >> 5;

  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) fetch(kt + 1);
    const char* sA = smem + (kt & 1) * STAGE;
    const char* sB = sA + BM * 128;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int ch = 2 * s + half;
      u32x4 fa[MT], fb[NT];
#pragma unroll
      for (int i = 0; i < MT; ++i)
        fa[i] = *reinterpret_cast<const u32x4*>(sA + lds_off(arow + i * 32, ch));
#pragma unroll
      for (int j = 0; j < NT; ++j)
        fb[j] = *reinterpret_cast<const u32x4*>(sB + lds_off(brow + j * 32, ch));
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) Mfma<E>::run(fa[i], fb[j], acc[i][j]);
    }
    if (more) stash((kt + 1) & 1);
    __syncthreads();
  }

  // ------------------------------------------------------------ epilogue
  // 32x32 MFMA result layout: lane l, register r -> row 8*(r/4) + 4*(l/32) + r%4,
  // column l%32.
  const float alpha =
      ((g.alpha_slot >= 0) ? g.scal[mi * kScalStride + g.alpha_slot] : 1.0f) * g.alpha_var[var];
  const int lcol = lane & 31;
  if constexpr (SYM) {
    char* pc = const_cast<char*>(mat_ptr(g.C, g.tab, var, mi));
    const char* pd = (EPI == EPI_POLY) ? mat_ptr(g.D, g.tab, var, mi) : nullptr;
    const bool diag = ti == tj;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int gc = n0 + wn * WTN + j * 32 + lcol;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int gr0 = m0 + wm * WTM + i * 32 + q * 8 + half * 4;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int gr = gr0 + e;
            if (gr >= g.M || gc >= g.N) continue;
            if (diag && gr < gc) continue;
            float v = acc[i][j][q * 4 + e];
            if constexpr (EPI == EPI_POLY) {
              v = g.c2 * v + g.c1 * load_state<E>(pd, g.D.ld, gr, gc);
              if (gr == gc) v += g.c0;
            } else {
              v *= alpha;
            }
            store_state<E>(pc, g.C.ld, gr, gc, v);
          }
        }
      }
  } else {
    const bool of32 = g.out_esize == 4;
    char* pc = const_cast<char*>(mat_ptr(EPI == EPI_UPD ? g.D : g.C, g.tab, var, mi));
    const int64_t ldc = EPI == EPI_UPD ? g.D.ld : g.C.ld;
    const float cA = (EPI == EPI_UPD) ? g.c1 * alpha : alpha;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int gc = n0 + wn * WTN + j * 32 + lcol;
        if (gc >= g.N) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int gr0 = m0 + wm * WTM + i * 32 + q * 8 + half * 4;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int gr = gr0 + e;
            if (gr >= g.M) continue;
            const int64_t idx = (int64_t)gr * ldc + gc;
            float v = cA * acc[i][j][q * 4 + e];
            if constexpr (EPI == EPI_UPD) v = fmaf(g.c0, load_out(pc, idx, of32), v);
            store_out(pc, idx, v, of32);
          }
        }
      }
  }
}

template <class E, int BT>
hipError_t launch_typed(GemmKind kind, const GemmArgs& a, hipStream_t st) {
  const int total = a.tiles * a.batch * a.nvar;
  const int grid = ((total + 7) / 8) * 8;
  if (total <= 0) return hipSuccess;
  switch (kind) {
    case KIND_SYM_KK:
      hipLaunchKernelGGL((gemm_kernel<E, BT, false, false, EPI_SYM>), dim3(grid), dim3(256), 0, st, a);
      break;
    case KIND_SYM_MM:
      hipLaunchKernelGGL((gemm_kernel<E, BT, true, true, EPI_SYM>), dim3(grid), dim3(256), 0, st, a);
      break;
    case KIND_POLY:
      hipLaunchKernelGGL((gemm_kernel<E, BT, false, false, EPI_POLY>), dim3(grid), dim3(256), 0, st, a);
      break;
    case KIND_OUT_KM:
      hipLaunchKernelGGL((gemm_kernel<E, BT, false, true, EPI_OUT>), dim3(grid), dim3(256), 0, st, a);
      break;
    case KIND_UPD_KM:
      hipLaunchKernelGGL((gemm_kernel<E, BT, false, true, EPI_UPD>), dim3(grid), dim3(256), 0, st, a);
      break;
    case KIND_OUT_KK:
      hipLaunchKernelGGL((gemm_kernel<E, BT, false, false, EPI_OUT>), dim3(grid), dim3(256), 0, st, a);
      break;
    case KIND_UPD_KK:
      hipLaunchKernelGGL((gemm_kernel<E, BT, false, false, EPI_UPD>), dim3(grid), dim3(256), 0, st, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class E>
hipError_t launch_tile(int tile, GemmKind kind, const GemmArgs& a, hipStream_t st) {
  switch (tile) {
    case 64: return launch_typed<E, 64>(kind, a, st);
    case 128: return launch_typed<E, 128>(kind, a, st);
    case 256: return launch_typed<E, 256>(kind, a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace
}  // namespace dmuon
