// HBM-bound kernels around the products: Frobenius norms (with an optional
// workspace copy), the Muon momentum, the per-matrix scalars and the
// zero-step output.  Reductions are deterministic: fixed per-thread order,
// wavefront shuffles, then a fixed order across waves and blocks.

#include "gemm_impl.h"

namespace dmuon {
namespace {

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Deterministic block sum of a per-thread double (256 threads); result valid in thread 0.
__device__ __forceinline__ double block_sum256(double v) {
  __shared__ double red[4];
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = 0.0;
  if (threadIdx.x == 0) t = (red[0] + red[1]) + (red[2] + red[3]);
  return t;
}

template <int ESIZE>
__device__ __forceinline__ double sumsq_chunk(const u32x4& x) {
  double s = 0.0;
  if constexpr (ESIZE == 2) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = __uint_as_float(x[j] << 16), hi = __uint_as_float(x[j] & 0xffff0000u);
      s += (double)(lo * lo) + (double)(hi * hi);  // squares of bf16 values are exact in fp32
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double f = (double)__uint_as_float(x[j]);
      s += f * f;
    }
  }
  return s;
}

template <int ESIZE>
__device__ __forceinline__ float load_elem(const char* p, int64_t i) {
  if constexpr (ESIZE == 2)
    return bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
  else
    return reinterpret_cast<const float*>(p)[i];
}

template <int ESIZE, int CSIZE>
__global__ void __launch_bounds__(256) norm_copy_kernel(const NormArgs a) {
  const int mat = blockIdx.y;
  const char* src = reinterpret_cast<const char*>(a.tab[mat]);
  char* dst = a.copy_base ? a.copy_base + (int64_t)mat * a.copy_stride : nullptr;
  const int64_t stride = (int64_t)a.nblk * 256;
  const int64_t first = (int64_t)blockIdx.x * 256 + threadIdx.x;
  double acc = 0.0;
  int64_t done = 0;
  if (a.vec_ok) {
    constexpr int V = 16 / ESIZE;
    const int64_t nvec = a.elems / V;
    for (int64_t v = first; v < nvec; v += stride) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(src + v * 16);
      if (dst) {
        if constexpr (CSIZE == ESIZE) {
          *reinterpret_cast<u32x4*>(dst + v * 16) = x;
        } else {  // bf16 -> f32: eight values, 32 bytes
          u32x4 lo, hi;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            lo[2 * j] = x[j] << 16;
            lo[2 * j + 1] = x[j] & 0xffff0000u;
            hi[2 * j] = x[j + 2] << 16;
            hi[2 * j + 1] = x[j + 2] & 0xffff0000u;
          }
          *reinterpret_cast<u32x4*>(dst + v * 32) = lo;
          *reinterpret_cast<u32x4*>(dst + v * 32 + 16) = hi;
        }
      }
      acc += sumsq_chunk<ESIZE>(x);
    }
    done = nvec * V;
  }
  for (int64_t e = done + first; e < a.elems; e += stride) {
    const float f = load_elem<ESIZE>(src, e);
    if (dst) {
      if constexpr (CSIZE == 2)
        reinterpret_cast<uint16_t*>(dst)[e] = reinterpret_cast<const uint16_t*>(src)[e];
      else
        reinterpret_cast<float*>(dst)[e] = f;
    }
    acc += (double)f * (double)f;
  }
  const double t = block_sum256(acc);
  if (threadIdx.x == 0) a.partial[(int64_t)mat * a.nblk + blockIdx.x] = t;
}

template <int ESIZE, int USIZE>
__global__ void __launch_bounds__(256) momentum_kernel(const MomentumArgs a) {
  const int mat = blockIdx.y;
  const char* g = reinterpret_cast<const char*>(a.g[mat]);
  float* buf = reinterpret_cast<float*>(a.buf[mat]);
  char* u = a.u_base + (int64_t)mat * a.u_stride;
  const int64_t stride = (int64_t)a.nblk * 256;
  const int64_t first = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const float mu = a.mu;
  double acc = 0.0;
  int64_t done = 0;
  if (a.vec_ok) {
    // eight elements per step: 32 bytes of momentum, 16 or 32 bytes of g and u
    // (every access a whole 16-byte vector)
    const int64_t no = a.elems / 8;
    for (int64_t q = first; q < no; q += stride) {
      float gv[8];
      if constexpr (ESIZE == 2) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(g + q * 16);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          gv[2 * j] = __uint_as_float(w[j] << 16);
          gv[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
        }
      } else {
        const u32x4 w0 = *reinterpret_cast<const u32x4*>(g + q * 32);
        const u32x4 w1 = *reinterpret_cast<const u32x4*>(g + q * 32 + 16);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          gv[j] = __uint_as_float(w0[j]);
          gv[j + 4] = __uint_as_float(w1[j]);
        }
      }
      u32x4 bw0 = *reinterpret_cast<const u32x4*>(buf + q * 8);
      u32x4 bw1 = *reinterpret_cast<const u32x4*>(buf + q * 8 + 4);
      float uv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float bo = __uint_as_float(j < 4 ? bw0[j] : bw1[j - 4]);
        const float bn = fmaf(mu, bo, gv[j]);
        if (j < 4)
          bw0[j] = __float_as_uint(bn);
        else
          bw1[j - 4] = __float_as_uint(bn);
        uv[j] = a.nesterov ? fmaf(mu, bn, gv[j]) : bn;
      }
      *reinterpret_cast<u32x4*>(buf + q * 8) = bw0;
      *reinterpret_cast<u32x4*>(buf + q * 8 + 4) = bw1;
      if constexpr (USIZE == 2) {
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t lo = f32_to_bf16(uv[2 * j]), hi = f32_to_bf16(uv[2 * j + 1]);
          const float rl = bf16_to_f32(lo), rh = bf16_to_f32(hi);
          acc += (double)(rl * rl);
          acc += (double)(rh * rh);
          o[j] = lo | (hi << 16);
        }
        *reinterpret_cast<u32x4*>(u + q * 16) = o;
      } else {
        u32x4 o0, o1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          o0[j] = __float_as_uint(uv[j]);
          o1[j] = __float_as_uint(uv[j + 4]);
          acc += (double)uv[j] * (double)uv[j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) acc += (double)uv[j + 4] * (double)uv[j + 4];
        *reinterpret_cast<u32x4*>(u + q * 32) = o0;
        *reinterpret_cast<u32x4*>(u + q * 32 + 16) = o1;
      }
    }
    done = no * 8;
  }
  for (int64_t e = done + first; e < a.elems; e += stride) {
    const float gv = load_elem<ESIZE>(g, e);
    const float bn = fmaf(mu, buf[e], gv);
    buf[e] = bn;
    const float uv = a.nesterov ? fmaf(mu, bn, gv) : bn;
    if constexpr (USIZE == 2) {
      const uint32_t h = f32_to_bf16(uv);
      reinterpret_cast<uint16_t*>(u)[e] = (uint16_t)h;
      const float r = bf16_to_f32(h);
      acc += (double)(r * r);
    } else {
      reinterpret_cast<float*>(u)[e] = uv;
      acc += (double)uv * (double)uv;
    }
  }
  const double t = block_sum256(acc);
  if (threadIdx.x == 0) a.partial[(int64_t)mat * a.nblk + blockIdx.x] = t;
}

__global__ void __launch_bounds__(64) finalize_kernel(const FinalizeArgs a) {
  const int mat = blockIdx.x;
  const double* p = a.partial + (int64_t)mat * a.nblk;
  double s = 0.0;
  for (int i = threadIdx.x; i < a.nblk; i += 64) s += p[i];
  s = wave_sum(s);
  if (threadIdx.x != 0) return;
  const double nrm = sqrt(s);
  const double kappa = 1.0 / (nrm + (double)a.eps);
  int e = 0;
  if (a.f16_inputs && nrm > 0.0 && nrm <= 1.0e300) {
    int q;
    frexp(nrm, &q);  // nrm < 2^q, nrm >= 2^(q-1)
    e = 14 - q;      // 2^e nrm in [2^13, 2^14): every scaled entry fits fp16
    e = e < -120 ? -120 : (e > 120 ? 120 : e);
  }
  const double sx = ldexp(1.0, e);
  float* o = a.scal + (int64_t)mat * kScalStride;
  o[kSlotKappa] = (float)kappa;
  o[kSlotSX] = (float)sx;
  o[kSlotSyrk] = (float)((double)a.state_scale * kappa * kappa);
  o[kSlotFinal] = (float)(kappa / sx);
  o[kSlotNorm] = (float)nrm;
  o[kSlotSyrkX] = (float)((double)a.state_scale * kappa * kappa / (sx * sx));
}

// Transposed (and optionally converted) operand copies.  A wave owns a 64 x 64
// tile as 8 x 8 blocks, lane l taking block row l / 8 and block column l % 8:
// for each of its 8 source rows the wave reads 8 rows x 128 contiguous bytes,
// transposes the block in registers and writes 8 transposed rows x 128
// contiguous bytes.  A workgroup covers 64 rows x 256 columns.
__global__ void __launch_bounds__(256) prep_kernel(const PrepArgs a) {
  const int mat = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r0 = blockIdx.y * 64 + (lane >> 3) * 8;
  const int c0 = blockIdx.x * 256 + wave * 64 + (lane & 7) * 8;
  if (r0 >= a.rows || c0 >= a.cols) return;
  char* src = a.src_base + (int64_t)mat * a.src_stride;
  char* dst = a.t_base + (int64_t)mat * a.t_stride;
  const float s = a.scal[mat * kScalStride + kSlotSX];
  const bool full = r0 + 8 <= a.rows && c0 + 8 <= a.cols && (a.cols % 8) == 0 && (a.t_ld % 8) == 0;
  if (full) {
    u32x4 x[8], y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = *reinterpret_cast<const u32x4*>(src + ((int64_t)(r0 + e) * a.cols + c0) * 2);
    transpose_block<2>(x, y);
    if (a.t_f16) {
#pragma unroll
      for (int e = 0; e < 8; ++e) cvt_chunk(y[e], s);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) *reinterpret_cast<u32x4*>(dst + ((int64_t)(c0 + e) * a.t_ld + r0) * 2) = y[e];
    if (a.s_f16) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        cvt_chunk(x[e], s);
        *reinterpret_cast<u32x4*>(src + ((int64_t)(r0 + e) * a.cols + c0) * 2) = x[e];
      }
    }
    return;
  }
  uint16_t* s16 = reinterpret_cast<uint16_t*>(src);
  uint16_t* d16 = reinterpret_cast<uint16_t*>(dst);
  for (int e = 0; e < 8 && r0 + e < a.rows; ++e) {
    for (int k = 0; k < 8 && c0 + k < a.cols; ++k) {
      const int64_t si = (int64_t)(r0 + e) * a.cols + c0 + k;
      const uint32_t b = s16[si];
      const uint32_t h = f32_to_f16(bf16_to_f32(b) * s);
      d16[(int64_t)(c0 + k) * a.t_ld + r0 + e] = (uint16_t)(a.t_f16 ? h : b);
      if (a.s_f16) s16[si] = (uint16_t)h;
    }
  }
}

__global__ void __launch_bounds__(256) fill_bf16_kernel(uint16_t* p, int64_t n, uint32_t seed) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
    uint32_t h = (uint32_t)i * 0x9E3779B1u ^ (uint32_t)(i >> 32) ^ seed;
    h ^= h >> 16;
    h *= 0x7FEB352Du;
    h ^= h >> 15;
    h *= 0x846CA68Bu;
    h ^= h >> 16;
    const float u = (float)(h >> 8) * (1.0f / 8388608.0f) - 1.0f;  // [-1, 1)
    p[i] = (uint16_t)f32_to_bf16(u);
  }
}

__global__ void __launch_bounds__(256) zero_bytes_kernel(char* base, int64_t stride, int64_t bytes) {
  char* p = base + (int64_t)blockIdx.y * stride;
  const int64_t step = (int64_t)gridDim.x * 256;
  const int64_t first = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int64_t done = 0;
  if (((uintptr_t)p & 15) == 0) {
    const int64_t nv = bytes / 16;
    for (int64_t v = first; v < nv; v += step) reinterpret_cast<u32x4*>(p)[v] = u32x4{0u, 0u, 0u, 0u};
    done = nv * 16;
  }
  for (int64_t b = done + first; b < bytes; b += step) p[b] = 0;
}

template <int ESIZE, int OSIZE>
__global__ void __launch_bounds__(256) scale_out_kernel(const ScaleOutArgs a) {
  const int mat = blockIdx.y;
  const char* src = a.src_base + (int64_t)mat * a.src_stride;
  char* out = reinterpret_cast<char*>(a.out[mat]);
  const float f = a.scal[mat * kScalStride + a.slot];
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < a.elems; e += stride) {
    float s;
    if constexpr (ESIZE == 2)
      s = a.src_f16 ? f16_to_f32(reinterpret_cast<const uint16_t*>(src)[e]) : load_elem<2>(src, e);
    else
      s = load_elem<ESIZE>(src, e);
    const float x = f * s;
    float v = x;
    if (a.update) v = fmaf(a.c0, load_elem<OSIZE>(out, e), a.c1 * x);
    if constexpr (OSIZE == 2)
      reinterpret_cast<uint16_t*>(out)[e] = (uint16_t)f32_to_bf16(v);
    else
      reinterpret_cast<float*>(out)[e] = v;
  }
}

}  // namespace

hipError_t launch_gemm(Prec prec, GemmKind kind, int tile, const GemmArgs& a, hipStream_t st, const char** name) {
  switch (prec) {
    case Prec::F16: return launch_gemm_f16(kind, tile, a, st, name);
    case Prec::BF16: return launch_gemm_bf16(kind, tile, a, st, name);
    case Prec::F32: return launch_gemm_f32(kind, tile, a, st, name);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_norm_copy(const NormArgs& a, int nmat, hipStream_t st) {
  if (nmat <= 0) return hipSuccess;
  dim3 grid(a.nblk, nmat);
  if (a.esize == 2 && a.copy_esize == 2)
    hipLaunchKernelGGL((norm_copy_kernel<2, 2>), grid, dim3(256), 0, st, a);
  else if (a.esize == 2 && a.copy_esize == 4)
    hipLaunchKernelGGL((norm_copy_kernel<2, 4>), grid, dim3(256), 0, st, a);
  else if (a.esize == 4 && a.copy_esize == 4)
    hipLaunchKernelGGL((norm_copy_kernel<4, 4>), grid, dim3(256), 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_momentum(const MomentumArgs& a, int nmat, hipStream_t st) {
  if (nmat <= 0) return hipSuccess;
  dim3 grid(a.nblk, nmat);
  if (a.esize == 2 && a.u_esize == 2)
    hipLaunchKernelGGL((momentum_kernel<2, 2>), grid, dim3(256), 0, st, a);
  else if (a.esize == 2 && a.u_esize == 4)
    hipLaunchKernelGGL((momentum_kernel<2, 4>), grid, dim3(256), 0, st, a);
  else if (a.esize == 4 && a.u_esize == 4)
    hipLaunchKernelGGL((momentum_kernel<4, 4>), grid, dim3(256), 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_finalize(const FinalizeArgs& a, int nmat, hipStream_t st) {
  if (nmat <= 0) return hipSuccess;
  hipLaunchKernelGGL(finalize_kernel, dim3(nmat), dim3(64), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_prep(const PrepArgs& a, int nmat, hipStream_t st) {
  if (nmat <= 0 || a.rows <= 0 || a.cols <= 0) return hipSuccess;
  if (a.t_ld < a.rows || nmat > 65535) return hipErrorInvalidValue;
  const int64_t gy = ((int64_t)a.rows + 63) / 64;
  if (gy > 65535) return hipErrorInvalidValue;
  dim3 grid((unsigned)((a.cols + 255) / 256), (unsigned)gy, (unsigned)nmat);
  hipLaunchKernelGGL(prep_kernel, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_fill_bf16(uint16_t* p, int64_t n, uint32_t seed, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, n, seed);
  return hipGetLastError();
}

hipError_t launch_zero_bytes(char* base, int64_t stride, int64_t bytes, int nmat, hipStream_t st) {
  if (nmat <= 0 || bytes <= 0) return hipSuccess;
  if (nmat > 65535) return hipErrorInvalidValue;
  int64_t blocks = (bytes / 16 + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(zero_bytes_kernel, dim3((unsigned)blocks, (unsigned)nmat), dim3(256), 0, st, base, stride, bytes);
  return hipGetLastError();
}

hipError_t launch_scale_out(const ScaleOutArgs& a, int nmat, hipStream_t st) {
  if (nmat <= 0) return hipSuccess;
  int64_t blocks = (a.elems + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  dim3 grid((unsigned)blocks, nmat);
  if (a.esize == 2 && a.out_esize == 2)
    hipLaunchKernelGGL((scale_out_kernel<2, 2>), grid, dim3(256), 0, st, a);
  else if (a.esize == 4 && a.out_esize == 2)
    hipLaunchKernelGGL((scale_out_kernel<4, 2>), grid, dim3(256), 0, st, a);
  else if (a.esize == 4 && a.out_esize == 4)
    hipLaunchKernelGGL((scale_out_kernel<4, 4>), grid, dim3(256), 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dmuon
