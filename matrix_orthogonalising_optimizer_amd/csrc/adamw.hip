// Fused AdamW step: the element-wise optimizer DMuon is measured against
// (gist.science technical summary, section 4: DMuon's per-step cost is
// compared with AdamW's).  Adam with decoupled weight decay and
// bias-corrected moments, per element:
//   m <- beta1 m + (1 - beta1) g
//   v <- beta2 v + (1 - beta2) g^2
//   W <- W (1 - lr wd) - (lr / (1 - beta1^t)) m / (sqrt(v) / sqrt(1 - beta2^t) + eps)
// One pass over HBM: W, g, m and v are read once and W, m and v written once
// (22 bytes per element for bf16 parameters, 28 for fp32).  Arithmetic in
// fp32; bf16 results are rounded to nearest even.
//
// A launch takes up to kMaxTab tensors.  Block b belongs to the tensor i with
// blk0[i] <= b < blk0[i + 1] and covers elements [(b - blk0[i]) * kAdamChunk,
// + kAdamChunk) of it: each of its 256 threads handles 8 consecutive elements
// per iteration (16-byte accesses of W and g when bf16, two of m and v), so
// a wave reads and writes whole contiguous lines.

#include "adamw.h"
#include "gemm_impl.h"

namespace dmuon {
namespace {

typedef __attribute__((address_space(1))) u32x4 gvec;

__device__ __forceinline__ void adam_elem(float& w, float g, float& m, float& v, const AdamwArgs& a) {
  m = fmaf(a.beta1, m, a.omb1 * g);
  v = fmaf(a.beta2, v, a.omb2 * (g * g));
  const float denom = fmaf(sqrtf(v), a.inv_sqrt_bc2, a.eps);
  w = fmaf(a.decay, w, -a.step_size * (m / denom));
}

template <int ESIZE>
__global__ void __launch_bounds__(256) adamw_kernel(const AdamwArgs a) {
  // tensor of this block (at most kMaxTab entries: a linear scan)
  int t = 0;
  while (t + 1 < a.ntens && (int64_t)blockIdx.x >= a.blk0[t + 1]) ++t;
  const int64_t n = a.numel[t];
  const int64_t e0 = ((int64_t)blockIdx.x - a.blk0[t]) * kAdamChunk;
  const int64_t e1 = e0 + kAdamChunk < n ? e0 + kAdamChunk : n;
  char* wp = reinterpret_cast<char*>(a.w[t]);
  const char* gp = reinterpret_cast<const char*>(a.g[t]);
  float* mp = reinterpret_cast<float*>(a.m[t]);
  float* vp = reinterpret_cast<float*>(a.v[t]);
  const bool vec = (a.vec_mask >> t) & 1ull;
  int64_t e = e0 + (int64_t)threadIdx.x * 8;
  if (vec) {
    for (; e + 8 <= e1; e += 256 * 8) {
      u32x4 w8[ESIZE / 2], g8[ESIZE / 2];
#pragma unroll
      for (int h = 0; h < ESIZE / 2; ++h) {
        w8[h] = *(const gvec*)(wp + e * ESIZE + 16 * h);
        g8[h] = *(const gvec*)(gp + e * ESIZE + 16 * h);
      }
      const u32x4 m0 = *(const gvec*)(mp + e), m1 = *(const gvec*)(mp + e + 4);
      const u32x4 v0 = *(const gvec*)(vp + e), v1 = *(const gvec*)(vp + e + 4);
      float w[8], g[8], m[8], v[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        m[k] = __uint_as_float(m0[k]);
        m[k + 4] = __uint_as_float(m1[k]);
        v[k] = __uint_as_float(v0[k]);
        v[k + 4] = __uint_as_float(v1[k]);
      }
      if constexpr (ESIZE == 2) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          w[2 * k] = __uint_as_float(w8[0][k] << 16);
          w[2 * k + 1] = __uint_as_float(w8[0][k] & 0xffff0000u);
          g[2 * k] = __uint_as_float(g8[0][k] << 16);
          g[2 * k + 1] = __uint_as_float(g8[0][k] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          w[k] = __uint_as_float(w8[0][k]);
          w[k + 4] = __uint_as_float(w8[1][k]);
          g[k] = __uint_as_float(g8[0][k]);
          g[k + 4] = __uint_as_float(g8[1][k]);
        }
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) adam_elem(w[k], g[k], m[k], v[k], a);
      u32x4 mo0, mo1, vo0, vo1;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        mo0[k] = __float_as_uint(m[k]);
        mo1[k] = __float_as_uint(m[k + 4]);
        vo0[k] = __float_as_uint(v[k]);
        vo1[k] = __float_as_uint(v[k + 4]);
      }
      *(gvec*)(mp + e) = mo0;
      *(gvec*)(mp + e + 4) = mo1;
      *(gvec*)(vp + e) = vo0;
      *(gvec*)(vp + e + 4) = vo1;
      if constexpr (ESIZE == 2) {
        u32x4 o;
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = pack_bf16(w[2 * k], w[2 * k + 1]);
        *(gvec*)(wp + e * 2) = o;
      } else {
        u32x4 o0, o1;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          o0[k] = __float_as_uint(w[k]);
          o1[k] = __float_as_uint(w[k + 4]);
        }
        *(gvec*)(wp + e * 4) = o0;
        *(gvec*)(wp + e * 4 + 16) = o1;
      }
    }
  }
  // element-wise: unaligned tensors, and the last partial group of 8
  for (; e < e1; e += 256 * 8) {
    const int64_t stop = e + 8 < e1 ? e + 8 : e1;
    for (int64_t i = e; i < stop; ++i) {
      float w, g;
      if constexpr (ESIZE == 2) {
        w = bf16_to_f32(reinterpret_cast<const uint16_t*>(wp)[i]);
        g = bf16_to_f32(reinterpret_cast<const uint16_t*>(gp)[i]);
      } else {
        w = reinterpret_cast<const float*>(wp)[i];
        g = reinterpret_cast<const float*>(gp)[i];
      }
      float m = mp[i], v = vp[i];
      adam_elem(w, g, m, v, a);
      mp[i] = m;
      vp[i] = v;
      if constexpr (ESIZE == 2)
        reinterpret_cast<uint16_t*>(wp)[i] = (uint16_t)f32_to_bf16(w);
      else
        reinterpret_cast<float*>(wp)[i] = w;
    }
  }
}

}  // namespace

hipError_t launch_adamw(const AdamwArgs& a, hipStream_t st, const char** name) {
  if (a.ntens < 1 || a.ntens > kMaxTab) return hipErrorInvalidValue;
  const int64_t blocks = a.blk0[a.ntens];
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (a.esize == 2) {
    if (name) *name = "adamw_kernel<2>";
    hipLaunchKernelGGL(adamw_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, st, a);
  } else if (a.esize == 4) {
    if (name) *name = "adamw_kernel<4>";
    hipLaunchKernelGGL(adamw_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, st, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dmuon
