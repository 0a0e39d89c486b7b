// Grouped symmetric / full NT product kernel for gfx950 (MI355X) MFMA, plus
// the element conversions shared with the elementwise kernels.
//
// The products of the Gram Newton-Schulz recurrence (DMuon, gist.science
// technical summary section 2.2) are all written as C = A B^T with both
// operands read as row panels whose K index is contiguous:
//   * Gram product      G  = X X^T      (A = B = X, K = long side)
//   * symmetric products A A, P A, R P, P Q: every m x m operand is
//     symmetric, so its column panel equals its row panel;
//   * final product     Q X (or X Q) against the transposed operand copy the
//     host prepares, optionally fused with the parameter update.
// Symmetric outputs are computed on lower-triangle tiles only, which halves
// the MFMA work of the dominant products.  By default the symmetric states
// are also stored as their lower triangle of tiles only: a row panel is read
// as stored up to the end of its diagonal block and, beyond it, transposed
// from the stored blocks below the diagonal with gfx950's transposing LDS
// reads (ds_read_b64_tr_b16), so no mirrored copy is ever written.
//
// Block tile BT x BT (64, 128 or 256), 256 threads = 2 x 2 waves, wave tile
// (BT/2) x (BT/2) of 32 x 32 MFMA blocks (v_mfma_f32_32x32x16 for 16-bit
// operands, 32x32x2 for fp32); at BT = 256 the fp32 accumulators fill all 256
// AGPRs of every wave (diagonal tiles of symmetric outputs at BT = 256 share
// their 36 lower blocks among the four waves instead: LayTri).  Whole-tile
// launches with 16-byte aligned K-contiguous operands (every 16-bit product)
// load both operands straight into LDS with
// global_load_lds_dwordx4 through a ring of five operand stages (one
// operand's BT rows x 128 bytes of K each, rows XOR-swizzled so that the
// loads, the fragment reads and the transposing reads are spread over the
// banks), one workgroup barrier per 64-deep K step.  Ragged launches and the
// fp32 buckets' N-contiguous operands take a two-stage path instead, through
// registers with bounds checks and zero fill.  Epilogues stage the tile in
// LDS and write 16-byte non-temporal row segments; symmetric tiles are staged
// transposed (four consecutive rows of a column are one LDS write) and
// transposed back in registers, 8 x 8 blocks at a time, on the way out.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <type_traits>

#include "kernels.h"

namespace dmuon {
namespace {

typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((vector_size(8)));

struct bf16_t {  // storage tag for bfloat16
  uint16_t x;
};

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
// Round to nearest even (gfx950 converts in hardware, two values per
// instruction for the packed forms).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t f32_to_f16(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (f16)f);
}
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// lo in bits 0..15, hi in bits 16..31
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, f16x2{(f16)lo, (f16)hi});
}
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)lo, (__bf16)hi});
}
// two state values in one dword (lo in bits 0..15), rounded to nearest even
template <class S>
__device__ __forceinline__ uint32_t pack_state(float lo, float hi);
template <>
__device__ __forceinline__ uint32_t pack_state<f16>(float lo, float hi) { return pack_f16(lo, hi); }
template <>
__device__ __forceinline__ uint32_t pack_state<bf16_t>(float lo, float hi) { return pack_bf16(lo, hi); }
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

__device__ __forceinline__ const char* mat_ptr(const MatRef& r, const uint64_t* tab, int tab0, int mi) {
  if (r.tab) return reinterpret_cast<const char*>(tab[tab0 + mi]);
  return reinterpret_cast<const char*>(r.base) + (int64_t)mi * r.stride;
}

// bf16 bits -> f16 bits times a power-of-two scale (exact for in-range values).
__device__ __forceinline__ uint32_t cvt_pair_bf16_f16(uint32_t w, float s) {
  return pack_f16(__uint_as_float(w << 16) * s, __uint_as_float(w & 0xffff0000u) * s);
}
__device__ __forceinline__ void cvt_chunk(u32x4& v, float s) {
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = cvt_pair_bf16_f16(v[j], s);
}

// Global-memory views.  Kernel pointers arrive through structs, so the
// compiler cannot prove their address space and would emit flat accesses;
// flat loads also count against the LDS counter, which would make every wait
// on an LDS read wait for the prefetch of the next K slice too.
typedef __attribute__((address_space(1))) char gchar;
typedef __attribute__((address_space(1))) const char cgchar;

__device__ __forceinline__ cgchar* gload_ptr(const void* p) { return (cgchar*)p; }
__device__ __forceinline__ gchar* gstore_ptr(void* p) { return (gchar*)p; }

__device__ __forceinline__ u32x4 gload16(cgchar* p) { return *(const __attribute__((address_space(1))) u32x4*)p; }

// Element-wise gather of up to VEC values starting at element index `idx` of
// row-contiguous data; missing values are zero.
template <int ESIZE>
__device__ __forceinline__ u32x4 load_chunk_partial(cgchar* p, int64_t idx, int nvalid) {
  u32x4 v = {0u, 0u, 0u, 0u};
  if constexpr (ESIZE == 2) {
    const __attribute__((address_space(1))) uint16_t* q = (const __attribute__((address_space(1))) uint16_t*)p + idx;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (e < nvalid) v[e >> 1] |= (uint32_t)q[e] << (16 * (e & 1));
  } else {
    const __attribute__((address_space(1))) uint32_t* q = (const __attribute__((address_space(1))) uint32_t*)p + idx;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (e < nvalid) v[e] = q[e];
  }
  return v;
}

// ---------------------------------------------------------------- tile loaders
// EXACT: the launch covers whole tiles in M, N and K with aligned rows, so no
// bounds are checked; otherwise every chunk is checked and ragged chunks are
// gathered element by element with zero fill.

// K-contiguous operand: tile rows are source rows, K runs along each row.
template <class E, int ROWS>
struct LoaderK {
  static constexpr int VEC = 16 / Elt<E>::kSize;
  static constexpr int CNT = (ROWS * 8 + 255) / 256;
  u32x4 r[CNT];

  template <bool EXACT>
  __device__ __forceinline__ void load(cgchar* p, int64_t ld, int row0, int rows_valid, int k0, int K,
                                       bool vec_ok, int tid) {
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const int L = i * 256 + tid;
      const int row = L >> 3, ch = L & 7;
      const int grow = row0 + row, gk = k0 + ch * VEC;
      const int64_t idx = (int64_t)grow * ld + gk;
      if constexpr (EXACT) {
        if ((ROWS * 8) % 256 == 0 || L < ROWS * 8) r[i] = gload16(p + idx * Elt<E>::kSize);
      } else if (L < ROWS * 8 && grow < rows_valid && gk < K) {
        if (vec_ok && gk + VEC <= K)
          r[i] = gload16(p + idx * Elt<E>::kSize);
        else
          r[i] = load_chunk_partial<Elt<E>::kSize>(p, idx, K - gk);
      } else {
        r[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const int L = i * 256 + tid;
      if ((ROWS * 8) % 256 == 0 || L < ROWS * 8) *reinterpret_cast<u32x4*>(lds + lds_off(L >> 3, L & 7)) = r[i];
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

  template <bool EXACT>
  __device__ __forceinline__ void load(cgchar* p, int64_t ld, int row0, int rows_valid, int k0, int K,
                                       bool vec_ok, int tid) {
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const int b = i * 256 + tid;
      const int mb = b % MB, kb = b / MB;
      const int gm = row0 + mb * VEC;
#pragma unroll
      for (int rr = 0; rr < VEC; ++rr) {
        const int gk = k0 + kb * VEC + rr;
        const int64_t idx = (int64_t)gk * ld + gm;
        if constexpr (EXACT) {
          if (NB % 256 == 0 || b < NB) r[i][rr] = gload16(p + idx * Elt<E>::kSize);
        } else if (b < NB && gk < K && gm < rows_valid) {
          if (vec_ok && gm + VEC <= rows_valid)
            r[i][rr] = gload16(p + idx * Elt<E>::kSize);
          else
            r[i][rr] = load_chunk_partial<Elt<E>::kSize>(p, idx, rows_valid - gm);
        } else {
          r[i][rr] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const int b = i * 256 + tid;
      if (NB % 256 != 0 && b >= NB) continue;
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

constexpr int EPI_SYM = 0, EPI_POLY = 1, EPI_OUT = 2, EPI_UPD = 3, EPI_AXPY = 4;

__device__ __forceinline__ void lower_tile(int t, int& ti, int& tj) {
  int i = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  while (i * (i + 1) / 2 > t) --i;
  ti = i;
  tj = t - i * (i + 1) / 2;
}

// Tile orders that keep the tiles running at the same time on one XCD within
// a few operand panels: tiles are visited in SB x SB super-blocks.
constexpr int kSuper = 4;

// Lower triangle of nt x nt tiles: super-block bands top to bottom; in band I
// the off-diagonal super-blocks J < I (row-major inside), then the diagonal
// super-block (lower triangle inside).
__device__ __forceinline__ void lower_tile_blocked(int t, int nt, int& ti, int& tj) {
  const int SB = kSuper;
  int I = 0, start = 0;
  while (true) {
    const int h = min(SB, nt - I * SB);
    const int band = I * h * SB + h * (h + 1) / 2;
    if (t < start + band) break;
    start += band;
    ++I;
  }
  const int h = min(SB, nt - I * SB);
  const int b = t - start;
  if (b < I * h * SB) {
    const int J = b / (h * SB), local = b - J * (h * SB);
    ti = I * SB + local / SB;
    tj = J * SB + local % SB;
  } else {
    int a, c;
    lower_tile(b - I * h * SB, a, c);
    ti = I * SB + a;
    tj = I * SB + c;
  }
}

// Full tm x tn tiling: bands of SB tile rows; in each band, super-blocks of
// SB x 2SB tiles left to right (row-major inside).
__device__ __forceinline__ void full_tile_blocked(int t, int tm, int tn, int& ti, int& tj) {
  const int SBM = kSuper, SBN = 2 * kSuper;
  const int R = t / (SBM * tn);
  const int h = min(SBM, tm - R * SBM);
  const int b = t - R * SBM * tn;
  const int C = b / (h * SBN);
  const int w = min(SBN, tn - C * SBN);
  const int local = b - C * h * SBN;
  ti = R * SBM + local / w;
  tj = C * SBN + local % w;
}

// Store one value of the symmetric state at (r, c) and (c, r).
template <class E>
__device__ __forceinline__ void store_state(gchar* C, int64_t ld, int r, int c, float v) {
  typedef __attribute__((address_space(1))) uint16_t g16;
  typedef __attribute__((address_space(1))) float gf32;
  if constexpr (Elt<E>::kSize == 2) {
    const uint16_t b = (uint16_t)Elt<E>::enc(v);
    ((g16*)C)[(int64_t)r * ld + c] = b;
    if (r != c) ((g16*)C)[(int64_t)c * ld + r] = b;
  } else {
    ((gf32*)C)[(int64_t)r * ld + c] = v;
    if (r != c) ((gf32*)C)[(int64_t)c * ld + r] = v;
  }
}

template <class E>
__device__ __forceinline__ float load_state(cgchar* D, int64_t ld, int r, int c) {
  typedef const __attribute__((address_space(1))) uint16_t g16;
  typedef const __attribute__((address_space(1))) float gf32;
  if constexpr (Elt<E>::kSize == 2)
    return Elt<E>::dec(((g16*)D)[(int64_t)r * ld + c]);
  else
    return ((gf32*)D)[(int64_t)r * ld + c];
}

// Caller-facing matrices are bf16 (2 bytes) or f32 (4 bytes).
__device__ __forceinline__ float load_out(cgchar* p, int64_t i, bool f32) {
  if (f32) return ((const __attribute__((address_space(1))) float*)p)[i];
  return bf16_to_f32(((const __attribute__((address_space(1))) uint16_t*)p)[i]);
}
__device__ __forceinline__ void store_out(gchar* p, int64_t i, float v, bool f32) {
  if (f32)
    ((__attribute__((address_space(1))) float*)p)[i] = v;
  else
    ((__attribute__((address_space(1))) uint16_t*)p)[i] = (uint16_t)f32_to_bf16(v);
}

// ---------------------------------------------------------------- direct loads
// gfx950 loads 16 bytes per lane straight into LDS: lane l of a wave writes
// LDS bytes [base + 16 l, base + 16 l + 16), base uniform over the wave.  One
// instruction therefore fills eight 128-byte LDS rows; lane l fills row
// l / 8, physical chunk l % 8, so it fetches the logical chunk that the
// swizzle maps there.  No registers hold the tile on its way to LDS.
template <class E, int ROWS>
__device__ __forceinline__ void direct_load(cgchar* p, int64_t ld, int row0, int k0, char* lds, int wave,
                                            int lane) {
  constexpr int VEC = 16 / Elt<E>::kSize;
  constexpr int BLOCKS = ROWS / 8;        // 8-row blocks of the operand tile
  constexpr int PER_WAVE = BLOCKS / 4;    // four waves share them
  const int rin = lane >> 3, pc = lane & 7;
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int blk = wave * PER_WAVE + i;
    const int r = blk * 8 + rin;
    const int ch = pc ^ lds_swz(r);
    cgchar* src = p + ((int64_t)(row0 + r) * ld + k0 + ch * VEC) * Elt<E>::kSize;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)(lds + blk * 1024), 16, 0, 0);
  }
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// One direct load for the ring: lane l copies 16 bytes at sbase + voff(l) to
// LDS byte lds + 16 l.  Issued as inline assembly so that the compiler does
// not track it as an LDS write: it would otherwise make every transposing
// LDS read (which it cannot prove disjoint from the buffers being loaded)
// wait for all loads in flight.  Ordering is explicit instead: the ring waits
// on vmcnt for its own loads before each barrier and drains them before the
// epilogue reuses LDS.  m0 is a reserved register, so the compiler ignores
// (and warns about) its clobber below; the generated code of these kernels
// touches m0 only in these loads, each of which sets it.
__device__ __forceinline__ void ring_load(uint64_t sbase, uint32_t voff, uint32_t lds) {
  // lds and sbase are wave-uniform; make that visible so they land in SGPRs
  // (readfirstlane returns int: widen through uint32_t, never sign-extend)
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(sbase >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)sbase);
  const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(__builtin_amdgcn_readfirstlane(lds)),
               "v"(voff), "s"(sb)
               : "memory", "m0");
}

// Workgroup barrier for the direct-load ring: this wave's LDS reads are
// complete, then s_barrier.  Unlike __syncthreads it does not make the wave
// wait for its direct loads still in flight (they are ordered by explicit
// vmcnt waits before it).
__device__ __forceinline__ void ring_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Ring layout for kernels whose two operands both load straight to LDS: LDS
// rows of 64 bytes (half of a 128-byte K slice), four 16-byte chunks per row,
// chunk swizzle ((r >> 2) & 3).  Sixteen consecutive rows read at one logical
// chunk then cover all sixteen 16-byte slots of a 256-byte bank window.
__device__ __forceinline__ int lds_off64(int r, int ch) { return (r << 6) + ((ch ^ ((r >> 2) & 3)) << 4); }

// One direct-load instruction fills 16 rows of 64 bytes; lane l fills row
// l / 4, physical chunk l % 4 and fetches the logical chunk mapped there.
// Instruction i (0 <= i < ROWS / 64) of this wave's share of a ROWS-row tile.
// `base` is wave-uniform (the tile's first row at column k0); the per-lane
// part is a 32-bit byte offset, so the load takes a scalar base and a single
// offset register.
template <class E, int ROWS>
__device__ __forceinline__ void direct_load64_one(cgchar* base, uint32_t ld_bytes, char* lds, int wave, int lane,
                                                  int i) {
  constexpr int VEC = 16 / Elt<E>::kSize;
  constexpr int PER_WAVE = ROWS / 64;
  const int blk = wave * PER_WAVE + i;
  const int r = blk * 16 + (lane >> 2);
  const int ch = (lane & 3) ^ ((r >> 2) & 3);
  const uint32_t off = (uint32_t)r * ld_bytes + (uint32_t)(ch * VEC * Elt<E>::kSize);
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(base + off),
                                   (__attribute__((address_space(3))) void*)(lds + blk * 1024), 16, 0, 0);
}

// ---------------------------------------------------------------- epilogue helpers
// Transpose a VEC x VEC block held as VEC 16-byte rows (x[e] = row e); the
// result y[e] holds column e.
template <int ESZ>
__device__ __forceinline__ void transpose_block(const u32x4* x, u32x4* y) {
  if constexpr (ESZ == 2) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int w = e >> 1, sh = 16 * (e & 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = (x[2 * j][w] >> sh) & 0xffffu;
        const uint32_t hi = (x[2 * j + 1][w] >> sh) & 0xffffu;
        y[e][j] = lo | (hi << 16);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int j = 0; j < 4; ++j) y[e][j] = x[j][e];
  }
}

// Element k (0 <= k < 16 / ESZ) of a 16-byte chunk, as raw bits.
template <int ESZ>
__device__ __forceinline__ uint32_t chunk_elem(const u32x4& v, int k) {
  if constexpr (ESZ == 2) return (v[k >> 1] >> (16 * (k & 1))) & 0xffffu;
  else return v[k];
}

// Store a 16-byte chunk of VEC elements at element index idx of a row with
// `nvalid` valid elements from there; `vec` allows one 16-byte store.
template <int ESZ>
__device__ __forceinline__ void store_chunk(gchar* p, int64_t idx, const u32x4& v, int nvalid, bool vec) {
  constexpr int V = 16 / ESZ;
  if (vec && nvalid >= V) {
    // outputs are consumed by a later launch, not from this L2: stream them
    // so they do not evict operand panels other tiles are still reading
    __builtin_nontemporal_store(v, (__attribute__((address_space(1))) u32x4*)(p + idx * ESZ));
  } else {
#pragma unroll
    for (int k = 0; k < V; ++k) {
      if (k < nvalid) {
        if constexpr (ESZ == 2)
          ((__attribute__((address_space(1))) uint16_t*)p)[idx + k] = (uint16_t)chunk_elem<2>(v, k);
        else
          ((__attribute__((address_space(1))) uint32_t*)p)[idx + k] = v[k];
      }
    }
  }
}

// ---------------------------------------------------------------- MFMA layouts
// The 32 x 32 blocks a wave accumulates over the K loop: job x multiplies A
// fragment ja(x) by B fragment jb(x) into accumulator slot x (acc[x / 4][x %
// 4] at four blocks per wave-tile row).
//
// Every wave of an ordinary tile runs the full MT x NT grid of its quadrant.
// A diagonal tile of a symmetric output at BT = 256 has 36 lower blocks (row
// block >= column block on its 8 x 8 grid) and 28 upper ones, whose values
// the epilogue takes from the lower ones.  There every wave runs the lower
// triangle of a 4 x 4 grid instead (10 jobs from 4 + 4 fragments): A
// fragment i covers tile block row ra0 + d i, B fragment j block row rb0 + d j
// of the B panel (output block column), with (ra0, rb0, d) per wave
//   wave 0: (0, 0, 1)   the upper-left triangle
//   wave 1: (4, 0, 1)   blocks (4 + a, b), a >= b, of the lower-left square
//   wave 2: (7, 3, -1)  blocks (4 + a, b), a <= b, of that square (its four
//                       a == b blocks are wave 1's too, and dropped)
//   wave 3: (4, 4, 1)   the lower-right triangle
// so each wave issues 10 MFMAs per 16-deep K step where the quadrant split
// gives three waves 16 and leaves the fourth nothing to compute.  SAMEB: the
// two operands are one matrix stored one way (the polynomial and Gram
// products), so a diagonal tile's B stages would repeat its A stages (both
// operands switch to transposed reads at the same K step there): B fragments
// are read from the A stages and the B stages are never loaded.
template <int MT_, int NT_>
struct LayQuad {
  static constexpr bool DIAG = false, SAMEB = false;
  static constexpr int NA = MT_, NB = NT_, NJ = MT_ * NT_;
  __device__ static constexpr int ja(int x) { return x / NT_; }
  __device__ static constexpr int jb(int x) { return x % NT_; }
};
template <bool SAME_>
struct LayTri {
  static constexpr bool DIAG = true, SAMEB = SAME_;
  static constexpr int NA = 4, NB = 4, NJ = 10;
  static constexpr int JA[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3}, JB[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};
  __device__ static constexpr int ja(int x) { return JA[x]; }
  __device__ static constexpr int jb(int x) { return JB[x]; }
};

// ---------------------------------------------------------------- GEMM kernel
// E: MFMA operand type; S: type of the symmetric m x m state written by the
// symmetric epilogues (and read by the polynomial epilogue).  A_MN / B_MN:
// the operand is stored with M (N) contiguous and is transposed through
// registers on its way to LDS (fp32 buckets only).  LOW: bit 0 (1) / bit 1
// (2): the A / B operand is a symmetric matrix of which only the lower
// triangle of BT x BT blocks is stored (diagonal blocks whole); its row panel
// is read as stored up to the end of its diagonal block and transposed from
// the blocks below beyond it.
template <class E, class S, int BT, bool A_MN, bool B_MN, int EPI, bool EXACT, int LOW>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, BT >= 256 ? 1 : 4)))
gemm_kernel(const GemmArgs g) {
  constexpr int BM = BT, BN = BT;
  constexpr int VEC = 16 / Elt<E>::kSize;
  constexpr int BK = 8 * VEC;
  constexpr int WTM = BM / 2, WTN = BN / 2;
  constexpr int MT = WTM / 32, NT = WTN / 32;
  constexpr bool SYM = EPI <= EPI_POLY;
  constexpr bool A_DIRECT = EXACT && !A_MN && BM >= 32;
  constexpr bool B_DIRECT = EXACT && !B_MN && BN >= 32;
  constexpr int STAGE = (BM + BN) * 128;
  // epilogue staging: symmetric kinds keep the whole tile in the state type,
  // full kinds stage fp32 rows in one or two passes; rows are padded by 16
  // bytes so the per-lane writes of the MFMA layout avoid bank conflicts
  constexpr int SSZ = Elt<S>::kSize;
  constexpr int PITCH_S = BT * SSZ + 16;
  constexpr int OUT_PASSES = (BT * (BT * 4 + 16) > 160 * 1024 - 16 * 1024) ? 2 : 1;
  constexpr int PITCH_F = BT * 4 + 16;
  constexpr int EPI_BYTES = SYM ? BT * PITCH_S : (BT / OUT_PASSES) * PITCH_F;
  // K-loop buffers: two K slices, or five operand stages for the ring
  constexpr bool DEEP = A_DIRECT && B_DIRECT && BM >= 64 && BN >= 64;
  constexpr int KBYTES = DEEP ? 5 * BM * 128 : 2 * STAGE;
  constexpr int SMEM = (KBYTES > EPI_BYTES) ? KBYTES : EPI_BYTES;
  static_assert(SMEM <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) char smem[SMEM];

  const int tid = threadIdx.x;
  // the wave index is uniform: keeping it in a scalar register makes every
  // LDS stage address of the operand loads scalar arithmetic
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // XCD-aware order: consecutive workgroups go round-robin over the 8 XCDs,
  // so give each XCD a contiguous range of every problem's tiles (shared
  // panels stay in that XCD's L2, and problems of different cost are spread
  // evenly over the XCDs).  Workgroup slot s of XCD x takes, in problem
  // order, tile lo_p + s' of problem p, [lo_p, hi_p) = [n_p x / 8,
  // n_p (x + 1) / 8) of its n_p tiles.
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  int pi = -1, rel = 0;
  for (int q = 0, acc = 0; q < g.nprob; ++q) {
    const int n = g.p[q].tiles * g.p[q].batch;
    const int lo = (int)(((int64_t)n * xcd) >> 3), hi = (int)(((int64_t)n * (xcd + 1)) >> 3);
    if (slot < acc + (hi - lo)) {
      pi = q;
      rel = lo + (slot - acc);
      break;
    }
    acc += hi - lo;
  }
  if (pi < 0) return;
  const GemmProb& P = g.p[pi];
  const int mi = rel / P.tiles;
  const int t = rel - mi * P.tiles;
  int ti, tj;
  if constexpr (SYM) {
    lower_tile_blocked(t, P.tiles_n, ti, tj);
  } else {
    full_tile_blocked(t, P.tiles / P.tiles_n, P.tiles_n, ti, tj);
  }
  if constexpr (LOW != 0 || SYM) {
    // the tile indices come out of float arithmetic: make them scalar so that
    // the K ranges (and the diagonal-tile branch) derived from them stay
    // uniform
    ti = __builtin_amdgcn_readfirstlane(ti);
    tj = __builtin_amdgcn_readfirstlane(tj);
  }
  const int m0 = ti * BM, n0 = tj * BN;
  // diagonal tiles of a symmetric output at BT = 256 (ring path) run the
  // triangle layout (LayTri) in place of the quadrant split: this wave's
  // first block rows and directions (uniform)
  constexpr bool DLAY = DEEP && SYM && MT == 4 && NT == 4;
  const bool dpath = DLAY && ti == tj;
  const int tra0 = wave == 0 ? 0 : (wave == 2 ? 7 : 4), trb0 = wave == 3 ? 4 : (wave == 2 ? 3 : 0);
  const int tdir = wave == 2 ? -1 : 1;  // d

  cgchar* pa = gload_ptr(mat_ptr(P.A, g.tab, P.tab0, mi));
  cgchar* pb = gload_ptr(mat_ptr(P.B, g.tab, P.tab0, mi));
  const bool va = ((P.A.ld % VEC) == 0) && (((uintptr_t)pa & 15) == 0);
  const bool vb = ((P.B.ld % VEC) == 0) && (((uintptr_t)pb & 15) == 0);

  typename LoaderSel<E, BM, A_MN>::T la;
  typename LoaderSel<E, BN, B_MN>::T lb;

  f32x16 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = (P.K + BK - 1) / BK;

  // issue the loads of K slice kt into LDS stage `stage` (direct operands) or
  // into registers (the others)
  auto fetch = [&](int kt, int stage) {
    char* sb = smem + stage * STAGE;
    if constexpr (A_DIRECT)
      direct_load<E, BM>(pa, P.A.ld, m0, kt * BK, sb, wave, lane);
    else
      la.template load<EXACT>(pa, P.A.ld, m0, P.M, kt * BK, P.K, va, tid);
    if constexpr (B_DIRECT)
      direct_load<E, BN>(pb, P.B.ld, n0, kt * BK, sb + BM * 128, wave, lane);
    else
      lb.template load<EXACT>(pb, P.B.ld, n0, P.N, kt * BK, P.K, vb, tid);
  };
  // move register-held operands into LDS stage `stage`
  auto stash = [&](int stage) {
    char* sb = smem + stage * STAGE;
    if constexpr (!A_DIRECT) la.store(sb, tid);
    if constexpr (!B_DIRECT) lb.store(sb + BM * 128, tid);
  };

  const int half = lane >> 5;
  const int lcol_d = lane & 31;
  const int arow_d = wm * WTM + lcol_d;
  const int brow_d = wn * WTN + lcol_d;
  // Polynomial kernels fold the c1 A~ term into the accumulator right after
  // the K loop (A = D = A~ there), from the tile's block of A~ loaded into
  // LDS: acc = A~ A~ + (c1 / c2) A~ and P = c2 acc + c0 I.  Without a square
  // term (c2 = 0) the fold clears the accumulator and adds c1 A~ (P = acc +
  // c0 I), so the epilogue never reads A~.
  constexpr bool FOLD = DEEP && EPI == EPI_POLY && Elt<E>::kSize == 2;
  uint32_t ratio_hi = 0, ratio_lo = 0;
  float fold_scale = 1.0f;
  if constexpr (FOLD) {
    const bool sq = P.pc2 != 0.0f;
    const float ratio = sq ? P.pc1 / P.pc2 : P.pc1;
    fold_scale = sq ? P.pc2 : 1.0f;
    ratio_hi = Elt<E>::enc(ratio);
    ratio_lo = Elt<E>::enc(ratio - Elt<E>::dec(ratio_hi));
  }
  if constexpr (DEEP) {
    // ------------------------------------------------ ring of operand stages
    // An operand stage is one operand's BT rows x 128 bytes of K (64 values),
    // rows laid out and swizzled as in the two-stage path, so that every row
    // request of a load instruction is a whole 128-byte line.  Five stage
    // buffers form a ring: K step j reads operand stages A_j and B_j from
    // buffers (2j) % 5 and (2j + 1) % 5.  The step's four 16-K sub-steps each
    // run the MFMAs of one fragment set interleaved with the LDS reads of the
    // next sub-step's set.  Between sub-steps 2 and 3 each wave waits for its
    // loads of step j + 1, then one barrier: every wave has read all of step
    // j (sub-step 3's fragments were read during sub-step 2), so the two
    // buffers of step j take B_{j+2} (all its loads in sub-step 3) and
    // A_{j+3} (spread over the next three sub-steps).  B operands are
    // therefore fetched one step ahead of use and A operands two.
    //
    // Lower-stored operands (LOW): beyond its diagonal block, an operand
    // stage of row panel p holds the 64 stored rows k of the K step at the
    // panel's BT columns (transposed: 64 rows of 2 BT bytes, 16-byte chunks
    // swizzled by (k & 3) << 2), and each fragment is two transposing LDS
    // reads.  The K loop runs in up to three ranges whose read modes are
    // compile-time: both operands as stored, then B transposed, then both.
    constexpr int NOB = 5;
    constexpr int OB = BM * 128;             // bytes per operand stage
    constexpr int LPO = BM / 32;             // load instructions per wave per operand stage
    // loads of a round per sub-step: B's (needed one step later) all in
    // sub-step 3, right after the barrier that frees their buffer; A's
    // (needed two steps later) spread over sub-steps 0, 1 and 2
    constexpr int LQ3 = LPO, LQ0 = (LPO + 2) / 3, LQ1 = (LPO + 1) / 3, LQ2 = LPO / 3;
    constexpr bool LA = (LOW & 1) != 0, LB = (LOW & 2) != 0;
    constexpr int TCH = BM / 8;              // 16-byte chunks per transposed row
    constexpr int TR = 64 / TCH;             // transposed rows per load instruction
    static_assert(BM == BN && NOB * OB <= SMEM && LQ0 + LQ1 + LQ2 == LPO, "operand-stage ring");
    static_assert(LOW == 0 || (Elt<E>::kSize == 2 && BM >= 128), "lower-stored operands: 16-bit, tiles >= 128");
    const int ns = P.K / BK;
    // first K step whose A (B) panel is read transposed
    const int hA = LA ? min(ns, (ti + 1) * (BM / BK)) : ns;
    const int hB = LB ? min(ns, (tj + 1) * (BN / BK)) : ns;
    cgchar* abase = pa + (int64_t)m0 * P.A.ld * Elt<E>::kSize;
    cgchar* bbase = pb + (int64_t)n0 * P.B.ld * Elt<E>::kSize;
    cgchar* atbase = pa + (int64_t)m0 * Elt<E>::kSize;
    cgchar* btbase = pb + (int64_t)n0 * Elt<E>::kSize;
    const uint32_t alb = (uint32_t)(P.A.ld * Elt<E>::kSize), blb = (uint32_t)(P.B.ld * Elt<E>::kSize);
    // instruction i of this wave for operand stage st of A or B, into buffer
    // `buf`: it fills 1 KB at blk * 1024 (blk = wave * LPO + i).  As stored:
    // rows blk * 8 .. + 7, lane l the physical chunk l % 8 of row
    // blk * 8 + l / 8.  Transposed: stored rows 64 st + blk * TR .. + TR - 1,
    // lane l the physical chunk l % TCH of row blk * TR + l / TCH.
    auto load_x = [&](bool isB, int st, int buf, int i) {
      const int blk = wave * LPO + i;
      const int r = blk * 8 + (lane >> 3);
      const int ch = (lane & 7) ^ lds_swz(r);
      const uint32_t ldb = isB ? blb : alb;
      // stages past the last step (the ring runs two ahead) re-read the last
      // stage into buffers nobody reads: in bounds, still cached, and no
      // per-lane select in the address
      const int sl = st < ns ? st : ns - 1;
      uint32_t off = (uint32_t)r * ldb + (uint32_t)(ch * 16);
      cgchar* src = (isB ? bbase : abase) + (int64_t)sl * 128;
      if constexpr (LOW != 0) {
        const bool tr = sl >= (isB ? hB : hA);
        const int rt = blk * TR + lane / TCH;
        const int ct = (lane % TCH) ^ ((rt & 3) << 2);
        const uint32_t offt = (uint32_t)rt * ldb + (uint32_t)(ct * 16);
        cgchar* srct = (isB ? btbase : atbase) + (int64_t)sl * 64 * ldb;
        off = tr ? offt : off;
        src = tr ? srct : src;
      }
      ring_load((uint64_t)(uintptr_t)src, off,
                (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(smem + buf * OB + blk * 1024));
    };
    // load number q (0 <= q < 2 LPO) of round R, issued after the barrier of
    // step R: B_{R+2} into step R's A buffer, then A_{R+3} into its B buffer
    auto load_round = [&](int R, int bufA_R, int bufB_R, int q) {
      if (q < LPO)
        load_x(true, R + 2, bufA_R, q);
      else
        load_x(false, R + 3, bufB_R, q - LPO);
    };
    u32x4 fa[2][MT], fb[2][NT];
    // fragment rows row0 + [0, 32) (this lane: row0 + lcol_d), K values
    // 16 sub + 8 half + [0, 8) of a transposed stage: in each group of 16
    // lanes, lane 4 q + x supplies K row k0 + q, columns row0 + 16 (group & 1)
    // + 4 x .. + 3, and the read hands lane j of the group the four K values
    // of column row0 + 16 (group & 1) + j
    // byte offset, within a transposed stage at sub-step 0, of this lane's
    // first read of the fragment whose rows start at row0; sub-step s lies
    // 16 s K rows further and the second read 4 K rows further (the chunk
    // swizzle depends on k & 3 only, which neither changes)
    auto tr_off = [&](int row0) -> uint32_t {
      const int grp16 = lane >> 4, lq = lane & 15;
      const int k0 = 8 * (grp16 >> 1) + (lq >> 2);
      const int col = row0 + 16 * (grp16 & 1) + 4 * (lq & 3);
      const int c = (col >> 3) ^ ((k0 & 3) << 2);
      return (uint32_t)(k0 * (2 * BM) + c * 16 + (col & 7) * 2);
    };
    auto rd_t = [&](const char* p) -> u32x4 {
      typedef __attribute__((address_space(3))) v4i16 lds4;
      const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds4*)const_cast<char*>(p)));
      const u32x2 hi =
          __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds4*)const_cast<char*>(p + 8 * BM)));
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };
    // this lane's fragment offsets within a stage buffer, computed once per
    // tile: as-stored stages per sub-step s and fragment parity p (fragment
    // r + 2 lies 64 rows = 8 KB further, where the row swizzle repeats), and
    // transposed stages per fragment at sub-step 0
    //   B's rows are A's moved by (wn - wm) WTM.  In an as-stored stage that
    //   changes no swizzle when WTM is a multiple of 64 (the row swizzle
    //   repeats every 64 rows); in a transposed stage the chunk index moves
    //   by WTM / 8, clear of the two bits (2 and 3) its swizzle flips when WTM
    //   is a multiple of 128.  Then B reads use A's offsets plus a uniform
    //   delta; otherwise B keeps offsets of its own.
    constexpr bool SHS = WTM == WTN && WTM % 64 == 0, SHT = WTM == WTN && WTM % 128 == 0;
    constexpr int NP = MT < 2 ? MT : 2;
    constexpr int NBS = SHS ? 1 : 2, NBT = SHT ? 1 : 2;
    uint32_t so[NBS][4][NP], to[NBT][MT];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        so[0][s][p] = (uint32_t)lds_off(arow_d + 32 * p, 2 * s + half);
        if constexpr (!SHS) so[NBS - 1][s][p] = (uint32_t)lds_off(brow_d + 32 * p, 2 * s + half);
      }
#pragma unroll
    for (int r = 0; r < MT; ++r) {
      to[0][r] = tr_off(wm * WTM + r * 32);
      if constexpr (!SHT) to[NBT - 1][r] = tr_off(wn * WTN + r * 32);
    }
    const int dso = SHS ? (wn - wm) * WTM * 128 : 0, dto = SHT ? (wn - wm) * WTM * 2 : 0;
    // the triangle layout's fragment offsets, per operand o (A, B) and
    // fragment f: as stored per sub-step s, and transposed at sub-step 0
    uint32_t dfo[2][4][4], dtr[2][4];
    if constexpr (DLAY) {
#pragma unroll
      for (int o = 0; o < 2; ++o)
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const int b = (o == 0 ? tra0 : trb0) + tdir * f;
#pragma unroll
          for (int s = 0; s < 4; ++s) dfo[o][s][f] = (uint32_t)lds_off(32 * b + lcol_d, 2 * s + half);
          dtr[o][f] = tr_off(32 * b);
        }
    }
    if constexpr (SYM && !DLAY) {
      // On a diagonal tile of a symmetric output (tiles below 256; at 256 they
      // run the triangle layout) the upper-right wave's
      // quadrant lies wholly above the diagonal, and the epilogue writes the
      // upper blocks of such a tile from the transposes of the lower ones:
      // that wave's products are never used.  It keeps its share of the
      // ring's loads and barriers, but all its lanes read one address
      // (broadcast reads take the LDS from the other waves for a fraction of
      // the cost, and its MFMAs see identical operand rows).
      if (ti == tj && wm == 0 && wn == 1) {
#pragma unroll
        for (int b = 0; b < NBS; ++b)
#pragma unroll
          for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int p = 0; p < NP; ++p) so[b][s][p] = (uint32_t)__builtin_amdgcn_readfirstlane((int)so[b][s][p]);
#pragma unroll
        for (int b = 0; b < NBT; ++b)
#pragma unroll
          for (int r = 0; r < MT; ++r) to[b][r] = (uint32_t)__builtin_amdgcn_readfirstlane((int)to[b][r]);
      }
    }
    // fragment r (A fragments first) of sub-step `sub`; TA / TB: the buffer
    // holds a transposed stage
    auto rd = [&](auto lay, auto ta_t, auto tb_t, int set, int bufA, int bufB, int sub, int r) {
      using L = decltype(lay);
      constexpr bool TA = decltype(ta_t)::value, TB = decltype(tb_t)::value;
      const char* sA = smem + bufA * OB;
      const char* sB = smem + bufB * OB;
      if constexpr (L::DIAG) {
        if (r < L::NA) {
          if constexpr (TA)
            fa[set][r] = rd_t(sA + dtr[0][r] + sub * (32 * BM));
          else
            fa[set][r] = *reinterpret_cast<const u32x4*>(sA + dfo[0][sub][r]);
        } else {
          const int rb = r - L::NA;
          const char* sBd = L::SAMEB ? sA : sB;
          if constexpr (TB)
            fb[set][rb] = rd_t(sBd + dtr[1][rb] + sub * (32 * BM));
          else
            fb[set][rb] = *reinterpret_cast<const u32x4*>(sBd + dfo[1][sub][rb]);
        }
      } else if (r < MT) {
        if constexpr (TA)
          fa[set][r] = rd_t(sA + to[0][r] + sub * (32 * BM));
        else
          fa[set][r] = *reinterpret_cast<const u32x4*>(sA + so[0][sub][r % NP] + (r / NP) * (64 * 128));
      } else {
        const int rb = r - MT;
        if constexpr (TB)
          fb[set][rb] = rd_t(sB + dto + to[NBT - 1][rb] + sub * (32 * BM));
        else
          fb[set][rb] = *reinterpret_cast<const u32x4*>(sB + dso + so[NBS - 1][sub][rb % NP] + (rb / NP) * (64 * 128));
      }
    };
    // sub-step SS of step j: MFMAs from set SS & 1, interleaved with the
    // fragment reads of sub-step rsub from buffers (rA, rB) into the other set
    // and with this sub-step's loads of round R (see LQ*)
    auto phase = [&](auto lay, auto s_t, auto ta_t, auto tb_t, int rA, int rB, int rsub, int R, int lA, int lB) {
      using L = decltype(lay);
      constexpr int NM = L::NJ, NR = L::NA + L::NB, NI = NM < NR ? NM : NR;
      constexpr int SS = decltype(s_t)::value;
      constexpr int SET = SS & 1;
      constexpr int LQ = SS == 3 ? (L::SAMEB ? 0 : LQ3) : SS == 0 ? LQ0 : SS == 1 ? LQ1 : LQ2;
      constexpr int lq0 = SS == 3 ? 0 : SS == 0 ? LPO : SS == 1 ? LPO + LQ0 : LPO + LQ0 + LQ1;
      constexpr int LSTEP = LQ == 0 ? NM + 1 : (NM / LQ > 0 ? NM / LQ : 1);
      constexpr bool TA = decltype(ta_t)::value, TB = decltype(tb_t)::value;
#pragma unroll
      for (int x = 0; x < NM; ++x) {
        Mfma<E>::run(fa[SET][L::ja(x)], fb[SET][L::jb(x)], acc[x / NT][x % NT]);
        if (x < NI) rd(lay, ta_t, tb_t, SET ^ 1, rA, rB, rsub, x);
        if (x % LSTEP == LSTEP - 1 && x / LSTEP < LQ) load_round(R, lA, lB, lq0 + x / LSTEP);
      }
#pragma unroll
      for (int r = NI; r < NR; ++r) rd(lay, ta_t, tb_t, SET ^ 1, rA, rB, rsub, r);
#pragma unroll
      for (int q = NM / LSTEP; q < LQ; ++q) load_round(R, lA, lB, lq0 + q);
      if constexpr (sizeof(E) == 2) {
#pragma unroll
        for (int x = 0; x < NM; ++x) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          if (x < NI) {  // LDS reads of one fragment: two when transposed
            if ((x < L::NA && TA) || (x >= L::NA && TB))
              __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            else
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          if (x % LSTEP == LSTEP - 1 && x / LSTEP < LQ)
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // prologue: A_0, B_0, A_1 and the B part of round -1 (B_1 into buffer
    // 3; its A part, A_2 into buffer 4, follows in step 0)
#pragma unroll
    for (int i = 0; i < LPO; ++i) load_x(false, 0, 0, i);
#pragma unroll
    for (int i = 0; i < LPO; ++i) load_x(true, 0, 1, i);
#pragma unroll
    for (int i = 0; i < LPO; ++i) load_x(false, 1, 2, i);
#pragma unroll
    for (int q = 0; q < LPO; ++q) load_round(-1, 3, 4, q);
    wait_vmcnt<2 * LPO>();  // A_0 and B_0 have landed
    ring_barrier();
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using S3 = std::integral_constant<int, 3>;
    using NO = std::false_type;
    using YES = std::true_type;
    // steps [j0, j1) with both read modes fixed; the step before j0 has made
    // step j0's stages visible.  The last step's sub-step 3 also reads step
    // j1's first fragments in this range's modes; the next range reads them
    // again in its own.
    int ca = 0;  // (2j) % 5: step j's A buffer; its B buffer is the next one
    auto run_range = [&](auto lay, auto ta_t, auto tb_t, int j0, int j1) {
      using L = decltype(lay);
      if (j0 >= j1) return;
#pragma unroll
      for (int r = 0; r < L::NA + L::NB; ++r) rd(lay, ta_t, tb_t, 0, ca, ca == 4 ? 0 : ca + 1, 0, r);
      for (int j = j0; j < j1; ++j) {
        const int cb = ca == 4 ? 0 : ca + 1;       // (2j + 1) % 5
        const int na = cb == 4 ? 0 : cb + 1;       // (2j + 2) % 5: step j + 1
        const int nb = na == 4 ? 0 : na + 1;       // (2j + 3) % 5
        const int pa_ = nb;                         // (2j - 2) % 5: step j - 1's A buffer
        const int pb_ = nb == 4 ? 0 : nb + 1;      // (2j - 1) % 5
        phase(lay, S0{}, ta_t, tb_t, ca, cb, 1, j - 1, pa_, pb_);
        phase(lay, S1{}, ta_t, tb_t, ca, cb, 2, j - 1, pa_, pb_);
        phase(lay, S2{}, ta_t, tb_t, ca, cb, 3, j - 1, pa_, pb_);
        wait_vmcnt<LPO>();  // everything but A_{j+2} has landed: B_{j+1}, A_{j+1}
        ring_barrier();
        phase(lay, S3{}, ta_t, tb_t, na, nb, 0, j, ca, cb);
        ca = na;
      }
    };
    auto run_all = [&](auto lay) {
      if constexpr (LOW == 0) {
        run_range(lay, NO{}, NO{}, 0, ns);
      } else if constexpr (LOW == 1) {
        run_range(lay, NO{}, NO{}, 0, hA);
        run_range(lay, YES{}, NO{}, hA, ns);
      } else if constexpr (LOW == 2) {
        run_range(lay, NO{}, NO{}, 0, hB);
        run_range(lay, NO{}, YES{}, hB, ns);
      } else {
        // lower tiles of a symmetric product: hB <= hA
        run_range(lay, NO{}, NO{}, 0, hB);
        run_range(lay, NO{}, YES{}, hB, hA);
        run_range(lay, YES{}, YES{}, hA, ns);
      }
    };
    if constexpr (DLAY) {
      // one matrix stored one way behind both operands (vmcnt waits stay
      // right without the B loads: each waits for all but the newest
      // stage's loads, and those are A loads).  Polynomial products always
      // square one matrix (launch_one checks); the others are tested here.
      if (dpath) {
        if constexpr (EPI == EPI_POLY) {
          run_all(LayTri<true>{});
        } else {
          if ((LOW == 0 || LOW == 3) && pa == pb && P.A.ld == P.B.ld)
            run_all(LayTri<true>{});
          else
            run_all(LayTri<false>{});
        }
      } else {
        run_all(LayQuad<MT, NT>{});
      }
    } else {
      run_all(LayQuad<MT, NT>{});
    }
    wait_vmem();  // the loads that ran past the end land before LDS is reused
    __syncthreads();
    if constexpr (FOLD) {
      if (P.pc2 == 0.0f) {
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
          for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
      }
      {
        // The polynomial's linear term, acc += rho A~ (rho = c1 / c2, or c1
        // without a square term), once per tile after the K loop.  The
        // tile's block of A~ (rows m0 + [0, BM), columns n0 + [0, BN)) is
        // the A panel's K steps n0 / 64 .. , stored as is (tj <= ti), loaded
        // like ring stages into buffers 0, 1, ...  Each wave reads, as A
        // fragments, the 16-column K sub-steps u that are its own output
        // columns (K offset wn WTN + 16 u in the block, accumulator column
        // block u / 2) and adds them through MFMAs against a scaled
        // identity, the ratio split as hi + lo in the operand type: element
        // t = lcol - 16 (u & 1) - 8 half of a lane's eight K values is the
        // one with k == column.
        static_assert(BN / BK <= NOB && WTN % 32 == 0, "fold block in the ring buffers");
        const int j0 = n0 / BK;
#pragma unroll
        for (int st = 0; st < BN / BK; ++st)
#pragma unroll
          for (int i = 0; i < LPO; ++i) load_x(false, j0 + st, st, i);
        wait_vmem();
        ring_barrier();
        // the identity operand of the 16 accumulator columns 16 uh + [0, 16)
        auto ident = [&](int uh, u32x4& idh, u32x4& idl) {
          const int t = lcol_d - 16 * uh - 8 * half;
          const uint32_t sh = 16u * (uint32_t)(t & 1);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const bool on = (t >> 1) == w;  // t in [0, 8)
            idh[w] = on ? ratio_hi << sh : 0u;
            idl[w] = on ? ratio_lo << sh : 0u;
          }
        };
        // A~ rows row0 + [0, 32) at the block's K columns kq + [0, 16)
        auto fold_rd = [&](int row0, int kq) -> u32x4 {
          const char* sA = smem + (kq / BK) * OB;
          const int ch = 2 * ((kq % BK) / 16) + half;
          return *reinterpret_cast<const u32x4*>(sA + lds_off(row0 + lcol_d, ch));
        };
        if (dpath) {
          // each wave adds the term to the blocks of its triangle layout
          if constexpr (DLAY) {
            u32x4 idh[2], idl[2];
            ident(0, idh[0], idl[0]);
            ident(1, idh[1], idl[1]);
#pragma unroll
            for (int x = 0; x < LayTri<false>::NJ; ++x) {
              const int br = tra0 + tdir * LayTri<false>::ja(x), bc = trb0 + tdir * LayTri<false>::jb(x);
#pragma unroll
              for (int uh = 0; uh < 2; ++uh) {
                const u32x4 a = fold_rd(32 * br, 32 * bc + 16 * uh);
                Mfma<E>::run(a, idh[uh], acc[x / NT][x % NT]);
                Mfma<E>::run(a, idl[uh], acc[x / NT][x % NT]);
              }
            }
          }
        } else if (!(ti == tj && wm == 0 && wn == 1)) {
          // (the upper-right wave of a diagonal tile has no use for the term)
#pragma unroll
          for (int u = 0; u < WTN / 16; ++u) {
            u32x4 idh, idl;
            ident(u & 1, idh, idl);
#pragma unroll
            for (int i = 0; i < MT; ++i) {
              const u32x4 a = fold_rd(arow_d - lcol_d + i * 32, wn * WTN + 16 * u);
              Mfma<E>::run(a, idh, acc[i][u >> 1]);
              Mfma<E>::run(a, idl, acc[i][u >> 1]);
            }
          }
        }
        ring_barrier();  // every wave has read the block before the epilogue stages over it
      }
    }
  } else {
  fetch(0, 0);
  stash(0);
  if constexpr (A_DIRECT || B_DIRECT) wait_vmem();
  __syncthreads();

  const int arow = arow_d;
  const int brow = brow_d;

  // MFMA fragments, double-buffered across the four sub-steps of a K slice
  // (16 deep for 16-bit operands, 32 for fp32): while the MFMAs of sub-step s
  // run, the fragments of sub-step s + 1 are read from LDS.  The source order
  // interleaves one LDS read after each of the first MT + NT MFMAs, and the
  // scheduling barriers keep that order.
  u32x4 fa[2][MT], fb[2][NT];
  auto rdA = [&](int set, const char* sA, int s, int i) {
    fa[set][i] = *reinterpret_cast<const u32x4*>(sA + lds_off(arow + i * 32, 2 * s + half));
  };
  auto rdB = [&](int set, const char* sB, int s, int j) {
    fb[set][j] = *reinterpret_cast<const u32x4*>(sB + lds_off(brow + j * 32, 2 * s + half));
  };

  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) fetch(kt + 1, (kt + 1) & 1);
    const char* sA = smem + (kt & 1) * STAGE;
    const char* sB = sA + BM * 128;
#pragma unroll
    for (int i = 0; i < MT; ++i) rdA(0, sA, 0, i);
#pragma unroll
    for (int j = 0; j < NT; ++j) rdB(0, sB, 0, j);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int cur = s & 1, nxt = cur ^ 1;
      // read r of the next sub-step: A fragments first, then B fragments
      auto rd = [&](int r) {
        if (r < MT)
          rdA(nxt, sA, s + 1, r);
        else
          rdB(nxt, sB, s + 1, r - MT);
      };
      constexpr int NM = MT * NT, NR = MT + NT, NI = NM < NR ? NM : NR;
#pragma unroll
      for (int x = 0; x < NM; ++x) {
        const int i = x / NT, j = x % NT;
        Mfma<E>::run(fa[cur][i], fb[cur][j], acc[i][j]);
        if (s < 3 && x < NI) rd(x);
      }
      if (s < 3) {
#pragma unroll
        for (int r = NI; r < NR; ++r) rd(r);
      }
      if constexpr (sizeof(E) == 2) {
        if (s < 3) {
#pragma unroll
          for (int r = 0; r < NI; ++r) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
          }
          if constexpr (NM > NI) __builtin_amdgcn_sched_group_barrier(0x008, NM - NI, 0);
          if constexpr (NR > NI) __builtin_amdgcn_sched_group_barrier(0x100, NR - NI, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (more) stash((kt + 1) & 1);
    if constexpr (A_DIRECT || B_DIRECT) wait_vmem();
    __syncthreads();
  }
  }  // !DEEP

  // ------------------------------------------------------------ epilogue
  // 32x32 MFMA result layout: lane l, register r -> row 8*(r/4) + 4*(l/32) + r%4,
  // column l%32.  Results are staged in LDS (the K-loop stages are free after
  // the final barrier) and written with 16-byte row-contiguous stores.
  const float alpha =
      ((g.alpha_slot >= 0) ? P.scal[mi * kScalStride + g.alpha_slot] : 1.0f) * P.alpha;
  const int lcol = lane & 31;
  if constexpr (SYM) {
    constexpr int V = 16 / SSZ;      // elements per 16-byte chunk
    constexpr int NBC = BT / V;      // V x V blocks per tile side
    gchar* pc = gstore_ptr(const_cast<char*>(mat_ptr(P.C, g.tab, P.tab0, mi)));
    cgchar* pd = gload_ptr((EPI == EPI_POLY) ? mat_ptr(P.D, g.tab, P.tab0, mi) : nullptr);
    const bool diag = ti == tj;
    // Stage the tile (after the polynomial or the scale) transposed, in the
    // state type: staging row c holds tile column c.  The four consecutive
    // rows a lane holds of one column are then one 4 SSZ-byte LDS write.
    // The 16-byte chunks of staging row c are swizzled by (c >> 3) & 15: the
    // write-out reads chunk rb of the rows 8 cb + e for consecutive cb, which
    // lie 32 banks apart and would otherwise meet in two bank groups.
    const bool on_diag = diag && wm == wn;
    constexpr int SWM = (BT * SSZ / 16 < 16 ? BT * SSZ / 16 : 16) - 1;
    auto stage_swz = [](int row) { return (row >> 3) & SWM; };
    // one accumulator block at tile rows r0 + [0, 32), columns c0 + [0, 32);
    // dblk: it lies on the tile's diagonal
    auto stage_blk = [&](const f32x16& a, int r0, int c0, bool dblk) {
      const int c = c0 + lcol;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = r0 + q * 8 + half * 4;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = a[q * 4 + e];
          if constexpr (EPI == EPI_POLY) {
            const int gr = m0 + r + e, gc = n0 + c;
            if constexpr (FOLD) {
              v[e] = fold_scale * v[e];
            } else {
              const bool in = EXACT || (gr < P.M && gc < P.N);
              v[e] = P.pc2 * v[e] + (in ? P.pc1 * load_state<S>(pd, P.D.ld, gr, gc) : 0.0f);
            }
            // c0 I: only diagonal blocks of a diagonal tile hold diagonal
            // elements (elsewhere rows and columns differ by at least 32)
            if (dblk && r + e == c) v[e] += g.c0;
          } else {
            v[e] *= alpha;
          }
        }
        char* dst = smem + c * PITCH_S + (((r * SSZ) >> 4) ^ stage_swz(c)) * 16 + ((r * SSZ) & 15);
        if constexpr (SSZ == 2) {
          u32x2 w;
          w[0] = pack_state<S>(v[0], v[1]);
          w[1] = pack_state<S>(v[2], v[3]);
          *reinterpret_cast<u32x2*>(dst) = w;
        } else {
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = __float_as_uint(v[e]);
          *reinterpret_cast<u32x4*>(dst) = w;
        }
      }
    };
    if (dpath) {
      if constexpr (DLAY) {
#pragma unroll
        for (int x = 0; x < LayTri<false>::NJ; ++x) {
          const int i = LayTri<false>::ja(x), j = LayTri<false>::jb(x);
          // wave 2's a == b blocks are wave 1's too
          if (wave == 2 && i == j) continue;
          const int br = tra0 + tdir * i, bc = trb0 + tdir * j;
          stage_blk(acc[x / NT][x % NT], 32 * br, 32 * bc, br == bc);
        }
      }
    } else if (!(diag && wm == 0 && wn == 1)) {
      // the upper-right wave of a diagonal tile stages nothing: its quadrant
      // is above the diagonal and never read back
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
          stage_blk(acc[i][j], wm * WTM + i * 32, wn * WTN + j * 32, i == j && on_diag);
    }
    __syncthreads();
    const bool cvec = (P.C.ld % V == 0) && (((uintptr_t)pc & 15) == 0);
    // staged block (x, y): staging rows x V + e, 16-byte chunk y.  It is the
    // transpose of tile block (y, x).
    auto rdblk = [&](int x_, int y_, u32x4* x) {
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const int row = x_ * V + e;
        x[e] = *reinterpret_cast<const u32x4*>(smem + row * PITCH_S + (y_ ^ stage_swz(row)) * 16);
      }
    };
    // write block rows x[e] to rows r0 + e, columns c0 .. c0 + V - 1 of C
    auto wrblk = [&](int r0, int c0, const u32x4* x) {
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const int r = r0 + e;
        if (EXACT || r < P.M)
          store_chunk<SSZ>(pc, (int64_t)r * P.C.ld + c0, x[e], EXACT ? V : P.N - c0, EXACT || cvec);
      }
    };
    // direct pass: consecutive threads take consecutive column blocks of one
    // block row, so each block row is written as contiguous 16-byte chunks
    for (int b = tid; b < NBC * NBC; b += 256) {
      const int rb = b / NBC, cb = b - rb * NBC;
      const int r0 = m0 + rb * V, c0 = n0 + cb * V;
      if (!EXACT && (r0 >= P.M || c0 >= P.N)) continue;
      u32x4 x[V], y[V];
      if (!diag || rb > cb) {
        // lower tile (or strictly lower block of a diagonal tile)
        rdblk(cb, rb, y);
        transpose_block<SSZ>(y, x);
        wrblk(r0, c0, x);
      } else if (rb < cb) {
        rdblk(rb, cb, x);  // the transpose of the lower block (cb, rb)
        wrblk(r0, c0, x);
      } else {
        // diagonal block: lower elements from the block, upper from its transpose
        rdblk(rb, cb, y);
        transpose_block<SSZ>(y, x);
#pragma unroll
        for (int e = 0; e < V; ++e) {
          u32x4 z;
          if constexpr (SSZ == 2) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const uint32_t lo = (2 * w <= e) ? (x[e][w] & 0xffffu) : (y[e][w] & 0xffffu);
              const uint32_t hi = (2 * w + 1 <= e) ? (x[e][w] & 0xffff0000u) : (y[e][w] & 0xffff0000u);
              z[w] = lo | hi;
            }
          } else {
#pragma unroll
            for (int w = 0; w < 4; ++w) z[w] = (w <= e) ? x[e][w] : y[e][w];
          }
          x[e] = z;
        }
        wrblk(r0, c0, x);
      }
    }
    // mirror pass (off-diagonal tiles, unless the output is stored as its
    // lower triangle only): tile block (rb, cb), transposed (staged block
    // (cb, rb)), goes to rows n0 + cb * V.., columns m0 + rb * V..;
    // consecutive threads take consecutive rb so that each output row is
    // again written contiguously
    if (!diag && (g.lower & kLowerOut) == 0) {
      for (int b = tid; b < NBC * NBC; b += 256) {
        const int cb = b / NBC, rb = b - cb * NBC;
        const int r0 = m0 + rb * V, c0 = n0 + cb * V;
        if (!EXACT && (r0 >= P.M || c0 >= P.N)) continue;
        u32x4 y[V];
        rdblk(cb, rb, y);
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const int r = c0 + e;
          if (EXACT || r < P.M)
            store_chunk<SSZ>(pc, (int64_t)r * P.C.ld + r0, y[e], EXACT ? V : P.M - r0, EXACT || cvec);
        }
      }
    }
  } else if constexpr (EPI == EPI_AXPY) {
    // X' = c0 D + c1 alpha A B^T in the operand type, written over D (each
    // element is read and written by one thread, and no operand of the launch
    // is D) and transposed into C: fp32 staging of PR rows per pass, then one
    // 8 x 8 block per thread: 8 row chunks of D, the combination, 8 row
    // stores, a register transpose and 8 stores of the transposed rows.
    static_assert(Elt<E>::kSize == 2, "16-bit operands only");
    gchar* pd = gstore_ptr(const_cast<char*>(mat_ptr(P.D, g.tab, P.tab0, mi)));
    gchar* pt = gstore_ptr(const_cast<char*>(mat_ptr(P.C, g.tab, P.tab0, mi)));
    const int64_t ldd = P.D.ld, ldt = P.C.ld;
    const float cA = g.c1 * alpha;
    const bool vec = (ldd % 8 == 0) && (ldt % 8 == 0) && (((uintptr_t)pd & 15) == 0) && (((uintptr_t)pt & 15) == 0);
    typedef __attribute__((address_space(1))) u32x4 gu32x4;
    typedef __attribute__((address_space(1))) uint16_t gu16;
    constexpr int PR = BT / OUT_PASSES;  // rows per pass
#pragma unroll
    for (int pass = 0; pass < OUT_PASSES; ++pass) {
      if (pass) __syncthreads();
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const int c = wn * WTN + j * 32 + lcol;
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = wm * WTM + i * 32 + q * 8 + half * 4 + e - pass * PR;
              if (r >= 0 && r < PR)
                *reinterpret_cast<float*>(smem + r * PITCH_F + c * 4) = cA * acc[i][j][q * 4 + e];
            }
        }
      __syncthreads();
      constexpr int NBR = PR / 8, NBCOL = BT / 8;
      for (int b = tid; b < NBR * NBCOL; b += 256) {
        const int rb = b / NBCOL, cb = b - rb * NBCOL;
        const int r0 = m0 + pass * PR + rb * 8, c0 = n0 + cb * 8;
        if (!EXACT && (r0 >= P.M || c0 >= P.N)) continue;
        if (EXACT || (vec && r0 + 8 <= P.M && c0 + 8 <= P.N)) {
          u32x4 x[8], y[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const char* srow = smem + (rb * 8 + e) * PITCH_F + cb * 32;
            const u32x4 lo = *reinterpret_cast<const u32x4*>(srow);
            const u32x4 hi = *reinterpret_cast<const u32x4*>(srow + 16);
            const u32x4 d = *(const gu32x4*)(pd + ((int64_t)(r0 + e) * ldd + c0) * 2);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const float a0 = __uint_as_float(k < 2 ? lo[2 * k] : hi[2 * k - 4]);
              const float a1 = __uint_as_float(k < 2 ? lo[2 * k + 1] : hi[2 * k - 3]);
              const float v0 = fmaf(g.c0, Elt<E>::dec(d[k] & 0xffffu), a0);
              const float v1 = fmaf(g.c0, Elt<E>::dec(d[k] >> 16), a1);
              x[e][k] = Elt<E>::enc(v0) | (Elt<E>::enc(v1) << 16);
            }
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) *(gu32x4*)(pd + ((int64_t)(r0 + e) * ldd + c0) * 2) = x[e];
          transpose_block<2>(x, y);
#pragma unroll
          for (int e = 0; e < 8; ++e) *(gu32x4*)(pt + ((int64_t)(c0 + e) * ldt + r0) * 2) = y[e];
        } else {
          for (int e = 0; e < 8 && r0 + e < P.M; ++e) {
            for (int k = 0; k < 8 && c0 + k < P.N; ++k) {
              const float a = *reinterpret_cast<const float*>(smem + (rb * 8 + e) * PITCH_F + (cb * 8 + k) * 4);
              gu16* dp = (gu16*)pd + (int64_t)(r0 + e) * ldd + c0 + k;
              const uint32_t o = Elt<E>::enc(fmaf(g.c0, Elt<E>::dec(*dp), a));
              *dp = (uint16_t)o;
              ((gu16*)pt)[(int64_t)(c0 + k) * ldt + r0 + e] = (uint16_t)o;
            }
          }
        }
      }
    }
  } else {
    // full output: fp32 staging in OUT_PASSES row passes, then 8 columns per
    // thread per row segment.  16-bit operand kernels always write the
    // 16-bit caller layout (fp32 caller data runs the fp32 kernels); the
    // launch checks that.
    const bool of32 = Elt<E>::kSize == 4 && g.out_esize == 4;
    gchar* pc = gstore_ptr(const_cast<char*>(mat_ptr(EPI == EPI_UPD ? P.D : P.C, g.tab, P.tab0, mi)));
    const int64_t ldc = EPI == EPI_UPD ? P.D.ld : P.C.ld;
    const float cA = (EPI == EPI_UPD) ? g.c1 * alpha : alpha;
    const bool ovec = (ldc % 8 == 0) && (((uintptr_t)pc & 15) == 0);
    constexpr int PR = BT / OUT_PASSES;  // rows per pass
    constexpr int SEGS = BT / 8;         // 8-column segments per row
    constexpr int ITER = (PR * SEGS + 255) / 256;
    // An update reads W before writing it, WG segments at a time.  The
    // loads of a group are issued before the stores of the group ahead of it
    // (one vmcnt counter orders both, so a load issued after a store could
    // only be waited for together with that store), and the first group's
    // loads right after the first pass is staged, before its barrier: every
    // W fetch overlaps a barrier or a group's arithmetic and stores.
    constexpr int WG = (EPI != EPI_UPD) ? 1 : (ITER < (EXACT ? 8 : 4) ? ITER : (EXACT ? 8 : 4));
    static_assert(ITER % WG == 0, "segment groups");
    constexpr int WV = (EPI == EPI_UPD) ? WG * (Elt<E>::kSize == 4 ? 2 : 1) : 1;
    // Pass p stages the accumulator row blocks i with i / MTP == p of every
    // wave (all waves work in every pass, and which accumulators a pass
    // consumes is known at compile time).  Stage row r holds tile row
    // tile_row(p, r): wave row wm of the stage is rows [wm RPW, (wm + 1) RPW).
    constexpr int MTP = MT / OUT_PASSES;  // row blocks per wave per pass
    constexpr int RPW = 32 * MTP;         // stage rows per wave row
    static_assert(MT % OUT_PASSES == 0 && 2 * RPW == PR, "pass row mapping");
    auto tile_row = [&](int pass, int r) { return (r / RPW) * WTM + pass * RPW + r % RPW; };
    auto stage = [&](int pass) {
      __builtin_amdgcn_sched_barrier(0);  // keep each pass's conversions in place
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        if (i / MTP != pass) continue;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const int c = wn * WTN + j * 32 + lcol;
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = wm * RPW + (i % MTP) * 32 + q * 8 + half * 4 + e;
              *reinterpret_cast<float*>(smem + r * PITCH_F + c * 4) = cA * acc[i][j][q * 4 + e];
            }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    // W segments it0 .. it0 + WG - 1 of this thread in pass `pass` (16-byte
    // aligned whole segments; the others are read element-wise by `emit`)
    auto load_w = [&](int pass, int it0, u32x4* wv) {
#pragma unroll
      for (int u = 0; u < WG; ++u) {
        const int sgi = tid + (it0 + u) * 256;
        const int r = sgi / SEGS, sc = sgi - r * SEGS;
        const int gr = m0 + tile_row(pass, r), gc = n0 + sc * 8;
        const bool full = sgi < PR * SEGS && (EXACT || (gr < P.M && gc + 8 <= P.N));
        if (ovec && full) {
          const int64_t idx = (int64_t)gr * ldc + gc;
          if (of32) {
            if constexpr (Elt<E>::kSize == 4) {
              const __attribute__((address_space(1))) u32x4* q =
                  (const __attribute__((address_space(1))) u32x4*)(pc + idx * 4);
              wv[2 * u] = q[0];
              wv[2 * u + 1] = q[1];
            }
          } else {
            wv[(Elt<E>::kSize == 4 ? 2 : 1) * u] = *(const __attribute__((address_space(1))) u32x4*)(pc + idx * 2);
          }
        }
      }
    };
    // segments it0 .. it0 + WG - 1 of pass `pass`: the staged values (plus
    // c0 W for an update), written in the caller's element type
    auto emit = [&](int pass, int it0, const u32x4* wv) {
#pragma unroll
      for (int u = 0; u < WG; ++u) {
        const int it = it0 + u;
        const int sgi = tid + it * 256;
        if ((PR * SEGS) % 256 != 0 && sgi >= PR * SEGS) continue;
        const int r = sgi / SEGS, sc = sgi - r * SEGS;
        const int gr = m0 + tile_row(pass, r), gc = n0 + sc * 8;
        if (!EXACT && (gr >= P.M || gc >= P.N)) continue;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(smem + r * PITCH_F + sc * 32);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(smem + r * PITCH_F + sc * 32 + 16);
        float v[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          v[k] = __uint_as_float(lo[k]);
          v[k + 4] = __uint_as_float(hi[k]);
        }
        const int64_t idx = (int64_t)gr * ldc + gc;
        const int nvalid = EXACT ? 8 : (P.N - gc < 8 ? P.N - gc : 8);
        if (ovec && nvalid == 8) {
          if (of32) {
            __attribute__((address_space(1))) u32x4* q = (__attribute__((address_space(1))) u32x4*)(pc + idx * 4);
            if constexpr (EPI == EPI_UPD && Elt<E>::kSize == 4) {
              const u32x4 w0 = wv[2 * u], w1 = wv[2 * u + 1];
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                v[k] = fmaf(g.c0, __uint_as_float(w0[k]), v[k]);
                v[k + 4] = fmaf(g.c0, __uint_as_float(w1[k]), v[k + 4]);
              }
            }
            u32x4 o0, o1;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              o0[k] = __float_as_uint(v[k]);
              o1[k] = __float_as_uint(v[k + 4]);
            }
            __builtin_nontemporal_store(o0, q);
            __builtin_nontemporal_store(o1, q + 1);
          } else {
            __attribute__((address_space(1))) u32x4* q = (__attribute__((address_space(1))) u32x4*)(pc + idx * 2);
            if constexpr (EPI == EPI_UPD) {
              const u32x4 w = wv[(Elt<E>::kSize == 4 ? 2 : 1) * u];
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                v[2 * k] = fmaf(g.c0, __uint_as_float(w[k] << 16), v[2 * k]);
                v[2 * k + 1] = fmaf(g.c0, __uint_as_float(w[k] & 0xffff0000u), v[2 * k + 1]);
              }
            }
            u32x4 o;
#pragma unroll
            for (int k = 0; k < 4; ++k) o[k] = pack_bf16(v[2 * k], v[2 * k + 1]);
            __builtin_nontemporal_store(o, q);
          }
        } else {
          for (int k = 0; k < nvalid; ++k) {
            float x = v[k];
            if constexpr (EPI == EPI_UPD) x = fmaf(g.c0, load_out(pc, idx + k, of32), x);
            store_out(pc, idx + k, x, of32);
          }
        }
      }
    };
    if constexpr (EPI == EPI_UPD) {
      constexpr int NG = ITER / WG;         // groups per pass
      constexpr int NGT = OUT_PASSES * NG;  // groups of the tile
      u32x4 wv[2][WV];
#pragma unroll
      for (int gi = 0; gi < NGT; ++gi) {
        const int pass = gi / NG, grp = gi - pass * NG;
        if (grp == 0) {
          // LDS-only barriers: the W loads in flight stay in flight
          if (pass) ring_barrier();  // every wave has read the previous pass
          stage(pass);
          if (gi == 0) load_w(0, 0, wv[0]);
          ring_barrier();
        }
        if (gi + 1 < NGT) load_w((gi + 1) / NG, ((gi + 1) % NG) * WG, wv[(gi + 1) & 1]);
        emit(pass, grp * WG, wv[gi & 1]);
        __builtin_amdgcn_sched_barrier(0);  // one group's registers at a time
      }
    } else {
      u32x4 none[1];
#pragma unroll
      for (int pass = 0; pass < OUT_PASSES; ++pass) {
        if (pass) __syncthreads();
        stage(pass);
        __syncthreads();
        for (int it0 = 0; it0 < ITER; ++it0) emit(pass, it0, none);
      }
    }
  }
}

// Whether a launch covers whole tiles with 16-byte aligned operand rows, so
// that the unchecked loader (and direct loads) can be used.
template <class E, int BT>
bool launch_is_exact(const GemmArgs& a) {
  constexpr int VEC = 16 / Elt<E>::kSize;
  constexpr int BK = 8 * VEC;
  for (int p = 0; p < a.nprob; ++p) {
    const GemmProb& q = a.p[p];
    if (q.M % BT || q.N % BT || q.K % BK) return false;
    auto aligned = [&](const MatRef& r) {
      if (r.ld % VEC) return false;
      if (r.tab) {
        for (int i = 0; i < q.batch; ++i)
          if (a.tab[q.tab0 + i] & 15) return false;
        return true;
      }
      if (r.stride % 16) return false;
      return (reinterpret_cast<uintptr_t>(r.base) & 15) == 0;
    };
    if (!aligned(q.A) || !aligned(q.B)) return false;
  }
  return true;
}

template <class T>
struct TypeName;
template <>
struct TypeName<f16> {
  static constexpr const char* s = "_Float16";
};
template <>
struct TypeName<bf16_t> {
  static constexpr const char* s = "dmuon::(anonymous namespace)::bf16_t";
};
template <>
struct TypeName<float> {
  static constexpr const char* s = "float";
};

// Kernel instance name in the profiler's demangled form (without namespace
// and argument list).
template <class E, class S, int BT, bool A_MN, bool B_MN, int EPI, bool EXACT, int LOW>
const char* kernel_name() {
  static const std::string n = std::string("gemm_kernel<") + TypeName<E>::s + ", " + TypeName<S>::s + ", " +
                               std::to_string(BT) + ", " + (A_MN ? "true" : "false") + ", " +
                               (B_MN ? "true" : "false") + ", " + std::to_string(EPI) + ", " +
                               (EXACT ? "true" : "false") + ", " + std::to_string(LOW) + ">";
  return n.c_str();
}

template <class E, class S, int BT, bool A_MN, bool B_MN, int EPI, bool EXACT, int LOW>
hipError_t launch_inst(const GemmArgs& a, int grid, hipStream_t st, const char** name) {
  if (name) *name = kernel_name<E, S, BT, A_MN, B_MN, EPI, EXACT, LOW>();
  hipLaunchKernelGGL((gemm_kernel<E, S, BT, A_MN, B_MN, EPI, EXACT, LOW>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <class E, class S, int BT, bool A_MN, bool B_MN, int EPI>
hipError_t launch_one(const GemmArgs& a, hipStream_t st, const char** name) {
  if (a.nprob < 1 || a.nprob > kMaxProb) return hipErrorInvalidValue;
  // full outputs of 16-bit operand kernels are written as bf16 only
  if constexpr (Elt<E>::kSize == 2 && (EPI == EPI_OUT || EPI == EPI_UPD))
    if (a.out_esize != 2) return hipErrorInvalidValue;
  // the polynomial kernels square one matrix: A and B are the same operand
  if constexpr (EPI == EPI_POLY) {
    for (int p = 0; p < a.nprob; ++p) {
      const MatRef& x = a.p[p].A;
      const MatRef& y = a.p[p].B;
      if (x.base != y.base || x.stride != y.stride || x.ld != y.ld || x.tab != y.tab) return hipErrorInvalidValue;
    }
  }
  // every XCD takes at most ceil(n_p / 8) tiles of problem p
  int per_xcd = 0;
  for (int p = 0; p < a.nprob; ++p) per_xcd += (a.p[p].tiles * a.p[p].batch + 7) / 8;
  if (per_xcd <= 0) return hipSuccess;
  const int grid = per_xcd * 8;
  const bool exact = launch_is_exact<E, BT>(a);
  const int low = a.lower & (kLowerA | kLowerB);
  if (low == 0) {
    if (exact) return launch_inst<E, S, BT, A_MN, B_MN, EPI, true, 0>(a, grid, st, name);
    return launch_inst<E, S, BT, A_MN, B_MN, EPI, false, 0>(a, grid, st, name);
  }
  // lower-stored operands: only the direct-load ring reads them, for 16-bit
  // operands, tiles of 128 or 256 and whole tiles; the planner asks for them
  // only there
  constexpr bool CAN = Elt<E>::kSize == 2 && BT >= 128 && !A_MN && !B_MN;
  if constexpr (CAN) {
    if (!exact) return hipErrorInvalidValue;
    if constexpr (EPI == EPI_SYM || EPI == EPI_POLY) {
      if (low == (kLowerA | kLowerB)) return launch_inst<E, S, BT, A_MN, B_MN, EPI, true, 3>(a, grid, st, name);
    } else if constexpr (EPI == EPI_OUT || EPI == EPI_UPD) {
      if (low == kLowerA) return launch_inst<E, S, BT, A_MN, B_MN, EPI, true, 1>(a, grid, st, name);
      if (low == kLowerB) return launch_inst<E, S, BT, A_MN, B_MN, EPI, true, 2>(a, grid, st, name);
    }
  }
  return hipErrorInvalidValue;
}

inline bool same_mat(const MatRef& x, const MatRef& y) {
  return x.base == y.base && x.stride == y.stride && x.ld == y.ld && x.tab == y.tab;
}

// Dispatch over the kinds for one MFMA operand type E, with state type S and
// the operand type of the Gram product G (from the input copy).  ROWS_ONLY:
// the host hands every operand over as row panels with K contiguous (16-bit
// buckets read transposed copies), so the N-contiguous kinds are not built.
template <class E, class S, class G, bool ROWS_ONLY, int BT>
hipError_t launch_kind(GemmKind kind, const GemmArgs& a, hipStream_t st, const char** n) {
  switch (kind) {
    case KIND_SYRK_KK: return launch_one<G, S, BT, false, false, EPI_SYM>(a, st, n);
    case KIND_SYM_KK: return launch_one<E, S, BT, false, false, EPI_SYM>(a, st, n);
    case KIND_POLY:
      // the kernels read the linear term D from A's panel: A, B and D must be
      // one matrix
      for (int i = 0; i < a.nprob; ++i) {
        const GemmProb& q = a.p[i];
        if (!same_mat(q.A, q.B) || !same_mat(q.A, q.D)) return hipErrorInvalidValue;
      }
      return launch_one<E, S, BT, false, false, EPI_POLY>(a, st, n);
    case KIND_OUT_KK: return launch_one<E, S, BT, false, false, EPI_OUT>(a, st, n);
    case KIND_UPD_KK: return launch_one<E, S, BT, false, false, EPI_UPD>(a, st, n);
    case KIND_AXPY_KK:
      if constexpr (Elt<E>::kSize == 2)
        return launch_one<E, S, BT, false, false, EPI_AXPY>(a, st, n);
      else
        return hipErrorInvalidValue;
    case KIND_SYRK_MM:
    case KIND_OUT_KM:
    case KIND_UPD_KM:
      if constexpr (ROWS_ONLY) {
        return hipErrorInvalidValue;
      } else {
        if (kind == KIND_SYRK_MM) return launch_one<G, S, BT, true, true, EPI_SYM>(a, st, n);
        if (kind == KIND_OUT_KM) return launch_one<E, S, BT, false, true, EPI_OUT>(a, st, n);
        return launch_one<E, S, BT, false, true, EPI_UPD>(a, st, n);
      }
  }
  return hipErrorInvalidValue;
}

template <class E, class S, class G, bool ROWS_ONLY>
hipError_t launch_tile(int tile, GemmKind kind, const GemmArgs& a, hipStream_t st, const char** n) {
  switch (tile) {
    case 64: return launch_kind<E, S, G, ROWS_ONLY, 64>(kind, a, st, n);
    case 128: return launch_kind<E, S, G, ROWS_ONLY, 128>(kind, a, st, n);
    case 256:
      // a 256 x 256 fp32 tile does not fit the LDS staging of the symmetric
      // epilogues; the planner caps fp32 buckets at 128
      if constexpr (Elt<S>::kSize == 4)
        return hipErrorInvalidValue;
      else
        return launch_kind<E, S, G, ROWS_ONLY, 256>(kind, a, st, n);
  }
  return hipErrorInvalidValue;
}

}  // namespace
}  // namespace dmuon
