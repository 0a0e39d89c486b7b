// Fused Gram Newton-Schulz for short sides up to 128: one workgroup runs the
// whole map for one matrix (DMuon, gist.science technical summary section 2.2:
// Gram product, the m x m recurrence P = aI + bA + cA^2, R = PA, A <- RP,
// Q <- PQ, and the final product Q X), with every m x m state held in LDS.
//
// At these sizes the grouped product kernel is latency-bound: each of the
// 4T + 1 products of a bucket is a launch of a few microseconds over a handful
// of tiles, with the states round-tripping through HBM in between.  Here the
// states never leave LDS and the launch count per bucket is one.
//
// Numerics follow the grouped path: the Gram product runs on the input's bf16
// bits with fp32 accumulation; the states are fp16 scaled by a power of two s
// (A~ = s A, so P = aI + (b/s) A~ + (c/s^2) A~^2), Q is stored divided by
// 2^e_k, and the final product multiplies Q by the input scaled into fp16
// range by a power of two sx.  The Frobenius norm is the square root of the
// Gram matrix's trace.
//
// Workgroup: 512 threads = 8 waves (two per SIMD, so that one wave's
// epilogue overlaps the other's MFMAs), MP = the short side padded to 64 or
// 128 with zero rows.  Every stored m x m state is symmetric, so a product
// C = A B needs only row panels of both operands (B's column panel is its row
// panel).  The symmetry has to be exact -- a product read this way with a
// slightly asymmetric B computes A B^T, and the recurrence amplifies the
// difference by about a^2 per step -- so, as in the grouped kernels, only the
// lower 32 x 32 blocks of a symmetric product are computed and each lower
// element is stored at both of its positions.  For MP = 128 (4 x 4 blocks)
// waves 0 .. 3 take the diagonal blocks, waves 4 .. 7 the off-diagonal ones --
// (1, 0) and (2, 0), (3, 0) and (3, 1), (2, 1), (3, 2) -- so that every SIMD
// (waves w and w + 4) carries at most three blocks and a wave with two shares
// one fragment between them; for MP = 64 (2 x 2 blocks) waves 0, 1 and 2 take
// one block each.  The final product (not symmetric) uses a 4 x 2 wave grid
// over each 128-column chunk of the output.
//
// The states take the whole 160 KB LDS, so a CU runs one workgroup: a launch
// carries up to 256 matrices (their pointers in the kernel arguments), one
// per CU, and larger batches take several launches that each fill the GPU.

#include "gemm_impl.h"
#include "small.h"

#include <type_traits>

namespace dmuon {
namespace {

constexpr int kSmallThreads = 512;
constexpr int kSmallNC = 128;  // output columns per chunk of the final product

template <int MP>
struct SmallCfg {
  static constexpr int ND = MP / 64;      // 32-row blocks per diagonal tile side
  static constexpr int KS = MP / 16;      // 16-deep MFMA steps over K = MP
  static constexpr int SB = MP * 2 * MP;  // bytes per fp16 state
  static constexpr int GST = MP * 128;    // Gram stage: MP rows x 64 K values (bf16)
  static constexpr int XST = MP * 256;    // final-product stage: MP K rows x 128 columns (fp16)
  static constexpr int OST = MP * kSmallNC * 4;  // fp32 output stage: MP rows x 128 columns
  // LDS map: states A~, R~, P and two Q buffers.  Before the recurrence the
  // two Gram stages use R and P; in the final phase A (and R) hold the X
  // stage and the output stage follows in R and P when it fits there.
  static constexpr int OFF_A = 0, OFF_R = SB, OFF_P = 2 * SB, OFF_Q0 = 3 * SB, OFF_Q1 = 4 * SB;
  static constexpr int OFF_G = OFF_R;
  static constexpr int OFF_X = 0;
  static constexpr int OFF_O = (OST <= 2 * SB) ? OFF_R : 5 * SB;
  static constexpr int LDS = (OFF_O + OST > 5 * SB) ? OFF_O + OST : 5 * SB;
  static_assert(2 * GST <= 2 * SB, "Gram stages must fit in R and P");
  static_assert(XST <= OFF_O && XST <= OFF_Q0, "X stage must fit below the output stage and Q");
  static_assert(LDS <= 160 * 1024, "LDS");
};

// State rows: 16-byte chunks XOR-swizzled so that the 16 lanes of a fragment
// read (16 consecutive rows, one logical chunk) hit 16 different bank groups.
template <int MP>
__device__ __forceinline__ int st_off(int r, int ch) {
  if constexpr (MP == 128)
    return r * 256 + ((ch ^ (r & 15)) << 4);
  else
    return r * 128 + ((ch ^ lds_swz(r)) << 4);
}
// byte offset of element (r, c) of a state
template <int MP>
__device__ __forceinline__ int st_elem(int r, int c) {
  return st_off<MP>(r, c >> 3) + (c & 7) * 2;
}
// Final-product stage: K row k holds 128 fp16 columns, chunks swizzled by
// (k & 3) << 2 for the transposing reads.
__device__ __forceinline__ int xs_off(int k, int ch) { return k * 256 + ((ch ^ ((k & 3) << 2)) << 4); }
// fp32 output stage: row i holds 128 values as 32 chunks of four.
__device__ __forceinline__ int os_off(int i, int jc) { return i * 512 + ((jc ^ (i & 31)) << 4); }

// Sum over the 64 lanes, in every lane: DPP within each row of 16 lanes
// (pairs, quads, then rotations by 4 and 8), then the four row sums read
// out lane by lane -- no LDS round trips.
__device__ __forceinline__ float wave_sum_f(float v) {
  auto dpp = [](float x, auto ctrl) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), decltype(ctrl)::value, 0xf, 0xf, false));
  };
  v += dpp(v, std::integral_constant<int, 0xb1>{});   // quad_perm [1, 0, 3, 2]
  v += dpp(v, std::integral_constant<int, 0x4e>{});   // quad_perm [2, 3, 0, 1]
  v += dpp(v, std::integral_constant<int, 0x124>{});  // row_ror 4
  v += dpp(v, std::integral_constant<int, 0x128>{});  // row_ror 8
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (r0 + r1) + (r2 + r3);
}

// The blocks of one wave: the blocks (ib0 + i, jb[j]) for i < NA, j < NB, of
// which block (0, 0) is a diagonal block (ib0 == jb[0]) when DG.  Every wave
// owns exactly one diagonal block.
template <int NA_, int NB_, bool DG_>
struct Shape {
  static constexpr int NA = NA_, NB = NB_;
  static constexpr bool DG = DG_;
};

__device__ __forceinline__ void zero16(f32x16& a) {
#pragma unroll
  for (int r = 0; r < 16; ++r) a[r] = 0.0f;
}
template <int N>
__device__ __forceinline__ void zero_acc(f32x16 (&acc)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) zero16(acc[i]);
}

// Accumulators of a wave's blocks: block (i, j) of its shape is entry
// i NB + j (at most two blocks).
constexpr int kMaxBlk = 2;
// acc[i NB + j] += sum over KS 16-deep steps of A fragment i times B fragment
// j; rdA(i, ks) / rdB(j, ks) return this lane's 8 K values of the step.  The
// next step's fragments are read while the current step's MFMAs run.  With
// TWO, acc2 += A B2 as well.  SAME: A and B are one matrix, so a diagonal
// block (shape DG, 1 x 1) reads its single fragment once.
template <class E, int KS, class SH, bool TWO, bool SAME = false, class RA, class RB, class RB2>
__device__ __forceinline__ void mma_shape(f32x16 (&acc)[kMaxBlk], f32x16 (&acc2)[kMaxBlk], RA rdA, RB rdB,
                                          RB2 rdB2) {
  static_assert(SH::NA * SH::NB <= kMaxBlk, "blocks per wave");
  constexpr int NA = SH::NA, NB = SH::NB;
  u32x4 fa[2][NA], fb[2][NB], fc[2][NB];
  constexpr bool ONE = SAME && SH::DG && NA == 1 && NB == 1;
  auto rd = [&](int set, int ks) {
#pragma unroll
    for (int i = 0; i < NA; ++i) fa[set][i] = rdA(i, ks);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if constexpr (ONE)
        fb[set][j] = fa[set][0];
      else
        fb[set][j] = rdB(j, ks);
      if constexpr (TWO) fc[set][j] = rdB2(j, ks);
    }
  };
  rd(0, 0);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int cur = ks & 1;
    if (ks + 1 < KS) rd(cur ^ 1, ks + 1);
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
        {
          Mfma<E>::run(fa[cur][i], fb[cur][j], acc[i * NB + j]);
          if constexpr (TWO) Mfma<E>::run(fa[cur][i], fc[cur][j], acc2[i * NB + j]);
        }
  }
}

// Block products listed as jobs: acc[n] += sum over KS 16-deep steps of A
// fragment JA[n] times B fragment JB[n], NA A fragments and NB B fragments
// read per step (the next step's while the current step's MFMAs run).
template <class E, int KS, int NA, int NB, int NJ, class RA, class RB>
__device__ __forceinline__ void mma_jobs(f32x16 (&acc)[NJ], const int (&JA)[NJ], const int (&JB)[NJ], RA rdA, RB rdB) {
  u32x4 fa[2][NA], fb[2][NB];
  auto rd = [&](int set, int ks) {
#pragma unroll
    for (int i = 0; i < NA; ++i) fa[set][i] = rdA(i, ks);
#pragma unroll
    for (int j = 0; j < NB; ++j) fb[set][j] = rdB(j, ks);
  };
  rd(0, 0);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int cur = ks & 1;
    if (ks + 1 < KS) rd(cur ^ 1, ks + 1);
#pragma unroll
    for (int n = 0; n < NJ; ++n) Mfma<E>::run(fa[cur][JA[n]], fb[cur][JB[n]], acc[n]);
  }
}

// The R~ and Q' products of one recurrence step at MP = 128 for waves 4-7:
// three off-diagonal block products each (with the diagonal waves' two, five
// per SIMD instead of 6, 6, 4, 4).  Wave 4 + w': A fragments are P's row
// panels ROW[i]; B fragments are row panels PAN[j] of A~ (BQ[j] = 0) or of Q
// (BQ[j] = 1); job n multiplies A fragment JA[n] by B fragment JB[n].
struct RqJobs4 {  // R~(1,0), R~(2,0), Q'(1,0)
  static constexpr int NA = 2, NB = 2;
  static constexpr int ROW[2] = {1, 2}, PAN[2] = {0, 0}, BQ[2] = {0, 1};
  static constexpr int JA[3] = {0, 1, 0}, JB[3] = {0, 0, 1};
};
struct RqJobs5 {  // R~(3,0), R~(3,1), Q'(3,0)
  static constexpr int NA = 1, NB = 3;
  static constexpr int ROW[1] = {3}, PAN[3] = {0, 1, 0}, BQ[3] = {0, 0, 1};
  static constexpr int JA[3] = {0, 0, 0}, JB[3] = {0, 1, 2};
};
struct RqJobs6 {  // R~(2,1), Q'(2,1), Q'(2,0)
  static constexpr int NA = 1, NB = 3;
  static constexpr int ROW[1] = {2}, PAN[3] = {1, 1, 0}, BQ[3] = {0, 1, 1};
  static constexpr int JA[3] = {0, 0, 0}, JB[3] = {0, 1, 2};
};
struct RqJobs7 {  // R~(3,2), Q'(3,2), Q'(3,1)
  static constexpr int NA = 1, NB = 3;
  static constexpr int ROW[1] = {3}, PAN[3] = {2, 2, 1}, BQ[3] = {0, 1, 1};
  static constexpr int JA[3] = {0, 0, 0}, JB[3] = {0, 1, 2};
};

// 16 bytes of row `r` (of `rows`), columns c .. c + 7 (of `cols`), from a
// row-major bf16 matrix with row pitch `ld`; zero outside the matrix.
__device__ __forceinline__ u32x4 load_piece(cgchar* p, int64_t ld, int r, int c, int rows, int cols, bool vec) {
  if (r >= rows || c >= cols) return u32x4{0u, 0u, 0u, 0u};
  const int64_t idx = (int64_t)r * ld + c;
  if (vec && c + 8 <= cols) return gload16(p + idx * 2);
  return load_chunk_partial<2>(p, idx, cols - c);
}

// PH: SMALL_ONE runs the whole map; SMALL_REC and SMALL_FINAL are its two
// parts for the split launches (small.h).
template <int MP, int PH>
__global__ void __launch_bounds__(kSmallThreads) small_ns_kernel(const SmallArgs g) {
  using C = SmallCfg<MP>;
  constexpr int ND = C::ND, KS = C::KS;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];
  // A~ lives in the second state buffer and R~ in the first: the Gram
  // stages occupy the buffers from the second on, and the first holds the
  // trace partials while the last Gram reads finish.
  char* const sA = smem + C::OFF_R;
  char* const sR = smem + C::OFF_A;
  char* const sP = smem + C::OFF_P;

  // The final launch's grid is (chunks, matrices).  Workgroups go to the
  // eight XCDs in turn by linear index, and the recurrence launch ran matrix
  // m on XCD m mod 8; when the matrix count is a multiple of 8 the final
  // launch's workgroups are renumbered so that every chunk of matrix m runs
  // on that XCD too, where its Q image and X are still in the L2.
  int mat = blockIdx.x, fchunk = 0;
  if constexpr (PH == SMALL_FINAL) {
    mat = blockIdx.y;
    fchunk = blockIdx.x;
    if ((gridDim.y & 7) == 0) {
      const int lin = blockIdx.y * gridDim.x + blockIdx.x;
      const int slot = lin >> 3;
      mat = (lin & 7) + 8 * (slot / (int)gridDim.x);
      fchunk = slot % (int)gridDim.x;
    }
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Waves w and w + 4 share a SIMD.  At MP = 128 waves 4-7 hold the
  // off-diagonal blocks, the longer share of their SIMD in every phase (the
  // partner has a diagonal block: one fragment per step, no transposed
  // writes); issuing them first takes their chain off the phase's tail.
  if constexpr (PH != SMALL_FINAL && MP == 128) {
    if (__builtin_amdgcn_readfirstlane(wave) >= 4) __builtin_amdgcn_s_setprio(1);
  }
  // split launches: this matrix's Q image and the final product's scalars
  char* const split = (PH == SMALL_ONE) ? nullptr : g.split_base + (int64_t)mat * g.split_stride;
  const int half = lane >> 5, l32 = lane & 31;
  const int rows = g.rows, cols = g.cols;

  gchar* const out = gstore_ptr(reinterpret_cast<void*>(g.tab[mat]));
  cgchar* const xsrc = g.x_base ? gload_ptr(g.x_base + (int64_t)mat * g.x_stride) : (cgchar*)out;
  const bool xvec = (cols % 8 == 0) && ((reinterpret_cast<uintptr_t>(xsrc) & 15) == 0);
  const bool ovec = (cols % 8 == 0) && ((reinterpret_cast<uintptr_t>(out) & 15) == 0);

  // ---- fragment readers
  // row panel of a state: rows row0 + [0, 32), K values 16 ks + 8 half + [0, 8)
  auto rd_st = [&](const char* base, int row0, int ks) -> u32x4 {
    return *reinterpret_cast<const u32x4*>(base + st_off<MP>(row0 + l32, 2 * ks + half));
  };
  // row panel of a Gram stage (64 K values per row)
  auto rd_g = [&](const char* base, int row0, int sub) -> u32x4 {
    return *reinterpret_cast<const u32x4*>(base + lds_off(row0 + l32, 2 * sub + half));
  };
  // columns j0 + [0, 32) of the final-product stage read as rows of its
  // transpose: in each group of 16 lanes, lane 4 q + x supplies K row k0 + q,
  // columns j0 + 16 (group & 1) + 4 x .. + 3, and the transposing read hands
  // lane j of the group the four K values of column j0 + 16 (group & 1) + j
  auto rd_x = [&](const char* base, int j0, int ks) -> u32x4 {
    const int grp = lane >> 4, lq = lane & 15;
    const int k0 = 16 * ks + 8 * (grp >> 1) + (lq >> 2);
    const int col = j0 + 16 * (grp & 1) + 4 * (lq & 3);
    auto at = [&](int k) {
      return (__attribute__((address_space(3))) v4i16*)(const_cast<char*>(base) + xs_off(k, col >> 3) +
                                                          (col & 7) * 2);
    };
    const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(at(k0)));
    const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(at(k0 + 4)));
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };

  // ---- the lower blocks of this wave (see the header): f(shape, ib0, jb)
  // with jb[j] the column block of column j of the shape
  auto for_shape = [&](auto&& f) {
    if constexpr (MP == 128) {
      if (wave < 4)
        f(Shape<1, 1, true>{}, wave, [=](int) { return wave; });
      else if (wave == 4)
        f(Shape<2, 1, false>{}, 1, [](int) { return 0; });
      else if (wave == 5)
        f(Shape<1, 2, false>{}, 3, [](int j) { return j; });
      else if (wave == 6)
        f(Shape<1, 1, false>{}, 2, [](int) { return 1; });
      else
        f(Shape<1, 1, false>{}, 3, [](int) { return 2; });
    } else {
      if (wave < 2)
        f(Shape<1, 1, true>{}, wave, [=](int) { return wave; });
      else if (wave == 2)
        f(Shape<1, 1, false>{}, 1, [](int) { return 0; });
    }
  };

  // Diagonal block at rows and columns d0 .. d0 + 31 of S whose upper
  // triangle holds the right values: copy it onto the lower triangle, in 4 x 4
  // sub-blocks, lane l taking sub-block (l / 8, l % 8) when it is on or below
  // the diagonal (sub-block (br, bc), br > bc, is the transpose of (bc, br); a
  // diagonal sub-block keeps its own diagonal and upper part).  Only the wave
  // that wrote the block touches it, and a wave's LDS accesses execute in
  // order, so no barrier is needed between the writes and this.
  auto mirror_diag = [&](char* S, int d0) {
    const int br = lane >> 3, bc = lane & 7;
    if (br >= bc) {
      u32x2 x[4], y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        x[e] = *reinterpret_cast<const u32x2*>(S + st_elem<MP>(d0 + 4 * bc + e, d0 + 4 * br));
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const int sh = 16 * (e & 1);
          const uint32_t lo = (x[2 * w][e >> 1] >> sh) & 0xffffu, hi = (x[2 * w + 1][e >> 1] >> sh) & 0xffffu;
          y[e][w] = lo | (hi << 16);
        }
      if (br == bc) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int w = 0; w < 2; ++w) {
            const uint32_t lo = (2 * w < e) ? (y[e][w] & 0xffffu) : (x[e][w] & 0xffffu);
            const uint32_t hi = (2 * w + 1 < e) ? (y[e][w] & 0xffff0000u) : (x[e][w] & 0xffff0000u);
            y[e][w] = lo | hi;
          }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *reinterpret_cast<u32x2*>(S + st_elem<MP>(d0 + 4 * br + e, d0 + 4 * bc)) = y[e];
    }
  };

  // 32 x 32 MFMA result layout: lane l, register 4 q + e -> row 8 q + 4 (l / 32)
  // + e, column l % 32.  For block (i, j) of a shape the four values of
  // (q, all e) are C[R + e][c], R = 32 (ib0 + i) + 8 q + 4 (l / 32),
  // c = 32 jb(j) + l % 32.  Stored symmetric: S[c][R .. R + 3] (one 8-byte
  // write) and, off the diagonal, S[R + x][c0 .. c0 + 3] (one 8-byte write),
  // where x = l % 4 and c0 = c - x: the four lanes of a quad hold columns
  // c0 .. c0 + 3 of rows R .. R + 3, and a 4 x 4 transpose across the quad
  // (two DPP exchanges, of 32-bit words between lanes x and x ^ 2, then of
  // 16-bit halves between x and x ^ 1) hands lane x row R + x.  (Sixteen
  // 2-byte writes per block in its place cost a fifth of the recurrence
  // launch.)  A diagonal block gets the transposed writes only -- its upper
  // triangle then holds its lower elements -- and then the in-wave mirror.
  auto store_sym = [&](auto sh, int ib0, auto jb, char* dst, auto&& val) {
    using SH = decltype(sh);
#pragma unroll
    for (int i = 0; i < SH::NA; ++i)
#pragma unroll
      for (int j = 0; j < SH::NB; ++j) {
        const bool dblk = SH::DG && i == 0 && j == 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int R = 32 * (ib0 + i) + 8 * q + 4 * half;
          const int c = 32 * jb(j) + l32;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = val(i, j, q, e, R + e == c);
          const uint32_t p01 = pack_f16(v[0], v[1]), p23 = pack_f16(v[2], v[3]);
          *reinterpret_cast<u32x2*>(dst + st_elem<MP>(c, R)) = u32x2{p01, p23};
          if (!dblk) {
            const int x = lane & 3;
            // words: lanes 0, 1 take the low word of lane x + 2 as their high
            // word, lanes 2, 3 the high word of lane x - 2 as their low word
            const bool lo2 = x < 2;
            const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)(lo2 ? p23 : p01), 0x4e, 0xf, 0xf, false);
            const uint32_t d0 = lo2 ? p01 : recv, d1 = lo2 ? recv : p23;
            // halves: even lanes pair their low halves with the partner's,
            // odd lanes their high halves (one byte permute per word)
            const uint32_t r0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)d0, 0xb1, 0xf, 0xf, false);
            const uint32_t r1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)d1, 0xb1, 0xf, 0xf, false);
            const uint32_t sel = (x & 1) ? 0x03020706u : 0x05040100u;
            *reinterpret_cast<u32x2*>(dst + st_elem<MP>(R + x, c - x)) =
                u32x2{__builtin_amdgcn_perm(r0, d0, sel), __builtin_amdgcn_perm(r1, d1, sel)};
          }
        }
      }
    if constexpr (SH::DG) mirror_diag(dst, 32 * ib0);
  };

  // ================================================================ Gram
  // A~ = s kappa^2 X X^T over chunks of 64 columns of X (bf16, MP rows; rows
  // past `rows` and columns past `cols` are zero).  Piece t of chunk ch in
  // this thread: row p / 8, columns 64 ch + 8 (p % 8) .. + 7, p = tid + 512 t.
  // Up to RCH chunks (512 columns) X is loaded whole, every load in flight at
  // once, staged whole in LDS (chunk c at OFF_R + c GST: the states are not
  // live yet) behind a single barrier, and the MFMAs run through all chunks
  // without another; longer rows stream through two stages, the next chunk
  // fetched while the current one feeds the MFMAs.  The final product reads X
  // again (from L2).
  constexpr int GP = C::GST / 16 / kSmallThreads;  // pieces per thread per chunk
  constexpr int RP = 16;                           // resident pieces per thread
  constexpr int RCH = (RP / GP) < (C::LDS - C::OFF_R) / C::GST ? (RP / GP) : (C::LDS - C::OFF_R) / C::GST;
  static_assert(C::OFF_R + RCH * C::GST <= C::LDS, "resident Gram chunks must fit in LDS");
  const int nch = (cols + 63) / 64;
  auto piece = [&](int ch, int t) {
    const int p = tid + t * kSmallThreads;
    return load_piece(xsrc, cols, p >> 3, ch * 64 + (p & 7) * 8, rows, cols, xvec);
  };
  auto gstore = [&](char* st, const u32x4* v) {
#pragma unroll
    for (int t = 0; t < GP; ++t) {
      const int p = tid + t * kSmallThreads;
      *reinterpret_cast<u32x4*>(st + lds_off(p >> 3, p & 7)) = v[t];
    }
  };
  f32x16 acc[kMaxBlk], acq[kMaxBlk];
  zero_acc(acc);
  auto no_b = [](int, int) { return u32x4{0u, 0u, 0u, 0u}; };
  auto gram_chunk = [&](const char* st) {
    for_shape([&](auto sh, int ib0, auto jb) {
      mma_shape<bf16_t, 4, decltype(sh), false, true>(
          acc, acq, [&](int i, int sub) { return rd_g(st, 32 * (ib0 + i), sub); },
          [&](int j, int sub) { return rd_g(st, 32 * jb(j), sub); }, no_b);
    });
  };
  double kappa = 0.0, sx = 1.0;
  float fsx = 1.0f, oscale = 1.0f;
  const char* sQ = smem + C::OFF_Q0;
  if constexpr (PH != SMALL_FINAL) {
  const bool resident = nch <= RCH;
  if (resident) {
    u32x4 xres[RP];
#pragma unroll
    for (int c = 0; c < RCH; ++c)
#pragma unroll
      for (int t = 0; t < GP; ++t) xres[c * GP + t] = piece(c, t);
#pragma unroll
    for (int c = 0; c < RCH; ++c)
      if (c < nch) gstore(smem + C::OFF_R + c * C::GST, xres + c * GP);
    __syncthreads();
    // All chunks are in LDS, so the fragments of chunk c + 1 are read while
    // chunk c's MFMAs run (two register sets of four 16-deep steps; past the
    // last chunk the read repeats the last chunk, unused).  A wave owns one
    // or two blocks, so one step is one to two MFMAs: reading one step ahead
    // left every step waiting on an LDS read.
    for_shape([&](auto sh, int ib0, auto jb) {
      using SH = decltype(sh);
      constexpr int NA = SH::NA, NB = SH::NB;
      constexpr bool ONE = SH::DG && NA == 1 && NB == 1;
      u32x4 fa[2][4][NA], fb[2][4][NB];
      auto rdc = [&](auto set, int c) {
        constexpr int S = decltype(set)::value;
        const char* st = smem + C::OFF_R + c * C::GST;
#pragma unroll
        for (int sub = 0; sub < 4; ++sub) {
#pragma unroll
          for (int i = 0; i < NA; ++i) fa[S][sub][i] = rd_g(st, 32 * (ib0 + i), sub);
#pragma unroll
          for (int j = 0; j < NB; ++j) fb[S][sub][j] = ONE ? fa[S][sub][0] : rd_g(st, 32 * jb(j), sub);
        }
      };
      auto mmac = [&](auto set) {
        constexpr int S = decltype(set)::value;
#pragma unroll
        for (int sub = 0; sub < 4; ++sub)
#pragma unroll
          for (int i = 0; i < NA; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j) Mfma<bf16_t>::run(fa[S][sub][i], fb[S][sub][j], acc[i * NB + j]);
      };
      using S0 = std::integral_constant<int, 0>;
      using S1 = std::integral_constant<int, 1>;
      rdc(S0{}, 0);
      for (int c = 0; c < nch; c += 2) {
        rdc(S1{}, c + 1 < nch ? c + 1 : nch - 1);
        mmac(S0{});
        if (c + 1 < nch) {
          rdc(S0{}, c + 2 < nch ? c + 2 : nch - 1);
          mmac(S1{});
        }
      }
    });
  } else {
    u32x4 gr[GP];
#pragma unroll
    for (int t = 0; t < GP; ++t) gr[t] = piece(0, t);
    for (int ch = 0; ch < nch; ++ch) {
      char* st = smem + C::OFF_G + (ch & 1) * C::GST;
      gstore(st, gr);
      __syncthreads();
      if (ch + 1 < nch) {
#pragma unroll
        for (int t = 0; t < GP; ++t) gr[t] = piece(ch + 1, t);
      }
      gram_chunk(st);
    }
  }
  // ||X||_F^2 = trace(X X^T): each diagonal block is the first block of the
  // wave that owns it (all four waves for MP = 128, waves 0 and 1 for 64).
  // The partials go to the R~ buffer, which no Gram stage uses and which is
  // first written by step 0's R~ product; the barrier after them also
  // ends every wave's Gram reads, so A~ may then overwrite the stages.
  constexpr int NDW = MP / 32;  // waves owning a diagonal block
  float* red = reinterpret_cast<float*>(sR);
  if (wave < NDW) {
    float t = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (8 * q + 4 * half + e == l32) t += acc[0][4 * q + e];
    t = wave_sum_f(t);
    if (lane == 0) red[wave] = t;
  }
  __syncthreads();
  double tr = 0.0;
#pragma unroll
  for (int w = 0; w < NDW; ++w) tr += (double)red[w];
  const double nrm = sqrt(tr);
  kappa = 1.0 / (nrm + (double)g.eps);
  int ex = 0;
  if (nrm > 0.0 && nrm <= 1.0e300) {
    int q;
    frexp(nrm, &q);  // nrm in [2^(q-1), 2^q)
    ex = 14 - q;     // 2^ex nrm < 2^14: every scaled entry fits fp16
    ex = ex < -120 ? -120 : (ex > 120 ? 120 : ex);
  }
  sx = ldexp(1.0, ex);
  fsx = (float)sx;
  {
    const float alpha = (float)(kappa / sx) * g.ofac;
    oscale = g.update ? g.c1 * alpha : alpha;
  }
  {
    const float as = (float)((double)g.sscale * kappa * kappa);
    for_shape([&](auto sh, int ib0, auto jb) {
      using SH = decltype(sh);
      store_sym(sh, ib0, jb, sA, [&](int i, int j, int q, int e, bool) { return acc[i * SH::NB + j][4 * q + e] * as; });
    });
  }
  __syncthreads();

  // ================================================================ recurrence
  char* qcur = smem + C::OFF_Q0;
  char* qnext = smem + C::OFF_Q1;
  for (int k = 0; k < g.steps; ++k) {
    char* const sPk = (k == 0) ? qcur : sP;  // P_0 is Q_1 itself
    // P = a I + b1 A~ + c2 A~^2; A~ at every accumulator position is read
    // (at the transposed position, one 8-byte read per four values) before
    // any P value is written
    for_shape([&](auto sh, int ib0, auto jb) {
      using SH = decltype(sh);
      zero_acc(acc);
      mma_shape<f16, KS, SH, false, true>(
          acc, acq, [&](int i, int ks) { return rd_st(sA, 32 * (ib0 + i), ks); },
          [&](int j, int ks) { return rd_st(sA, 32 * jb(j), ks); }, no_b);
      u32x2 old[SH::NA][SH::NB][4];
#pragma unroll
      for (int i = 0; i < SH::NA; ++i)
#pragma unroll
        for (int j = 0; j < SH::NB; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int R = 32 * (ib0 + i) + 8 * q + 4 * half;
            const int c = 32 * jb(j) + l32;
            old[i][j][q] = *reinterpret_cast<const u32x2*>(sA + st_elem<MP>(c, R));
          }
      store_sym(sh, ib0, jb, sPk, [&](int i, int j, int q, int e, bool diag) {
        const uint32_t w = old[i][j][q][e >> 1];
        const float ae = f16_to_f32((w >> (16 * (e & 1))) & 0xffffu);
        const float v = fmaf(g.c2, acc[i * SH::NB + j][4 * q + e], g.b1 * ae);
        return diag ? v + g.a : v;
      });
    });
    __syncthreads();
    const bool need_a = k + 1 < g.steps;
    const bool need_q = k >= 1;
    const float qm = g.qmul[k];
    // R~ = P A~ into R, Q' = P Q into the other Q buffer
    // waves 4-7 at MP = 128 with both products: the balanced job lists
    auto rq_jobs = [&](auto tbl) {
      using T = decltype(tbl);
      f32x16 jacc[3];
      zero_acc(jacc);
      mma_jobs<f16, KS, T::NA, T::NB, 3>(
          jacc, T::JA, T::JB, [&](int i, int ks) { return rd_st(sPk, 32 * T::ROW[i], ks); },
          [&](int j, int ks) { return rd_st(T::BQ[j] ? qcur : sA, 32 * T::PAN[j], ks); });
#pragma unroll
      for (int n = 0; n < 3; ++n) {
        const bool isq = T::BQ[T::JB[n]] != 0;
        const float mul = isq ? qm : 1.0f;
        store_sym(Shape<1, 1, false>{}, T::ROW[T::JA[n]], [=](int) { return T::PAN[T::JB[n]]; }, isq ? qnext : sR,
                  [&](int, int, int q, int e, bool) { return jacc[n][4 * q + e] * mul; });
      }
    };
    bool balanced = false;
    if constexpr (MP == 128) {
      if (need_a && need_q && wave >= 4) {
        balanced = true;
        if (wave == 4)
          rq_jobs(RqJobs4{});
        else if (wave == 5)
          rq_jobs(RqJobs5{});
        else if (wave == 6)
          rq_jobs(RqJobs6{});
        else
          rq_jobs(RqJobs7{});
      }
    }
    if (need_a || need_q) {
      if (!balanced) for_shape([&](auto sh, int ib0, auto jb) {
        using SH = decltype(sh);
        zero_acc(acc);
        zero_acc(acq);
        auto rdP = [&](int i, int ks) { return rd_st(sPk, 32 * (ib0 + i), ks); };
        auto rdA = [&](int j, int ks) { return rd_st(sA, 32 * jb(j), ks); };
        auto rdQ = [&](int j, int ks) { return rd_st(qcur, 32 * jb(j), ks); };
        if (need_a && need_q)
          mma_shape<f16, KS, SH, true>(acc, acq, rdP, rdA, rdQ);
        else if (need_a)
          mma_shape<f16, KS, SH, false>(acc, acq, rdP, rdA, no_b);
        else
          mma_shape<f16, KS, SH, false>(acq, acc, rdP, rdQ, no_b);
        if (need_a)
          store_sym(sh, ib0, jb, sR, [&](int i, int j, int q, int e, bool) { return acc[i * SH::NB + j][4 * q + e]; });
        if (need_q)
          store_sym(sh, ib0, jb, qnext,
                    [&](int i, int j, int q, int e, bool) { return acq[i * SH::NB + j][4 * q + e] * qm; });
      });
      __syncthreads();
    }
    if (need_q) {
      char* t = qcur;
      qcur = qnext;
      qnext = t;
    }
    if (need_a) {
      // A~' = R~ P; every read of A~ finished before the last barrier
      for_shape([&](auto sh, int ib0, auto jb) {
        using SH = decltype(sh);
        zero_acc(acc);
        mma_shape<f16, KS, SH, false>(
            acc, acq, [&](int i, int ks) { return rd_st(sR, 32 * (ib0 + i), ks); },
            [&](int j, int ks) { return rd_st(sPk, 32 * jb(j), ks); }, no_b);
        store_sym(sh, ib0, jb, sA, [&](int i, int j, int q, int e, bool) { return acc[i * SH::NB + j][4 * q + e]; });
      });
      __syncthreads();
    }
  }

  if constexpr (PH == SMALL_REC) {
    // Q's LDS image and the final product's two scalars, for the final launch
    // (all of a thread's LDS reads first, then its stores: one LDS latency)
    constexpr int QP = C::SB / 16 / kSmallThreads;  // Q-image pieces per thread
    static_assert(QP * 16 * kSmallThreads == C::SB, "Q image pieces");
    gchar* const dst = gstore_ptr(split);
    u32x4 qv[QP];
#pragma unroll
    for (int t = 0; t < QP; ++t) qv[t] = *reinterpret_cast<const u32x4*>(qcur + 16 * (tid + t * kSmallThreads));
#pragma unroll
    for (int t = 0; t < QP; ++t)
      *reinterpret_cast<__attribute__((address_space(1))) u32x4*>(dst + 16 * (tid + t * kSmallThreads)) = qv[t];
    if (tid == 0) {
      __attribute__((address_space(1))) float* f = (__attribute__((address_space(1))) float*)(dst + C::SB);
      f[0] = fsx;
      f[1] = oscale;
    }
    return;
  }
  sQ = qcur;
  }
  // (the final launch reads the recurrence launch's Q image and scalars below,
  // together with its X chunk)

  // ================================================================ final
  // O^T (chunk of 128 columns of X) = X_chunk^T Q: A operand the X stage read
  // transposed (rows j of the chunk), B operand Q's rows.  Waves form a 4 x 2
  // grid: 32 chunk columns by MP / 2 rows of O each.  A lane's four rows
  // j .. j + 3 in column i are four consecutive outputs O[i][j .. j + 3].
  constexpr int XP = C::XST / 16 / kSmallThreads;  // 16-byte pieces per thread per chunk
  constexpr int OP = MP * 16 / kSmallThreads;      // 8-column output units per thread per chunk
  char* const sX = smem + C::OFF_X;
  char* const sO = smem + C::OFF_O;
  const int nfc = (cols + kSmallNC - 1) / kSmallNC;
  const int wm = wave >> 1, wn = wave & 1;
  const int j0w = wm * 32, i0w = wn * (MP / 2);
  f32x16 fac[1][ND];
  // chunk fc with the X stage written: MFMAs, the fp32 output stage, then the
  // write-out (or the update of W), 8 columns per unit
  auto final_chunk = [&](int fc) {
    zero_acc(fac[0]);
    {
      u32x4 fa[2][1], fb[2][ND];
      auto rd = [&](int set, int ks) {
        fa[set][0] = rd_x(sX, j0w, ks);
#pragma unroll
        for (int b = 0; b < ND; ++b) fb[set][b] = rd_st(sQ, i0w + 32 * b, ks);
      };
      rd(0, 0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int cur = ks & 1;
        if (ks + 1 < KS) rd(cur ^ 1, ks + 1);
#pragma unroll
        for (int b = 0; b < ND; ++b) Mfma<f16>::run(fa[cur][0], fb[cur][b], fac[0][b]);
      }
    }
#pragma unroll
    for (int b = 0; b < ND; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = i0w + 32 * b + l32;
        const int j = j0w + 8 * q + 4 * half;
        const f32x16& v = fac[0][b];
        float4 o = {v[4 * q] * oscale, v[4 * q + 1] * oscale, v[4 * q + 2] * oscale, v[4 * q + 3] * oscale};
        *reinterpret_cast<float4*>(sO + os_off(i, j >> 2)) = o;
      }
    // every W value of the chunk is loaded before any result is stored (the
    // stores go to the same matrix, so they would otherwise hold back each
    // following load)
    u32x4 wv[OP];
    if (g.update) {
#pragma unroll
      for (int t = 0; t < OP; ++t) {
        const int u = tid + t * kSmallThreads;
        const int i = u >> 4, col = fc * kSmallNC + (u & 15) * 8;
        const int64_t idx = (int64_t)i * cols + col;
        const int nvalid = cols - col;
        wv[t] = (i >= rows || col >= cols) ? u32x4{0u, 0u, 0u, 0u}
                : (ovec && nvalid >= 8)    ? gload16((cgchar*)out + idx * 2)
                                           : load_chunk_partial<2>((cgchar*)out, idx, nvalid);
      }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < OP; ++t) {
      const int u = tid + t * kSmallThreads;
      const int i = u >> 4, gq = u & 15;
      const int col = fc * kSmallNC + gq * 8;
      if (i >= rows || col >= cols) continue;
      const float4 lo = *reinterpret_cast<const float4*>(sO + os_off(i, 2 * gq));
      const float4 hi = *reinterpret_cast<const float4*>(sO + os_off(i, 2 * gq + 1));
      float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      const int64_t idx = (int64_t)i * cols + col;
      const int nvalid = cols - col;
      if (g.update) {
        const u32x4 w = wv[t];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[2 * e] = fmaf(g.c0, __uint_as_float(w[e] << 16), v[2 * e]);
          v[2 * e + 1] = fmaf(g.c0, __uint_as_float(w[e] & 0xffff0000u), v[2 * e + 1]);
        }
      }
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = pack_bf16(v[2 * e], v[2 * e + 1]);
      store_chunk<2>(out, idx, o, nvalid, ovec);
    }
  };
  // piece t of chunk fc in this thread: K row p / 16, columns 128 fc +
  // 8 (p % 16) .. + 7 (raw bf16); stored to the X stage as fp16 times 2^e
  auto xpiece = [&](int fc, int t) {
    const int p = tid + t * kSmallThreads;
    return load_piece(xsrc, cols, p >> 4, fc * kSmallNC + (p & 15) * 8, rows, cols, xvec);
  };
  auto xstore = [&](const u32x4* v) {
#pragma unroll
    for (int t = 0; t < XP; ++t) {
      const int p = tid + t * kSmallThreads;
      u32x4 x = v[t];
      cvt_chunk(x, fsx);
      *reinterpret_cast<u32x4*>(sX + xs_off(p >> 4, p & 15)) = x;
    }
  };
  constexpr int FR = 16;       // pieces per thread read up front
  constexpr int FCH = FR / XP;  // chunks read up front: 512 columns at MP = 128, 1024 at 64
  if constexpr (PH == SMALL_FINAL) {
    // one chunk per workgroup.  The chunk of X, the recurrence launch's Q
    // image (into the Q_0 buffer) and its two scalars are all requested
    // before the first wait, so the launch pays one memory latency, not one
    // per piece; the barrier ahead of the MFMAs orders the LDS writes.
    constexpr int QP = C::SB / 16 / kSmallThreads;  // Q-image pieces per thread
    static_assert(QP * 16 * kSmallThreads == C::SB, "Q image pieces");
    const int fc = fchunk;
    u32x4 v[XP], qv[QP];
#pragma unroll
    for (int t = 0; t < XP; ++t) v[t] = xpiece(fc, t);
    cgchar* const src = gload_ptr(split);
#pragma unroll
    for (int t = 0; t < QP; ++t) qv[t] = gload16(src + 16 * (tid + t * kSmallThreads));
    const __attribute__((address_space(1))) float* f = (const __attribute__((address_space(1))) float*)(src + C::SB);
    fsx = f[0];
    oscale = f[1];
#pragma unroll
    for (int t = 0; t < QP; ++t)
      *reinterpret_cast<u32x4*>(smem + C::OFF_Q0 + 16 * (tid + t * kSmallThreads)) = qv[t];
    xstore(v);
    __syncthreads();
    final_chunk(fc);
  } else if (nfc <= FCH) {
    // every chunk's loads in flight at once (the recurrence's registers are
    // free by now); chunk fc is consumed when its turn comes
    u32x4 xf[FR];
#pragma unroll
    for (int c = 0; c < FCH; ++c)
#pragma unroll
      for (int t = 0; t < XP; ++t) xf[c * XP + t] = xpiece(c, t);
    for (int fc = 0; fc < nfc; ++fc) {
      u32x4 v[XP];
#pragma unroll
      for (int c = 0; c < FCH; ++c) {
        if (c == fc) {
#pragma unroll
          for (int t = 0; t < XP; ++t) v[t] = xf[c * XP + t];
        }
      }
      xstore(v);
      __syncthreads();
      final_chunk(fc);
    }
  } else {
    // longer rows: chunks read again one ahead, the next fetched during this one
    u32x4 xr[XP];
#pragma unroll
    for (int t = 0; t < XP; ++t) xr[t] = xpiece(0, t);
    for (int fc = 0; fc < nfc; ++fc) {
      xstore(xr);
      __syncthreads();
      if (fc + 1 < nfc) {
#pragma unroll
        for (int t = 0; t < XP; ++t) xr[t] = xpiece(fc + 1, t);
      }
      final_chunk(fc);
    }
  }
}

}  // namespace

namespace {

template <int MP>
hipError_t launch_mp(const SmallArgs& a, int nmat, SmallLaunch which, hipStream_t st, const char** name) {
  const unsigned nfc = (unsigned)((a.cols + kSmallNC - 1) / kSmallNC);
  const dim3 block(kSmallThreads);
  switch (which) {
    case SMALL_ONE:
      if (name) *name = MP == 64 ? "small_ns_kernel<64>" : "small_ns_kernel<128>";
      hipLaunchKernelGGL((small_ns_kernel<MP, SMALL_ONE>), dim3((unsigned)nmat), block, 0, st, a);
      break;
    case SMALL_REC:
      if (name) *name = MP == 64 ? "small_ns_kernel<64>:rec" : "small_ns_kernel<128>:rec";
      hipLaunchKernelGGL((small_ns_kernel<MP, SMALL_REC>), dim3((unsigned)nmat), block, 0, st, a);
      break;
    case SMALL_FINAL:
      if (name) *name = MP == 64 ? "small_ns_kernel<64>:final" : "small_ns_kernel<128>:final";
      hipLaunchKernelGGL((small_ns_kernel<MP, SMALL_FINAL>), dim3(nfc, (unsigned)nmat), block, 0, st, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int64_t small_split_bytes(int rows) {
  const int64_t mp = rows <= 64 ? 64 : 128;
  return mp * mp * 2 + 16;
}

hipError_t launch_small_ns(const SmallArgs& a, int nmat, SmallLaunch which, hipStream_t st, const char** name) {
  if (nmat <= 0) return hipSuccess;
  if (nmat > kSmallMaxTab || a.rows <= 0 || a.rows > 128 || a.cols < a.rows || a.steps < 1 ||
      a.steps > kSmallMaxSteps)
    return hipErrorInvalidValue;
  if (which != SMALL_ONE) {
    // the split region must hold Q's image and the scalars of each of the
    // nmat matrices
    if (!a.split_base || a.split_stride < small_split_bytes(a.rows) ||
        a.split_stride % 16 != 0 || ((uintptr_t)a.split_base & 15) != 0)
      return hipErrorInvalidValue;
    if ((a.cols + kSmallNC - 1) / kSmallNC > 65535) return hipErrorInvalidValue;
  }
  return a.rows <= 64 ? launch_mp<64>(a, nmat, which, st, name) : launch_mp<128>(a, nmat, which, st, name);
}

}  // namespace dmuon
