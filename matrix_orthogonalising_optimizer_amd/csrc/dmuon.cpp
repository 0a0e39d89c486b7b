// libdmuon host side: argument validation, the shape planner, workspace
// management and the launch sequence of the Gram Newton-Schulz path.
//
// Method: DMuon (gist.science technical summary, section 2.2 for the Gram-space
// recurrence, symmetric products and batching; section 2.4 for the per-shape
// tile choice cached across steps; sections 1 and 5 for the Muon update).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "dmuon.h"
#include "errors.h"
#include "adamw.h"
#include "kernels.h"
#include "scratch.h"
#include "small.h"

namespace dmuon {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

namespace {

#define HIP_TRY(expr)                                                              \
  do {                                                                             \
    hipError_t e_ = (expr);                                                        \
    if (e_ != hipSuccess)                                                          \
      return fail(DMUON_EHIP, "%s failed: %s", #expr, hipGetErrorString(e_));      \
  } while (0)

constexpr double kDefaultEps = 1e-7;
constexpr size_t kAlign = 256;
// fused buckets: groups of at most this many matrices run the two-launch
// split under DMUON_FUSED_AUTO (its final product then takes 256 workgroups
// for rows of 512 columns)
constexpr int64_t kSplitMax = 64;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// --------------------------------------------------------------------- timing
struct TimingRec {
  std::string name;
  double flops = 0, bytes = 0;
  hipEvent_t a = nullptr, b = nullptr;
};
std::mutex g_tmu;
bool g_timing = false;
std::vector<TimingRec> g_trecs;

template <class F>
hipError_t timed(const std::string& name, double flops, double bytes, hipStream_t st, F&& launch) {
  if (!g_timing) return launch();
  TimingRec r;
  r.name = name;
  r.flops = flops;
  r.bytes = bytes;
  hipError_t e = hipEventCreate(&r.a);
  if (e == hipSuccess) e = hipEventCreate(&r.b);
  if (e == hipSuccess) e = hipEventRecord(r.a, st);
  if (e != hipSuccess) return e;
  e = launch();
  if (e != hipSuccess) return e;
  e = hipEventRecord(r.b, st);
  std::lock_guard<std::mutex> lk(g_tmu);
  g_trecs.push_back(r);
  return e;
}

bool sym_kind(GemmKind k) {
  return k == KIND_SYRK_KK || k == KIND_SYRK_MM || k == KIND_SYM_KK || k == KIND_POLY;
}

hipError_t gemm(Prec p, GemmKind k, int tile, const GemmArgs& a, hipStream_t st) {
  if (!g_timing) return launch_gemm(p, k, tile, a, st);
  double flops = 0.0;
  for (int i = 0; i < a.nprob; ++i) {
    const GemmProb& q = a.p[i];
    flops += sym_kind(k) ? (double)q.batch * q.M * (q.M + 1.0) * q.K : (double)q.batch * 2.0 * q.M * q.N * q.K;
  }
  const char* name = "gemm_kernel";
  // the launch names its kernel instance; record the events around it
  TimingRec r;
  r.flops = flops;
  hipError_t e = hipEventCreate(&r.a);
  if (e == hipSuccess) e = hipEventCreate(&r.b);
  if (e == hipSuccess) e = hipEventRecord(r.a, st);
  if (e != hipSuccess) return e;
  e = launch_gemm(p, k, tile, a, st, &name);
  if (e != hipSuccess) return e;
  e = hipEventRecord(r.b, st);
  r.name = name;
  std::lock_guard<std::mutex> lk(g_tmu);
  g_trecs.push_back(r);
  return e;
}

// --------------------------------------------------------------------- tune table
// Square block tile per launch, keyed by the short side m of the recurrence
// bucket and the number of matrices in it (the pages' per-shape, cached
// configuration choice: gist.science technical summary, section 2.4).
constexpr int64_t kAnyBatch = INT64_MAX;
struct TuneEntry {
  int64_t max_m;      // entry applies to m <= max_m ...
  int64_t max_batch;  // ... and to buckets of at most max_batch matrices
  int rec;            // tile of the m x m recurrence products
  int syrk;           // tile of the Gram product
  int fin;            // tile of the final product
};

std::vector<TuneEntry> builtin_table() {
  return {
      {96, kAnyBatch, 64, 64, 64},
      {384, kAnyBatch, 128, 128, 128},
      {1 << 30, kAnyBatch, 256, 256, 256},
  };
}

bool valid_tile(int t) { return t == 64 || t == 128 || t == 256; }

// Minimal reader for the tune-table JSON:
//   {"entries": [{"max_m": 96, "max_batch": 8, "rec": 64, "syrk": 64, "final": 64}, ...]}
// "max_batch" is optional (any batch).  Entries must be sorted by (max_m,
// max_batch), strictly increasing; other keys and objects outside
// "entries" are ignored.
bool parse_tune_json(const std::string& text, std::vector<TuneEntry>& out, std::string& err) {
  out.clear();
  size_t pos = text.find("\"entries\"");
  if (pos == std::string::npos) {
    err = "no \"entries\" key";
    return false;
  }
  pos = text.find('[', pos);
  if (pos == std::string::npos) {
    err = "no entry list";
    return false;
  }
  while (true) {
    size_t ob = text.find('{', pos);
    size_t close = text.find(']', pos);
    if (ob == std::string::npos || (close != std::string::npos && close < ob)) break;
    size_t cb = text.find('}', ob);
    if (cb == std::string::npos) {
      err = "unterminated entry";
      return false;
    }
    std::string obj = text.substr(ob, cb - ob);
    auto field = [&](const char* key, long long& v) -> bool {
      std::string k = std::string("\"") + key + "\"";
      size_t p = obj.find(k);
      if (p == std::string::npos) return false;
      p = obj.find(':', p);
      if (p == std::string::npos) return false;
      char* end = nullptr;
      v = std::strtoll(obj.c_str() + p + 1, &end, 10);
      return end != obj.c_str() + p + 1;
    };
    long long mm, r, s, f, mb = kAnyBatch;
    if (!field("max_m", mm) || !field("rec", r) || !field("syrk", s) || !field("final", f)) {
      err = "entry lacks max_m/rec/syrk/final";
      return false;
    }
    if (obj.find("\"max_batch\"") != std::string::npos && (!field("max_batch", mb) || mb <= 0)) {
      err = "max_batch must be a positive integer";
      return false;
    }
    if (!valid_tile((int)r) || !valid_tile((int)s) || !valid_tile((int)f) || mm <= 0) {
      err = "tile must be 64, 128 or 256 and max_m positive";
      return false;
    }
    if (!out.empty() && (mm < out.back().max_m || (mm == out.back().max_m && mb <= out.back().max_batch))) {
      err = "entries must be sorted by increasing (max_m, max_batch)";
      return false;
    }
    out.push_back({(int64_t)mm, (int64_t)mb, (int)r, (int)s, (int)f});
    pos = cb + 1;
  }
  if (out.empty()) {
    err = "empty entry list";
    return false;
  }
  return true;
}

// The first entry with m <= max_m and count <= max_batch; else the last.
const TuneEntry& lookup(const std::vector<TuneEntry>& t, int64_t m, int64_t count) {
  for (const auto& e : t)
    if (m <= e.max_m && count <= e.max_batch) return e;
  return t.back();
}

// --------------------------------------------------------------------- precision
// Short sides up to this size run on fp32 MFMA under DMUON_PREC_AUTO unless
// every member is wide (long side >= 2 x short side): 16-bit operands lose
// too much on small, nearly square Gram matrices (their smallest eigenvalues
// are squared singular values; measured 1.6e-2 .. 2.4e-2 relative error at
// 64 x 64 and 128 x 128 against the 2e-2 bar), while wide members stay near
// 3e-3 and run the fused fp16 kernel.
constexpr int64_t kSmallM = 128;

// Largest |entry| allowed in the fp16 state (fp16 max is 65504).
constexpr double kF16Lim = 30000.0;
// Q is stored divided by a power of two that keeps it below this bound.
constexpr double kQTarget = 8192.0;

// Scan of the scalar recurrence.  Every stored m x m matrix is symmetric and a
// polynomial in A0, whose eigenvalues are squared singular values of the
// normalised input and lie in [0, 1); a symmetric matrix's entries are bounded
// by its spectral norm, so bounds on the scalar images bound every entry.
//   A~_k = s sigma_k^2, P_k = p_k = a + b sigma_k^2 + c sigma_k^4,
//   R_k = A~_k p_k, A~_{k+1} = A~_k p_k^2, Q_k = prod_{j<k} p_j.
struct RangeScan {
  double state_max = 0;         // max over A~, P, R (for s = 1)
  double p_max = 0;             // max |P|
  std::vector<double> q_max;    // q_max[k] = max |Q_k|, k = 0..T
};

RangeScan scan_recurrence_uncached(double a, double b, double c, int steps) {
  RangeScan r;
  r.q_max.assign(steps + 1, 0.0);
  const int N = 4096;
  for (int i = 0; i <= N; ++i) {
    double x = (double)i / N, q = 1.0;
    r.q_max[0] = 1.0;
    for (int k = 0; k < steps; ++k) {
      const double lam = x * x;
      const double p = a + b * lam + c * lam * lam;
      q *= p;
      r.p_max = std::max(r.p_max, std::fabs(p));
      r.state_max = std::max({r.state_max, lam, std::fabs(lam * p), std::fabs(lam * p * p)});
      r.q_max[k + 1] = std::max(r.q_max[k + 1], std::fabs(q));
      x = p * x;
    }
  }
  return r;
}

// The scan walks 4097 sample points through every step: about 0.1 ms of host
// time, more than the GPU work of a small step.  Callers repeat the same
// coefficients call after call, so each thread keeps its last result.
RangeScan scan_recurrence(double a, double b, double c, int steps) {
  struct Last {
    bool valid = false;
    double a = 0, b = 0, c = 0;
    int steps = 0;
    RangeScan r;
  };
  thread_local Last last;
  if (!last.valid || last.a != a || last.b != b || last.c != c || last.steps != steps) {
    last.r = scan_recurrence_uncached(a, b, c, steps);
    last.a = a;
    last.b = b;
    last.c = c;
    last.steps = steps;
    last.valid = true;
  }
  return last.r;
}

double state_scale_for(int64_t m) {
  // largest power of two <= min(m, 8192): the fp16 Gram state is A0 * s, with
  // diagonal entries of order s/m at the start and at most about s later on
  int64_t s = 1;
  while (s * 2 <= std::min<int64_t>(m, 8192)) s *= 2;
  return (double)s;
}

// Power-of-two exponents e_k with Q_k / 2^e_k <= kQTarget (e_1 = 0: Q_1 = P_0).
std::vector<int> q_exponents(const RangeScan& r) {
  std::vector<int> e(r.q_max.size(), 0);
  for (size_t k = 2; k < e.size(); ++k) {
    int x = 0;
    while (r.q_max[k] / std::ldexp(1.0, x) > kQTarget && x < 1000) ++x;
    e[k] = x;
  }
  return e;
}

// Largest Q exponent allowed: Q entries of magnitude 1/4 and up (the
// directions the iteration has converged, where the products p_j stay near 1)
// must stay normal fp16 numbers (>= 2^-14) after the division by 2^e_k.  Long
// runs of coefficients with a large linear term grow Q so fast on the null
// directions (like a^k) that the scale would flush the rest to zero.
constexpr int kQMaxExp = 12;

bool f16_range_ok(const RangeScan& r, double s) {
  if (!(std::isfinite(r.state_max) && r.state_max * s < kF16Lim && r.p_max < kF16Lim && r.p_max <= kQTarget))
    return false;
  for (int e : q_exponents(r))
    if (e > kQMaxExp) return false;
  return true;
}

// --------------------------------------------------------------------- plan layout
struct Group {  // matrices with identical caller shape
  int64_t rows = 0, cols = 0, m = 0, n = 0;
  bool trans = false;
  std::vector<int64_t> members;  // plan indices
  int rec = -1;                  // recurrence bucket
  int64_t slot0 = 0;             // first slot in that bucket
  size_t x_off = 0;              // workspace copy of X (or u), caller layout
  int64_t x_stride = 0;          // bytes per matrix
  size_t xt_off = 0;             // its transpose (16-bit buckets): cols x rows
  int64_t xt_stride = 0;
  int64_t xt_ld = 0;             // row pitch of the transpose, elements
  size_t xt2_off = 0;            // standard form: second buffer of X^T rows (n x m)
  int64_t xt2_stride = 0;
  int64_t xc_ld = 0;             // its row pitch
  size_t part_off = 0;           // fp64 partial sums
  int nblk = 1;
  int tile_syrk = 256, tile_fin = 256;
  // fused bucket run as two launches (small.h): the workspace region that
  // carries one launch's Q images to the final product
  bool split = false;
  size_t split_off = 0;
  int64_t split_stride = 0;
};

struct RecBucket {  // matrices with identical short side m
  int64_t m = 0, ldm = 0, count = 0;
  std::vector<int> groups;
  size_t st_off[5] = {0, 0, 0, 0, 0};  // A~, P, R, Qa, Qb
  int64_t st_stride = 0;
  size_t scal_off = 0;
  int tile = 256;
  bool f32 = false;       // runs on fp32 MFMA with fp32 state and input copies
  bool standard = false;  // standard form (16-bit buckets only)
  bool lower = false;     // symmetric states stored as their lower triangle of tiles
  bool small = false;     // eligible for the fused one-launch kernel (fp16 state only)
};

}  // namespace

struct PlanImpl {
  int dtype = DMUON_BF16;
  int precision_req = DMUON_PREC_AUTO;
  int form_req = DMUON_FORM_AUTO;
  int storage_req = DMUON_STORAGE_AUTO;
  int fused_req = DMUON_FUSED_AUTO;
  double pad_ratio = 0.0;
  int scale_mode = DMUON_SCALE_SQRT_RATIO;
  double eps = kDefaultEps;
  bool device = true;
  int device_id = -1;
  int64_t count = 0;
  std::vector<int64_t> rows, cols;
  std::vector<Group> groups;
  std::vector<RecBucket> buckets;
  std::vector<TuneEntry> table;
  std::string table_source = "builtin";
  size_t ws_bytes = 0;  // for the widest precision the plan can run
  char* ws = nullptr;   // owned when owns_ws
  bool owns_ws = false;
};

namespace {

int elem_size(int dtype) { return dtype == DMUON_F32 ? 4 : 2; }

// Whether a bucket runs on fp32 MFMA for a given precision request.
// `wide`: every member of the bucket has long side >= 2 x its short side.
bool bucket_is_f32(int dtype, int req, int64_t m, bool wide) {
  if (dtype == DMUON_F32 || req == DMUON_PREC_F32) return true;
  return req == DMUON_PREC_AUTO && m <= kSmallM && !wide;
}

bool groups_wide(const PlanImpl& p, const std::vector<int>& gs) {
  for (int gi : gs)
    if (p.groups[gi].n < 2 * p.groups[gi].m) return false;
  return true;
}

// Sizes and offsets of every workspace region.
void layout(PlanImpl& p) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = round_up(off + bytes, kAlign);
    return o;
  };
  for (auto& b : p.buckets) {
    b.f32 = bucket_is_f32(p.dtype, p.precision_req, b.m, groups_wide(p, b.groups));
    // form: STANDARD on request (16-bit buckets), or under AUTO for plain
    // bf16 products on near-square members (every n <= 2 m)
    bool near_square = true;
    for (int gi : b.groups) near_square = near_square && p.groups[gi].n <= 2 * b.m;
    b.standard = !b.f32 && (p.form_req == DMUON_FORM_STANDARD ||
                            (p.form_req == DMUON_FORM_AUTO && p.precision_req == DMUON_PREC_BF16 && near_square));
    const int se = b.f32 ? 4 : 2;
    b.ldm = (int64_t)round_up((size_t)b.m, 64);
    b.st_stride = (int64_t)round_up((size_t)(b.m * b.ldm * se), kAlign);
    for (int s = 0; s < 5; ++s) b.st_off[s] = take((size_t)b.st_stride * b.count);
    b.scal_off = take(sizeof(float) * kScalStride * b.count);
  }
  for (auto& g : p.groups) {
    const int ce = p.buckets[g.rec].f32 ? 4 : 2;
    const int64_t elems = g.rows * g.cols;
    // a padded bucket's Gram product reads pm >= m rows of X, the rows past
    // m zero: the copy that holds X's rows gets them
    const int64_t pm = p.buckets[g.rec].m;
    g.x_stride = (int64_t)round_up((size_t)((g.trans ? elems : pm * g.cols) * ce), kAlign);
    g.x_off = take((size_t)g.x_stride * g.members.size());
    if (!p.buckets[g.rec].f32) {
      g.xt_ld = (int64_t)round_up((size_t)g.rows, 64);
      g.xt_stride = (int64_t)round_up((size_t)((g.trans ? pm : g.cols) * g.xt_ld * 2), kAlign);
      g.xt_off = take((size_t)g.xt_stride * g.members.size());
      if (p.buckets[g.rec].standard) {
        // second buffer of X^T rows (n x m): same pitch as the buffer it
        // alternates with (the transpose copy for wide matrices, the
        // caller-layout copy for tall ones)
        g.xc_ld = g.trans ? g.m : g.xt_ld;
        g.xt2_stride = (int64_t)round_up((size_t)(g.n * g.xc_ld * 2), kAlign);
        g.xt2_off = take((size_t)g.xt2_stride * g.members.size());
      }
    }
    // blocks per matrix of the elementwise passes: about 16K elements each,
    // and at least 2048 over the group (a few workgroups per CU) while every
    // thread still has a full 4-element step: one block per CU leaves the
    // grid-stride loops of a group of small matrices latency-bound
    const int64_t nmem = (int64_t)g.members.size();
    int64_t nb = (elems + 16383) / 16384;
    nb = std::max(nb, std::min((2048 + nmem - 1) / nmem, (elems + 1023) / 1024));
    g.nblk = (int)std::max<int64_t>(1, std::min<int64_t>(nb, 1024));
    g.part_off = take(sizeof(double) * g.nblk * g.members.size());
  }
  p.ws_bytes = off;
}

int build_plan(PlanImpl& p, const int64_t* rows, const int64_t* cols, int64_t count) {
  p.count = count;
  p.rows.assign(rows, rows + count);
  p.cols.assign(cols, cols + count);
  std::map<std::pair<int64_t, int64_t>, int> gidx;
  std::map<int64_t, int> bidx;
  std::vector<int> group_order;
  for (int64_t i = 0; i < count; ++i) {
    const int64_t r = rows[i], c = cols[i];
    auto key = std::make_pair(r, c);
    auto it = gidx.find(key);
    if (it == gidx.end()) {
      Group g;
      g.rows = r;
      g.cols = c;
      g.trans = r > c;
      g.m = std::min(r, c);
      g.n = std::max(r, c);
      gidx[key] = (int)p.groups.size();
      p.groups.push_back(g);
      it = gidx.find(key);
    }
    p.groups[it->second].members.push_back(i);
  }
  // Recurrence size of each short side: itself, or -- with padding -- the
  // size of a bucket of similar short sides.  Largest first, a side opens a
  // bucket of size round_up(m, 64) (m itself if that exceeds m (1 + ratio))
  // or joins the smallest open bucket within m (1 + ratio).  fp32 buckets
  // are never padded.
  std::map<int64_t, int64_t> rec_size;
  {
    std::vector<int64_t> ms;
    for (const Group& g : p.groups) ms.push_back(g.m);
    std::sort(ms.begin(), ms.end(), std::greater<int64_t>());
    ms.erase(std::unique(ms.begin(), ms.end()), ms.end());
    std::vector<int64_t> open;
    for (int64_t m : ms) {
      std::vector<int> with_m;
      for (int gi = 0; gi < (int)p.groups.size(); ++gi)
        if (p.groups[gi].m == m) with_m.push_back(gi);
      if (p.pad_ratio <= 0.0 || bucket_is_f32(p.dtype, p.precision_req, m, groups_wide(p, with_m))) {
        rec_size[m] = m;
        continue;
      }
      const double lim = (double)m * (1.0 + p.pad_ratio);
      int64_t best = -1;
      for (int64_t M : open)
        if (M >= m && (double)M <= lim && (best < 0 || M < best)) best = M;
      if (best < 0) {
        best = (int64_t)round_up((size_t)m, 64);
        if ((double)best > lim) best = m;
        open.push_back(best);
      }
      rec_size[m] = best;
    }
  }
  // recurrence buckets by that size, in first-appearance order of their groups
  for (int gi = 0; gi < (int)p.groups.size(); ++gi) {
    Group& g = p.groups[gi];
    const int64_t M = rec_size[g.m];
    auto it = bidx.find(M);
    if (it == bidx.end()) {
      RecBucket b;
      b.m = M;
      bidx[M] = (int)p.buckets.size();
      p.buckets.push_back(b);
      it = bidx.find(M);
    }
    RecBucket& b = p.buckets[it->second];
    g.rec = it->second;
    g.slot0 = b.count;
    b.count += (int64_t)g.members.size();
    b.groups.push_back(gi);
  }
  layout(p);
  // fp32 buckets run with tiles of at most 128 (their epilogue staging of a
  // 256 x 256 fp32 tile would not fit in LDS)
  for (auto& b : p.buckets) b.tile = std::min(lookup(p.table, b.m, b.count).rec, b.f32 ? 128 : 256);
  for (auto& g : p.groups) {
    const TuneEntry& e = lookup(p.table, g.m, p.buckets[g.rec].count);
    const int cap = p.buckets[g.rec].f32 ? 128 : 256;
    g.tile_syrk = std::min(e.syrk, cap);
    g.tile_fin = std::min(e.fin, cap);
  }
  // fp32 MFMA runs at 1/16 of the 16-bit rate, so an fp32 launch with fewer
  // tiles than the GPU has CUs is bound by the time of one tile: with the
  // built-in table, such buckets halve their tiles (down to 64) until a
  // launch fills the GPU.  (One fp32 256 x 1024 matrix: 0.43 -> 0.17 ms per
  // step.)  A tune-table file is taken as given.
  if (p.table_source == "builtin") {
    constexpr int64_t kFillTiles = 256;
    auto lower_tiles = [](int64_t m, int t) {
      const int64_t nt = (m + t - 1) / t;
      return nt * (nt + 1) / 2;
    };
    for (auto& b : p.buckets) {
      if (!b.f32) continue;
      while (b.tile > 64 && lower_tiles(b.m, b.tile) * b.count < kFillTiles) b.tile /= 2;
    }
    for (auto& g : p.groups) {
      const RecBucket& b = p.buckets[g.rec];
      if (!b.f32) continue;
      const int64_t cnt = (int64_t)g.members.size();
      while (g.tile_syrk > 64 && lower_tiles(b.m, g.tile_syrk) * cnt < kFillTiles) g.tile_syrk /= 2;
      auto full_tiles = [&](int t) { return ((g.rows + t - 1) / t) * ((g.cols + t - 1) / t) * cnt; };
      while (g.tile_fin > 64 && full_tiles(g.tile_fin) < kFillTiles) g.tile_fin /= 2;
    }
  }
  // Lower-triangle storage of the states: every product that reads them
  // must run the direct-load ring (16-bit operands, whole tiles of 128 or
  // 256, 16-byte aligned rows), and every producer and consumer must use
  // the bucket's tile, so that "lower" means the same blocks for all.
  for (auto& b : p.buckets) {
    bool ok = p.storage_req == DMUON_STORAGE_AUTO && !b.f32 && !b.standard && (b.tile == 128 || b.tile == 256) &&
              b.m % b.tile == 0 && b.ldm % 8 == 0 && b.st_stride % 16 == 0;
    for (int gi : b.groups) {
      const Group& g = p.groups[gi];
      const int64_t xld = g.trans ? g.cols : g.xt_ld;        // the final product's X operand
      const int64_t xst = g.trans ? g.x_stride : g.xt_stride;
      ok = ok && g.tile_syrk == b.tile && g.tile_fin == b.tile && g.rows % b.tile == 0 && g.cols % b.tile == 0 &&
           xld % 8 == 0 && xst % 16 == 0;
    }
    b.lower = ok;
  }
  // Fused kernel: 16-bit Gram buckets of short side <= 128 whose members are
  // all stored rows <= cols (the kernel reads X's rows as stored)
  for (auto& b : p.buckets) {
    bool ok = p.fused_req != DMUON_FUSED_OFF && p.dtype == DMUON_BF16 && !b.f32 && !b.standard && b.m <= 128;
    for (int gi : b.groups) ok = ok && !p.groups[gi].trans;
    b.small = ok;
  }
  // Its split into two launches (recurrence, then the final product with one
  // workgroup per 128 output columns), for groups small enough that one
  // workgroup per matrix leaves CUs idle: under AUTO for short sides above
  // 64 and at most kSplitMax matrices; SPLIT asks for it always.
  for (auto& g : p.groups) {
    const RecBucket& b = p.buckets[g.rec];
    const int64_t n = (int64_t)g.members.size();
    g.split = b.small && (p.fused_req == DMUON_FUSED_SPLIT ||
                          (p.fused_req == DMUON_FUSED_AUTO && b.m > 64 && n <= kSplitMax));
    if (!g.split) continue;
    g.split_stride = (int64_t)round_up((size_t)small_split_bytes((int)g.rows), kAlign);
    g.split_off = round_up(p.ws_bytes, kAlign);
    p.ws_bytes = g.split_off + (size_t)g.split_stride * (size_t)std::min<int64_t>(n, kSmallMaxTab);
  }
  return DMUON_OK;
}

int load_table(PlanImpl& p, const char* path) {
  p.table = builtin_table();
  p.table_source = "builtin";
  if (!path || !*path) path = std::getenv("DMUON_TUNE_TABLE");
  if (!path || !*path) return DMUON_OK;
  FILE* f = std::fopen(path, "rb");
  if (!f) return fail(DMUON_EINVAL, "cannot open tune table '%s'", path);
  std::string text;
  char buf[4096];
  size_t k;
  while ((k = std::fread(buf, 1, sizeof buf, f)) > 0) text.append(buf, k);
  std::fclose(f);
  std::vector<TuneEntry> t;
  std::string err;
  if (!parse_tune_json(text, t, err)) return fail(DMUON_EINVAL, "tune table '%s': %s", path, err.c_str());
  p.table = t;
  p.table_source = path;
  return DMUON_OK;
}

// --------------------------------------------------------------------- execution
struct RunSpec {
  enum Mode { NS, STEP } mode = NS;
  int steps = 5;
  float a = 0, b = 0, c = 0;
  void* const* io = nullptr;             // NS: matrices (in place); STEP: params
  const void* const* grads = nullptr;    // STEP
  void* const* momenta = nullptr;        // STEP
  float lr = 0, wd = 0, mu = 0;
  int nesterov = 1;
};

// Arithmetic of one bucket.  F16 needs the fp16 range check of the
// recurrence to pass; AUTO falls back to BF16 when it does not.
int bucket_prec(const PlanImpl& p, const RecBucket& b, const RangeScan& r, Prec* out) {
  if (b.f32) {
    *out = Prec::F32;
    return DMUON_OK;
  }
  if (p.precision_req == DMUON_PREC_BF16) {
    *out = Prec::BF16;
    return DMUON_OK;
  }
  const bool ok = f16_range_ok(r, state_scale_for(b.m));
  if (!ok && p.precision_req == DMUON_PREC_F16)
    return fail(DMUON_EUNSUPPORTED, "the fp16 state would overflow, or Q's scale flush it, for these coefficients (m = %lld)",
                (long long)b.m);
  *out = ok ? Prec::F16 : Prec::BF16;
  return DMUON_OK;
}

GemmArgs gemm_args() {
  GemmArgs a{};
  for (auto& q : a.p) q.alpha = 1.0f;
  a.alpha_slot = -1;
  a.nprob = 1;
  return a;
}

MatRef ws_ref(char* ws, size_t off, int64_t stride, int64_t ld, int64_t first) {
  MatRef r{};
  r.base = ws + off + first * stride;
  r.stride = stride;
  r.ld = ld;
  r.tab = 0;
  return r;
}

// Collects independent problems of one kind into multi-problem launches: a
// launch takes up to kMaxProb problems that share the kernel instance and the
// launch-wide parameters, so that small groups fill the GPU together instead
// of leaving most of it idle one after the other.  Only problems with no
// dependence between them may be added between two flushes.
struct Batcher {
  hipStream_t st;
  bool open = false;
  Prec prec = Prec::F16;
  GemmKind kind = KIND_SYM_KK;
  int tile = 0;
  int ntab = 0;
  GemmArgs a{};
  explicit Batcher(hipStream_t s) : st(s) {}
  static bool same(const GemmArgs& x, const GemmArgs& y) {
    return x.alpha_slot == y.alpha_slot && x.c0 == y.c0 && x.c1 == y.c1 && x.c2 == y.c2 &&
           x.out_esize == y.out_esize && x.lower == y.lower;
  }
  hipError_t flush() {
    if (!open) return hipSuccess;
    open = false;
    // longest K first: every XCD starts with its most expensive tiles, the
    // cheap ones fill in behind them
    std::stable_sort(a.p, a.p + a.nprob, [](const GemmProb& x, const GemmProb& y) { return x.K > y.K; });
    return gemm(prec, kind, tile, a, st);
  }
  // `proto` carries the launch-wide fields and problem 0; its caller
  // pointers are proto.tab[0 .. batch) when a ref of problem 0 uses the table
  hipError_t add(Prec pr, GemmKind k, int t, const GemmArgs& proto) {
    const GemmProb& q = proto.p[0];
    const bool uses_tab = q.A.tab || q.B.tab || q.C.tab || q.D.tab;
    const int need = uses_tab ? q.batch : 0;
    if (open && (pr != prec || k != kind || t != tile || !same(a, proto) || a.nprob == kMaxProb ||
                 ntab + need > kMaxTab)) {
      hipError_t e = flush();
      if (e != hipSuccess) return e;
    }
    if (!open) {
      a = proto;
      a.nprob = 0;
      prec = pr;
      kind = k;
      tile = t;
      ntab = 0;
      open = true;
    }
    GemmProb qq = q;
    qq.tab0 = ntab;
    for (int i = 0; i < need; ++i) a.tab[ntab + i] = proto.tab[i];
    ntab += need;
    a.p[a.nprob++] = qq;
    return hipSuccess;
  }
};

// Zero rows [m, bucket size) of the copy the Gram product reads (rows of X),
// for every matrix of group g.  Inputs overwrite only the first m rows.
hipError_t zero_pad_rows(const PlanImpl& p, const RecBucket& b, const Group& g, char* ws, hipStream_t st) {
  (void)p;
  const int64_t pitch_bytes = g.trans ? g.xt_ld * 2 : g.cols * 2;
  char* base = ws + (g.trans ? g.xt_off : g.x_off);
  const int64_t stride = g.trans ? g.xt_stride : g.x_stride;
  const int64_t bytes = (b.m - g.m) * pitch_bytes;
  return timed("zero_bytes_kernel", 0.0, (double)bytes * g.members.size(), st,
               [&] { return launch_zero_bytes(base + g.m * pitch_bytes, stride, bytes, (int)g.members.size(), st); });
}

// Standard form on one bucket (16-bit), after the input pass, the scalars and
// the operand copies: X~ = X * input scale is held in two layouts, Xr (rows
// of X, m x n) and Xc (rows of X^T, n x m).  Each step:
//   A~ = s kappa^2 / sx^2 X~ X~^T            (symmetric product, lower tiles)
//   P' = (b / s) A~ + (c / s^2) A~^2          (polynomial product, c0 = 0)
//   X~ <- a X~ + P' X~                        (Xr in place, X~^T into the other Xc)
// and the result kappa / sx X~ is written (or applied as the update) in the
// caller's layout, which is Xr for wide matrices and Xc for tall ones.
int run_standard(const PlanImpl& p, const RecBucket& b, Prec prec, double sscale, char* ws, const RunSpec& rs,
                 hipStream_t st) {
  const int T = rs.steps;
  const int ie = elem_size(p.dtype);
  const bool f16 = prec == Prec::F16;
  char* scal_b = ws + b.scal_off;
  const int bt = b.tile;
  const int nt = (int)((b.m + bt - 1) / bt);
  auto st_ref = [&](int buf, int64_t first) { return ws_ref(ws, b.st_off[buf], b.st_stride, b.ldm, first); };
  // iterate buffers of group g: Xr and the two Xc buffers
  auto xr = [&](const Group& g) {
    return g.trans ? ws_ref(ws, g.xt_off, g.xt_stride, g.xt_ld, 0) : ws_ref(ws, g.x_off, g.x_stride, g.cols, 0);
  };
  auto xc = [&](const Group& g, int k) {  // Xc holding X~_k
    if (k % 2 == 0)
      return g.trans ? ws_ref(ws, g.x_off, g.x_stride, g.cols, 0) : ws_ref(ws, g.xt_off, g.xt_stride, g.xt_ld, 0);
    return ws_ref(ws, g.xt2_off, g.xt2_stride, g.xc_ld, 0);
  };
  Batcher batch(st);
  for (int k = 0; k < T; ++k) {
    for (int gi : b.groups) {
      const Group& g = p.groups[gi];
      float* scal_g = reinterpret_cast<float*>(scal_b) + g.slot0 * kScalStride;
      GemmArgs ga = gemm_args();
      GemmProb& q = ga.p[0];
      q.M = q.N = (int)b.m;
      q.K = (int)g.n;
      q.batch = (int)g.members.size();
      const int ts = g.tile_syrk;
      const int nts = (int)((b.m + ts - 1) / ts);
      q.tiles = nts * (nts + 1) / 2;
      q.tiles_n = nts;
      q.A = q.B = xr(g);
      q.C = st_ref(0, g.slot0);
      q.scal = scal_g;
      ga.alpha_slot = kSlotSyrkX;
      HIP_TRY(batch.add(prec, KIND_SYM_KK, ts, ga));
    }
    HIP_TRY(batch.flush());
    GemmArgs gp = gemm_args();
    GemmProb& qp = gp.p[0];
    qp.M = qp.N = qp.K = (int)b.m;
    qp.batch = (int)b.count;
    qp.tiles = nt * (nt + 1) / 2;
    qp.tiles_n = nt;
    qp.A = qp.B = qp.D = st_ref(0, 0);
    qp.C = st_ref(1, 0);
    gp.c0 = 0.0f;
    qp.pc1 = (float)(rs.b / sscale);
    qp.pc2 = (float)(rs.c / (sscale * sscale));
    HIP_TRY(gemm(prec, KIND_POLY, bt, gp, st));
    for (int gi : b.groups) {
      const Group& g = p.groups[gi];
      GemmArgs ga = gemm_args();
      GemmProb& q = ga.p[0];
      q.M = (int)g.m;
      q.N = (int)g.n;
      q.K = (int)g.m;
      q.batch = (int)g.members.size();
      const int ft = g.tile_fin;
      const int tm = (int)((g.m + ft - 1) / ft), tn = (int)((g.n + ft - 1) / ft);
      q.tiles = tm * tn;
      q.tiles_n = tn;
      q.A = st_ref(1, g.slot0);
      q.B = xc(g, k);
      q.D = xr(g);
      q.C = xc(g, k + 1);
      ga.c0 = rs.a;
      ga.c1 = 1.0f;
      HIP_TRY(batch.add(prec, KIND_AXPY_KK, ft, ga));
    }
    HIP_TRY(batch.flush());
  }
  // result in the caller's layout
  for (int gi : b.groups) {
    const Group& g = p.groups[gi];
    float* scal_g = reinterpret_cast<float*>(scal_b) + g.slot0 * kScalStride;
    const MatRef src = g.trans ? xc(g, T) : xr(g);
    if (src.ld != g.cols) return fail(DMUON_EUNSUPPORTED, "internal: padded result layout");
    const float shape = (p.scale_mode == DMUON_SCALE_NONE)
                            ? 1.0f
                            : (float)std::sqrt(std::max(1.0, (double)g.rows / (double)g.cols));
    const size_t cnt = g.members.size();
    for (size_t s0 = 0; s0 < cnt; s0 += kMaxTab) {
      const size_t s1 = std::min(cnt, s0 + kMaxTab);
      ScaleOutArgs so{};
      for (size_t i = s0; i < s1; ++i) so.out[i - s0] = reinterpret_cast<uint64_t>(rs.io[g.members[i]]);
      so.src_base = static_cast<const char*>(src.base) + (int64_t)s0 * src.stride;
      so.src_stride = src.stride;
      so.elems = g.rows * g.cols;
      so.esize = 2;
      so.out_esize = ie;
      so.update = rs.mode == RunSpec::STEP;
      so.src_f16 = f16 ? 1 : 0;
      so.slot = kSlotFinal;
      so.scal = scal_g + s0 * kScalStride;
      so.c0 = 1.0f - rs.lr * rs.wd;
      so.c1 = -rs.lr * shape;
      const double sb = (double)(s1 - s0) * so.elems * (2.0 + ie * (so.update ? 2.0 : 1.0));
      HIP_TRY(timed(std::string("scale_out_kernel<2, ") + std::to_string(ie) + ">", 0.0, sb, st,
                    [&] { return launch_scale_out(so, (int)(s1 - s0), st); }));
    }
  }
  return DMUON_OK;
}

// Momentum of members [s0, s1) of group g: buf <- mu buf + G and u (Nesterov
// or not) into the workspace copy of X, with partial sums of u^2.
int momentum_pass(const PlanImpl& p, const Group& g, int ce, char* ws, const RunSpec& rs, size_t s0, size_t s1,
                  hipStream_t st) {
  const int ie = elem_size(p.dtype);
  const int64_t elems = g.rows * g.cols;
  MomentumArgs ma{};
  bool vec = true;
  for (size_t i = s0; i < s1; ++i) {
    const void* gp = rs.grads[g.members[i]];
    const void* bp = rs.momenta[g.members[i]];
    ma.g[i - s0] = reinterpret_cast<uint64_t>(gp);
    ma.buf[i - s0] = reinterpret_cast<uint64_t>(bp);
    vec = vec && ((reinterpret_cast<uintptr_t>(gp) & 15) == 0) && ((reinterpret_cast<uintptr_t>(bp) & 15) == 0);
  }
  ma.u_base = ws + g.x_off + s0 * g.x_stride;
  ma.u_stride = g.x_stride;
  ma.elems = elems;
  ma.esize = ie;
  ma.u_esize = ce;
  ma.nblk = g.nblk;
  ma.nesterov = rs.nesterov;
  ma.vec_ok = vec;
  ma.mu = rs.mu;
  ma.partial = reinterpret_cast<double*>(ws + g.part_off) + s0 * g.nblk;
  const double mb = (double)(s1 - s0) * elems * (ie + ce + 8.0);
  HIP_TRY(timed(std::string("momentum_kernel<") + std::to_string(ie) + ", " + std::to_string(ce) + ">", 0.0, mb,
                st, [&] { return launch_momentum(ma, (int)(s1 - s0), st); }));
  return DMUON_OK;
}

// Whether bucket b runs the fused kernel for this precision and step count.
bool runs_small(const RecBucket& b, Prec prec, int steps) {
  return b.small && prec == Prec::F16 && steps >= 1 && steps <= kSmallMaxSteps;
}

// A whole 16-bit Gram bucket of short side <= 128 in one fused launch per
// group (per kSmallMaxTab members, enough to fill the GPU): NS mode reads and
// overwrites the caller's matrices; step mode first runs the momentum pass
// (per kMaxTab members) into the workspace copy and then applies the update
// to the parameters.
int run_small(const PlanImpl& p, const RecBucket& b, double sscale, const std::vector<int>& qe, char* ws,
              const RunSpec& rs, hipStream_t st) {
  const int T = rs.steps;
  for (int gi : b.groups) {
    const Group& g = p.groups[gi];
    const float shape = (p.scale_mode == DMUON_SCALE_NONE)
                            ? 1.0f
                            : (float)std::sqrt(std::max(1.0, (double)g.rows / (double)g.cols));
    const size_t cnt = g.members.size();
    for (size_t s0 = 0; s0 < cnt; s0 += kSmallMaxTab) {
      const size_t s1 = std::min(cnt, s0 + (size_t)kSmallMaxTab);
      SmallArgs sa{};
      sa.rows = (int32_t)g.rows;
      sa.cols = (int32_t)g.cols;
      sa.steps = T;
      sa.a = rs.a;
      sa.b1 = (float)(rs.b / sscale);
      sa.c2 = (float)(rs.c / (sscale * sscale));
      sa.sscale = (float)sscale;
      sa.eps = (float)p.eps;
      for (int k = 0; k < T; ++k) sa.qmul[k] = (float)std::ldexp(1.0, qe[k] - qe[k + 1]);
      const float qfin = (float)std::ldexp(1.0, qe[T]);
      if (rs.mode == RunSpec::STEP) {
        for (size_t m0 = s0; m0 < s1; m0 += kMaxTab) {
          int e = momentum_pass(p, g, 2, ws, rs, m0, std::min(s1, m0 + (size_t)kMaxTab), st);
          if (e != DMUON_OK) return e;
        }
        sa.x_base = ws + g.x_off + s0 * g.x_stride;
        sa.x_stride = g.x_stride;
        sa.update = 1;
        sa.c0 = 1.0f - rs.lr * rs.wd;
        sa.c1 = -rs.lr;
        sa.ofac = qfin * shape;
      } else {
        sa.x_base = nullptr;
        sa.update = 0;
        sa.ofac = qfin;
      }
      for (size_t i = s0; i < s1; ++i) sa.tab[i - s0] = reinterpret_cast<uint64_t>(rs.io[g.members[i]]);
      const double m = (double)g.m, n = (double)g.n;
      const double nm = (double)(s1 - s0);
      const double f_gram = nm * m * (m + 1) * n, f_rec = nm * (4.0 * T - 3.0) * m * m * (m + 1),
                   f_fin = nm * 2 * m * m * n;
      const int nmat = (int)(s1 - s0);
      if (!g.split) {
        const char* name = g.m <= 64 ? "small_ns_kernel<64>" : "small_ns_kernel<128>";
        HIP_TRY(timed(name, f_gram + f_rec + f_fin, 0.0, st,
                      [&] { return launch_small_ns(sa, nmat, SMALL_ONE, st); }));
        continue;
      }
      // two launches: the Gram product and the recurrence, then the final
      // product per 128 columns
      sa.split_base = ws + g.split_off;
      sa.split_stride = g.split_stride;
      const std::string mp = g.m <= 64 ? "64" : "128";
      HIP_TRY(timed("small_ns_kernel<" + mp + ">:rec", f_gram + f_rec, 0.0, st,
                    [&] { return launch_small_ns(sa, nmat, SMALL_REC, st); }));
      HIP_TRY(timed("small_ns_kernel<" + mp + ">:final", f_fin, 0.0, st,
                    [&] { return launch_small_ns(sa, nmat, SMALL_FINAL, st); }));
    }
  }
  return DMUON_OK;
}

int run(const PlanImpl& p, char* ws, const RunSpec& rs, hipStream_t st) {
  const int ie = elem_size(p.dtype);
  const int T = rs.steps;
  const RangeScan range = scan_recurrence(rs.a, rs.b, rs.c, T);
  // validate every bucket before anything is enqueued
  std::vector<Prec> precs(p.buckets.size());
  for (size_t i = 0; i < p.buckets.size(); ++i) {
    int e = bucket_prec(p, p.buckets[i], range, &precs[i]);
    if (e != DMUON_OK) return e;
  }

  auto chunks = [](size_t n, auto&& fn) -> int {
    for (size_t s = 0; s < n; s += kMaxTab) {
      int e = fn(s, std::min(n, s + kMaxTab));
      if (e != DMUON_OK) return e;
    }
    return DMUON_OK;
  };

  std::vector<int> pend;  // buckets whose Gram-space recurrence is still to run
  for (size_t bi = 0; bi < p.buckets.size(); ++bi) {
    const RecBucket& b = p.buckets[bi];
    const Prec prec = precs[bi];
    const bool f16 = prec == Prec::F16;
    const int ce = b.f32 ? 4 : 2;  // element size of the workspace input copy
    const double sscale = f16 ? state_scale_for(b.m) : 1.0;
    const std::vector<int> qe = f16 ? q_exponents(range) : std::vector<int>(T + 1, 0);
    if (runs_small(b, prec, T)) {
      int e = run_small(p, b, sscale, qe, ws, rs, st);
      if (e != DMUON_OK) return e;
      continue;
    }
    char* scal_b = ws + b.scal_off;
    // ---- per group: input pass, scalars, Gram product
    for (int gi : b.groups) {
      const Group& g = p.groups[gi];
      const size_t cnt = g.members.size();
      const int64_t elems = g.rows * g.cols;
      float* scal_g = reinterpret_cast<float*>(scal_b) + g.slot0 * kScalStride;
      double* part = reinterpret_cast<double*>(ws + g.part_off);
      int e = chunks(cnt, [&](size_t s0, size_t s1) -> int {
        if (rs.mode == RunSpec::NS) {
          NormArgs na{};
          bool vec = true;
          for (size_t i = s0; i < s1; ++i) {
            const void* ptr = rs.io[g.members[i]];
            na.tab[i - s0] = reinterpret_cast<uint64_t>(ptr);
            vec = vec && ((reinterpret_cast<uintptr_t>(ptr) & 15) == 0);
          }
          na.copy_base = ws + g.x_off + s0 * g.x_stride;
          na.copy_stride = g.x_stride;
          na.elems = elems;
          na.esize = ie;
          na.copy_esize = ce;
          na.nblk = g.nblk;
          na.vec_ok = vec;
          na.partial = part + s0 * g.nblk;
          const double nb = (double)(s1 - s0) * elems * (ie + ce);
          HIP_TRY(timed(std::string("norm_copy_kernel<") + std::to_string(ie) + ", " + std::to_string(ce) + ">",
                        0.0, nb, st,
                        [&] { return launch_norm_copy(na, (int)(s1 - s0), st); }));
        } else {
          int e = momentum_pass(p, g, ce, ws, rs, s0, s1, st);
          if (e != DMUON_OK) return e;
        }
        return DMUON_OK;
      });
      if (e != DMUON_OK) return e;
      FinalizeArgs fa{};
      fa.partial = part;
      fa.nblk = g.nblk;
      fa.scal = scal_g;
      fa.eps = (float)p.eps;
      fa.state_scale = (float)sscale;
      fa.f16_inputs = f16 ? 1 : 0;
      HIP_TRY(timed("finalize_kernel", 0.0, (double)cnt * g.nblk * 8.0, st,
                    [&] { return launch_finalize(fa, (int)cnt, st); }));

      if (T == 0) continue;
      if (!b.f32) {
        // row-contiguous operands for both products: X for the Gram product,
        // X^T (scaled fp16 on the fp16 path) for the final one
        PrepArgs pa{};
        pa.src_base = ws + g.x_off;
        pa.src_stride = g.x_stride;
        pa.t_base = ws + g.xt_off;
        pa.t_stride = g.xt_stride;
        pa.t_ld = g.xt_ld;
        pa.rows = (int32_t)g.rows;
        pa.cols = (int32_t)g.cols;
        // standard form: both layouts are iterates, so both are converted
        pa.t_f16 = (f16 && (!g.trans || b.standard)) ? 1 : 0;
        pa.s_f16 = (f16 && (g.trans || b.standard)) ? 1 : 0;
        pa.scal = scal_g;
        const double pb = (double)cnt * elems * (pa.s_f16 ? 8.0 : 4.0);
        HIP_TRY(timed("prep_kernel", 0.0, pb, st, [&] { return launch_prep(pa, (int)cnt, st); }));
      }
      if (b.m > g.m) HIP_TRY(zero_pad_rows(p, b, g, ws, st));
    }
    // ---- Gram products of all groups, batched into multi-problem launches
    if (T > 0 && !b.standard) {  // standard-form Gram products run inside the iteration
      Batcher batch(st);
      for (int gi : b.groups) {
        const Group& g = p.groups[gi];
        float* scal_g = reinterpret_cast<float*>(scal_b) + g.slot0 * kScalStride;
        GemmArgs ga = gemm_args();
        GemmProb& q = ga.p[0];
        q.M = q.N = (int)b.m;  // padded rows of X are zero, so the padded state is too
        q.K = (int)g.n;
        q.batch = (int)g.members.size();
        const int bt = g.tile_syrk;
        const int nt = (int)((b.m + bt - 1) / bt);
        q.tiles = nt * (nt + 1) / 2;
        q.tiles_n = nt;
        GemmKind sk = KIND_SYRK_KK;
        if (b.f32)
          q.A = ws_ref(ws, g.x_off, g.x_stride, g.cols, 0), sk = g.trans ? KIND_SYRK_MM : KIND_SYRK_KK;
        else if (g.trans)
          q.A = ws_ref(ws, g.xt_off, g.xt_stride, g.xt_ld, 0);  // X = the transpose of the caller layout
        else
          q.A = ws_ref(ws, g.x_off, g.x_stride, g.cols, 0);
        q.B = q.A;
        q.C = ws_ref(ws, b.st_off[0], b.st_stride, b.ldm, g.slot0);
        q.scal = scal_g;
        ga.alpha_slot = kSlotSyrk;
        if (b.lower) ga.lower = kLowerOut;
        HIP_TRY(batch.add(prec, sk, bt, ga));
      }
      HIP_TRY(batch.flush());
    }

    // ---- standard form: T steps on the m x n iterates
    if (T > 0 && b.standard) {
      int e = run_standard(p, b, prec, sscale, ws, rs, st);
      if (e != DMUON_OK) return e;
      continue;
    }
    // ---- m x m recurrence: deferred, so that the buckets that share a
    // kernel instance run their steps in lockstep and share launches
    if (T > 0) {
      pend.push_back(bi);
      continue;
    }
    // ---- zero steps: the normalised input itself
    for (int gi : b.groups) {
      const Group& g = p.groups[gi];
      float* scal_g = reinterpret_cast<float*>(scal_b) + g.slot0 * kScalStride;
      const float shape = (p.scale_mode == DMUON_SCALE_NONE)
                              ? 1.0f
                              : (float)std::sqrt(std::max(1.0, (double)g.rows / (double)g.cols));
      int e = chunks(g.members.size(), [&](size_t s0, size_t s1) -> int {
        ScaleOutArgs so{};
        for (size_t i = s0; i < s1; ++i) so.out[i - s0] = reinterpret_cast<uint64_t>(rs.io[g.members[i]]);
        so.src_base = ws + g.x_off + s0 * g.x_stride;
        so.src_stride = g.x_stride;
        so.elems = g.rows * g.cols;
        so.esize = ce;
        so.out_esize = ie;
        so.update = rs.mode == RunSpec::STEP;
        so.slot = kSlotKappa;
        so.src_f16 = 0;
        so.scal = scal_g + s0 * kScalStride;
        so.c0 = 1.0f - rs.lr * rs.wd;
        so.c1 = -rs.lr * shape;
        const double sb = (double)(s1 - s0) * so.elems * (ce + ie * (so.update ? 2.0 : 1.0));
        HIP_TRY(timed(std::string("scale_out_kernel<") + std::to_string(ce) + ", " + std::to_string(ie) + ">",
                      0.0, sb, st,
                      [&] { return launch_scale_out(so, (int)(s1 - s0), st); }));
        return DMUON_OK;
      });
      if (e != DMUON_OK) return e;
    }
  }
  if (pend.empty()) return DMUON_OK;

  // ---- recurrences.  Buckets with the same arithmetic, tile and storage run
  // each phase of a step together: their products go to one Batcher, which
  // packs up to kMaxProb of them per launch (longest K first), so that one
  // bucket's tiles fill the last, partial round of another's.
  enum { AT = 0, PB = 1, RB = 2, QA = 3, QB = 4 };
  std::vector<int> qcur(p.buckets.size(), QA);
  std::vector<std::vector<int>> rgroups;
  for (int bi : pend) {
    const RecBucket& b = p.buckets[bi];
    bool placed = false;
    for (auto& grp : rgroups) {
      const RecBucket& b0 = p.buckets[grp[0]];
      if (precs[grp[0]] == precs[bi] && b0.tile == b.tile && b0.lower == b.lower && b0.f32 == b.f32) {
        grp.push_back(bi);
        placed = true;
        break;
      }
    }
    if (!placed) rgroups.push_back({bi});
  }
  auto ref = [&](const RecBucket& b, int buf) { return ws_ref(ws, b.st_off[buf], b.st_stride, b.ldm, 0); };
  auto square = [&](const RecBucket& b, GemmProb& q) {
    const int nt = (int)((b.m + b.tile - 1) / b.tile);
    q.M = q.N = q.K = (int)b.m;
    q.batch = (int)b.count;
    q.tiles = nt * (nt + 1) / 2;
    q.tiles_n = nt;
  };
  for (const auto& grp : rgroups) {
    const Prec prec = precs[grp[0]];
    const bool f16 = prec == Prec::F16;
    const std::vector<int> qe = f16 ? q_exponents(range) : std::vector<int>(T + 1, 0);
    const int bt = p.buckets[grp[0]].tile;
    // symmetric products: both operands and the output stored lower
    const int32_t sym_lower = p.buckets[grp[0]].lower ? (kLowerA | kLowerB | kLowerOut) : 0;
    for (int k = 0; k < T; ++k) {
      const int pk = (k == 0) ? QA : PB;  // P0 is Q1 itself
      const bool need_a = k < T - 1;
      const bool need_q = k >= 1;
      // P = a I + b A + c A^2 with A~ = s A stored: a I + (b/s) A~ + (c/s^2) A~^2
      Batcher bp(st);
      for (int bi : grp) {
        const RecBucket& b = p.buckets[bi];
        const double sscale = f16 ? state_scale_for(b.m) : 1.0;
        GemmArgs ga = gemm_args();
        GemmProb& q = ga.p[0];
        square(b, q);
        q.A = q.B = q.D = ref(b, AT);
        q.C = ref(b, pk);
        q.pc1 = (float)(rs.b / sscale);
        q.pc2 = (float)(rs.c / (sscale * sscale));
        ga.c0 = rs.a;
        ga.lower = sym_lower;
        HIP_TRY(bp.add(prec, KIND_POLY, bt, ga));
      }
      HIP_TRY(bp.flush());
      // R~ = P A~ and Q_{k+1} = P_k Q_k (stored divided by 2^e_{k+1})
      if (need_a || need_q) {
        Batcher br(st);
        const float qmul = (float)std::ldexp(1.0, qe[k] - qe[k + 1]);
        for (int bi : grp) {
          const RecBucket& b = p.buckets[bi];
          GemmArgs ga = gemm_args();
          GemmProb& q = ga.p[0];
          square(b, q);
          ga.lower = sym_lower;
          q.A = ref(b, pk);
          if (need_a) {
            q.B = ref(b, AT);
            q.C = ref(b, RB);
            HIP_TRY(br.add(prec, KIND_SYM_KK, bt, ga));
          }
          if (need_q) {
            q.B = ref(b, qcur[bi]);
            q.C = ref(b, qcur[bi] == QA ? QB : QA);
            q.alpha = qmul;
            HIP_TRY(br.add(prec, KIND_SYM_KK, bt, ga));
          }
        }
        HIP_TRY(br.flush());
        if (need_q)
          for (int bi : grp) qcur[bi] = (qcur[bi] == QA) ? QB : QA;
      }
      // A~ = R~ P
      if (need_a) {
        Batcher ba(st);
        for (int bi : grp) {
          const RecBucket& b = p.buckets[bi];
          GemmArgs ga = gemm_args();
          GemmProb& q = ga.p[0];
          square(b, q);
          q.A = ref(b, RB);
          q.B = ref(b, pk);
          q.C = ref(b, AT);
          ga.lower = sym_lower;
          HIP_TRY(ba.add(prec, KIND_SYM_KK, bt, ga));
        }
        HIP_TRY(ba.flush());
      }
    }
  }

  // ---- final products of every bucket, batched into multi-problem launches
  Batcher batch(st);
  for (int bi : pend) {
    const RecBucket& b = p.buckets[bi];
    const Prec prec = precs[bi];
    const bool f16 = prec == Prec::F16;
    const std::vector<int> qe = f16 ? q_exponents(range) : std::vector<int>(T + 1, 0);
    char* scal_b = ws + b.scal_off;
    for (int gi : b.groups) {
      const Group& g = p.groups[gi];
      float* scal_g = reinterpret_cast<float*>(scal_b) + g.slot0 * kScalStride;
      const float shape = (p.scale_mode == DMUON_SCALE_NONE)
                              ? 1.0f
                              : (float)std::sqrt(std::max(1.0, (double)g.rows / (double)g.cols));
      int e = chunks(g.members.size(), [&](size_t s0, size_t s1) -> int {
        GemmArgs ga = gemm_args();
        GemmProb& q = ga.p[0];
        q.M = (int)g.rows;
        q.N = (int)g.cols;
        q.K = (int)g.m;
        q.batch = (int)(s1 - s0);
        ga.out_esize = ie;
        // undo the scale of Q_T; the update's shape factor rides along, so
        // that every group of the bucket shares the launch-wide c1 = -lr
        q.alpha = (float)std::ldexp(1.0, qe[T]) * (rs.mode == RunSpec::NS ? 1.0f : shape);
        const int ft = g.tile_fin;
        const int tm = (int)((g.rows + ft - 1) / ft), tn = (int)((g.cols + ft - 1) / ft);
        q.tiles = tm * tn;
        q.tiles_n = tn;
        MatRef xr = ws_ref(ws, g.x_off, g.x_stride, g.cols, (int64_t)s0);
        MatRef qr = ws_ref(ws, b.st_off[qcur[bi]], b.st_stride, b.ldm, g.slot0 + (int64_t)s0);
        const bool rowx = !b.f32 && !g.trans;  // X^T copy available
        if (rowx) xr = ws_ref(ws, g.xt_off, g.xt_stride, g.xt_ld, (int64_t)s0);
        if (!g.trans) {  // O = Q X: A = Q, B = X^T (16-bit) or X read N-contiguous (fp32)
          q.A = qr;
          q.B = xr;
          if (b.lower) ga.lower = kLowerA;
        } else {  // O^T = X^T Q in the caller layout: A = the caller-layout copy, B = Q
          q.A = xr;
          q.B = qr;
          if (b.lower) ga.lower = kLowerB;
        }
        MatRef out{};
        out.tab = 1;
        out.ld = g.cols;
        for (size_t i = s0; i < s1; ++i) ga.tab[i - s0] = reinterpret_cast<uint64_t>(rs.io[g.members[i]]);
        q.scal = scal_g + s0 * kScalStride;
        ga.alpha_slot = kSlotFinal;
        GemmKind kind;
        const bool kk = g.trans || rowx;
        if (rs.mode == RunSpec::NS) {
          q.C = out;
          kind = kk ? KIND_OUT_KK : KIND_OUT_KM;
        } else {
          q.D = out;
          ga.c0 = 1.0f - rs.lr * rs.wd;
          ga.c1 = -rs.lr;
          kind = kk ? KIND_UPD_KK : KIND_UPD_KM;
        }
        HIP_TRY(batch.add(prec, kind, ft, ga));
        return DMUON_OK;
      });
      if (e != DMUON_OK) return e;
    }
  }
  HIP_TRY(batch.flush());
  return DMUON_OK;
}

// --------------------------------------------------------------------- implicit workspace
// One growing workspace per device serves every plan-free call.  A buffer it
// outgrows is retired, not freed: enqueued work, or a HIP graph that captured
// an earlier call, may still address it.  Retired buffers are freed only by
// dmuon_release_workspace (or at process exit).  Growth is geometric (at
// least 1.5 x), so the retired buffers together stay below twice the live one.
struct DeviceCache {
  char* ws = nullptr;
  size_t bytes = 0;
  std::vector<std::pair<char*, size_t>> retired;
  std::map<std::tuple<int64_t, int64_t, int64_t, int>, PlanImpl> plans;
};
std::mutex g_cache_mu;
std::map<int, DeviceCache> g_cache;

// Debug aid (environment variable DMUON_POISON_WORKSPACE=1): fill every new
// device workspace with 0xFF bytes, a NaN in fp32, fp16 and bf16, so that a
// read of workspace memory no kernel has written (for instance the upper
// triangle of a lower-stored state) turns the results into NaN.  The fill is
// a synchronous hipMemset at allocation time.
bool poison_workspace() {
  const char* v = std::getenv("DMUON_POISON_WORKSPACE");
  return v && *v && std::strcmp(v, "0") != 0;
}

int alloc_workspace(size_t bytes, char** out) {
  void* p = nullptr;
  hipError_t e = hipMalloc(&p, bytes ? bytes : 1);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(DMUON_ENOMEM, "workspace of %zu bytes: %s", bytes, hipGetErrorString(e));
  }
  if (poison_workspace() && bytes) {
    e = hipMemset(p, 0xFF, bytes);
    if (e != hipSuccess) {
      (void)hipFree(p);
      return fail(DMUON_EHIP, "poisoning the workspace: %s", hipGetErrorString(e));
    }
  }
  *out = static_cast<char*>(p);
  return DMUON_OK;
}

int ensure_workspace(DeviceCache& dc, size_t need, hipStream_t st) {
  if (dc.bytes >= need && dc.ws) return DMUON_OK;
  // a graph being captured on the caller's stream would record kernels that
  // address a buffer allocated in the middle of the capture: grow outside it
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (st && hipStreamIsCapturing(st, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone)
    return fail(DMUON_EUNSUPPORTED,
                "the implicit workspace must grow to %zu bytes while the stream is being captured: make one "
                "call of the same shape outside the capture first, or use a plan",
                need);
  const size_t grow = dc.bytes + dc.bytes / 2;
  const size_t bytes = round_up(std::max(need, grow), kAlign);
  char* p = nullptr;
  int e = alloc_workspace(bytes, &p);
  if (e != DMUON_OK) return e;
  if (dc.ws) dc.retired.push_back({dc.ws, dc.bytes});
  dc.ws = p;
  dc.bytes = bytes;
  return DMUON_OK;
}


std::string describe_plan(const PlanImpl& p) {
  std::string s;
  char tmp[256];
  auto add = [&](const char* fmt, auto... args) {
    snprintf(tmp, sizeof tmp, fmt, args...);
    s += tmp;
  };
  add("{\"count\": %lld, \"dtype\": \"%s\", \"precision\": %d, \"scale_mode\": %d, \"eps\": %.9g, ",
      (long long)p.count, p.dtype == DMUON_F32 ? "f32" : "bf16", p.precision_req, p.scale_mode, p.eps);
  add("\"device\": %s, \"workspace_bytes\": %zu, \"tune_table\": \"", p.device ? "true" : "false", p.ws_bytes);
  for (char ch : p.table_source) {
    if (ch == '"' || ch == '\\') s += '\\';
    s += ch;
  }
  s += "\", \"gemm\": [";
  for (size_t i = 0; i < p.groups.size(); ++i) {
    const Group& g = p.groups[i];
    const int nt = (int)((g.m + g.tile_syrk - 1) / g.tile_syrk);
    add("%s{\"rows\": %lld, \"cols\": %lld, \"m\": %lld, \"n\": %lld, \"transposed\": %s, \"rec\": %d, "
        "\"tile_syrk\": %d, \"tile_final\": %d, \"syrk_tiles\": %d, \"split\": %s, \"members\": [",
        i ? ", " : "", (long long)g.rows, (long long)g.cols, (long long)g.m, (long long)g.n,
        g.trans ? "true" : "false", g.rec, g.tile_syrk, g.tile_fin, nt * (nt + 1) / 2, g.split ? "true" : "false");
    for (size_t j = 0; j < g.members.size(); ++j) add("%s%lld", j ? ", " : "", (long long)g.members[j]);
    s += "]}";
  }
  s += "], \"recurrence\": [";
  for (size_t i = 0; i < p.buckets.size(); ++i) {
    const RecBucket& b = p.buckets[i];
    const int nt = (int)((b.m + b.tile - 1) / b.tile);
    add("%s{\"m\": %lld, \"count\": %lld, \"tile\": %d, \"lower_tiles\": %d, \"fp32\": %s, \"form\": \"%s\", "
        "\"storage\": \"%s\", \"fused\": %s, \"members\": [",
        i ? ", " : "", (long long)b.m, (long long)b.count, b.tile, nt * (nt + 1) / 2, b.f32 ? "true" : "false",
        b.standard ? "standard" : "gram", b.lower ? "lower" : "full", b.small ? "true" : "false");
    bool first = true;
    for (int gi : b.groups)
      for (int64_t mbr : p.groups[gi].members) {
        add("%s%lld", first ? "" : ", ", (long long)mbr);
        first = false;
      }
    s += "]}";
  }
  s += "]}";
  return s;
}

// DMUON_LOG set (and not "0"): print each new plan's description to stderr.
void log_plan(const char* what, const PlanImpl& p) {
  const char* v = std::getenv("DMUON_LOG");
  if (!v || !*v || std::strcmp(v, "0") == 0) return;
  std::fprintf(stderr, "dmuon %s: %s\n", what, describe_plan(p).c_str());
}


int check_coeffs(int steps, float a, float b, float c) {
  if (steps < 0) return fail(DMUON_EINVAL, "steps must be >= 0 (got %d)", steps);
  if (!std::isfinite(a) || !std::isfinite(b) || !std::isfinite(c))
    return fail(DMUON_EINVAL, "coefficients must be finite");
  return DMUON_OK;
}

// noalloc: run in the statically allocated device scratch instead of the
// implicit workspace (no hipMalloc, hipFree or synchronisation on any path)
int ns_batched_impl(void* const* ptrs, int64_t m, int64_t n, int64_t batch, int dtype, int precision,
                    int steps, float a, float b, float c, void* stream, bool noalloc = false) {
  if (!ptrs) return fail(DMUON_EINVAL, "ptrs is NULL");
  if (m <= 0 || n <= 0) return fail(DMUON_EINVAL, "m and n must be positive (got %lld x %lld)", (long long)m, (long long)n);
  if (batch <= 0) return fail(DMUON_EINVAL, "batch must be positive (got %lld)", (long long)batch);
  if (m > (1 << 30) / 1 || n > (1 << 30) || m * n > ((int64_t)1 << 40))
    return fail(DMUON_EINVAL, "matrix too large");
  if (dtype != DMUON_BF16 && dtype != DMUON_F32) return fail(DMUON_EINVAL, "unknown dtype %d", dtype);
  if (precision < DMUON_PREC_AUTO || precision > DMUON_PREC_F32)
    return fail(DMUON_EINVAL, "unknown precision %d", precision);
  int e = check_coeffs(steps, a, b, c);
  if (e) return e;
  for (int64_t i = 0; i < batch; ++i)
    if (!ptrs[i]) return fail(DMUON_EINVAL, "ptrs[%lld] is NULL", (long long)i);
  if (dtype == DMUON_F32 && precision != DMUON_PREC_AUTO && precision != DMUON_PREC_F32)
    return fail(DMUON_EUNSUPPORTED, "f32 matrices run on the fp32 path only (precision %d)", precision);
  if (precision == DMUON_PREC_F16 &&
      !f16_range_ok(scan_recurrence(a, b, c, steps), state_scale_for(std::min(m, n))))
    return fail(DMUON_EUNSUPPORTED, "the fp16 state would overflow, or Q's scale flush it, for these coefficients");

  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lock(g_cache_mu);
  DeviceCache& dc = g_cache[dev];
  auto key = std::make_tuple(m, n, batch, dtype * 16 + precision);
  auto it = dc.plans.find(key);
  if (it == dc.plans.end()) {
    PlanImpl p;
    p.dtype = dtype;
    p.precision_req = precision;
    p.device = true;
    p.device_id = dev;
    e = load_table(p, nullptr);
    if (e) return e;
    std::vector<int64_t> rows(batch, m), cols(batch, n);
    build_plan(p, rows.data(), cols.data(), batch);
    log_plan("implicit plan", p);
    if (dc.plans.size() > 64) dc.plans.clear();
    it = dc.plans.emplace(key, std::move(p)).first;
  }
  char* ws = nullptr;
  if (noalloc) {
    if (it->second.ws_bytes > kScratchBytes)
      return fail(DMUON_ENOMEM,
                  "%lld matrices of %lld x %lld need %zu bytes of workspace; the allocation-free scratch holds "
                  "%zu",
                  (long long)batch, (long long)m, (long long)n, it->second.ws_bytes, kScratchBytes);
    HIP_TRY(scratch_address(&ws));
  } else {
    e = ensure_workspace(dc, it->second.ws_bytes, static_cast<hipStream_t>(stream));
    if (e) return e;
    ws = dc.ws;
  }
  RunSpec rs;
  rs.mode = RunSpec::NS;
  rs.steps = steps;
  rs.a = a;
  rs.b = b;
  rs.c = c;
  rs.io = ptrs;
  return run(it->second, ws, rs, static_cast<hipStream_t>(stream));
}


}  // namespace
}  // namespace dmuon

using dmuon::PlanImpl;
struct dmuon_plan {
  PlanImpl impl;
};

extern "C" {

int dmuon_ns_batched(void* const* ptrs, int64_t m, int64_t n, int64_t batch, int steps, float a,
                     float b, float c, void* stream) {
  try {
    return dmuon::ns_batched_impl(ptrs, m, n, batch, DMUON_BF16, DMUON_PREC_AUTO, steps, a, b, c, stream);
  } catch (...) {
    return dmuon::fail(DMUON_ENOMEM, "host allocation failed");
  }
}

int dmuon_ns_batched_f32(void* const* ptrs, int64_t m, int64_t n, int64_t batch, int steps, float a,
                         float b, float c, void* stream) {
  try {
    return dmuon::ns_batched_impl(ptrs, m, n, batch, DMUON_F32, DMUON_PREC_F32, steps, a, b, c, stream);
  } catch (...) {
    return dmuon::fail(DMUON_ENOMEM, "host allocation failed");
  }
}

int dmuon_ns_batched_ex(void* const* ptrs, int64_t m, int64_t n, int64_t batch, int dtype, int precision,
                        int steps, float a, float b, float c, void* stream) {
  try {
    return dmuon::ns_batched_impl(ptrs, m, n, batch, dtype, precision, steps, a, b, c, stream);
  } catch (...) {
    return dmuon::fail(DMUON_ENOMEM, "host allocation failed");
  }
}

int dmuon_ns_batched_noalloc(void* const* ptrs, int64_t m, int64_t n, int64_t batch, int steps, float a,
                             float b, float c, void* stream) {
  try {
    return dmuon::ns_batched_impl(ptrs, m, n, batch, DMUON_BF16, DMUON_PREC_AUTO, steps, a, b, c, stream, true);
  } catch (...) {
    return dmuon::fail(DMUON_ENOMEM, "host allocation failed");
  }
}

void dmuon_plan_opts_default(dmuon_plan_opts* o) {
  if (!o) return;
  std::memset(o, 0, sizeof *o);
  o->precision = DMUON_PREC_AUTO;
  o->scale_mode = DMUON_SCALE_SQRT_RATIO;
  o->no_device = 0;
  o->eps = (float)dmuon::kDefaultEps;
  o->max_workspace = 0;
  o->tune_path = nullptr;
  o->form = DMUON_FORM_AUTO;
  o->pad_ratio = 0.0f;
  o->storage = DMUON_STORAGE_AUTO;
  o->fused = DMUON_FUSED_AUTO;
}

int dmuon_plan(const int64_t* rows, const int64_t* cols, int64_t count, int dtype,
               const dmuon_plan_opts* opts, dmuon_plan_t** out) {
  using namespace dmuon;
  if (!out) return fail(DMUON_EINVAL, "out is NULL");
  *out = nullptr;
  if (!rows || !cols) return fail(DMUON_EINVAL, "rows/cols is NULL");
  if (count <= 0) return fail(DMUON_EINVAL, "count must be positive (got %lld)", (long long)count);
  if (dtype != DMUON_BF16 && dtype != DMUON_F32) return fail(DMUON_EINVAL, "unknown dtype %d", dtype);
  for (int64_t i = 0; i < count; ++i) {
    if (rows[i] <= 0 || cols[i] <= 0)
      return fail(DMUON_EINVAL, "shape %lld is %lld x %lld", (long long)i, (long long)rows[i], (long long)cols[i]);
    if (rows[i] > (1 << 30) || cols[i] > (1 << 30) || rows[i] * cols[i] > ((int64_t)1 << 40))
      return fail(DMUON_EINVAL, "shape %lld too large", (long long)i);
  }
  dmuon_plan_opts o;
  dmuon_plan_opts_default(&o);
  if (opts) o = *opts;
  if (o.precision < DMUON_PREC_AUTO || o.precision > DMUON_PREC_F32)
    return fail(DMUON_EINVAL, "unknown precision %d", o.precision);
  if (o.scale_mode != DMUON_SCALE_SQRT_RATIO && o.scale_mode != DMUON_SCALE_NONE)
    return fail(DMUON_EINVAL, "unknown scale mode %d", o.scale_mode);
  if (o.form != DMUON_FORM_AUTO && o.form != DMUON_FORM_GRAM && o.form != DMUON_FORM_STANDARD)
    return fail(DMUON_EINVAL, "unknown form %d", o.form);
  if (!(o.pad_ratio >= 0.0f && o.pad_ratio <= 1.0f))
    return fail(DMUON_EINVAL, "pad_ratio must be in [0, 1] (got %g)", (double)o.pad_ratio);
  if (o.storage != DMUON_STORAGE_AUTO && o.storage != DMUON_STORAGE_FULL)
    return fail(DMUON_EINVAL, "unknown storage %d", o.storage);
  if (o.fused < DMUON_FUSED_AUTO || o.fused > DMUON_FUSED_SPLIT)
    return fail(DMUON_EINVAL, "unknown fused %d", o.fused);
  if (dtype == DMUON_F32 && o.precision != DMUON_PREC_AUTO && o.precision != DMUON_PREC_F32)
    return fail(DMUON_EUNSUPPORTED, "f32 matrices run on the fp32 path only (precision %d)", o.precision);
  try {
    auto* p = new struct dmuon_plan();
    PlanImpl& pi = p->impl;
    pi.dtype = dtype;
    pi.precision_req = o.precision;
    pi.form_req = o.form;
    pi.storage_req = o.storage;
    pi.fused_req = o.fused;
    pi.pad_ratio = o.pad_ratio;
    pi.scale_mode = o.scale_mode;
    pi.eps = o.eps > 0 ? (double)o.eps : kDefaultEps;
    pi.device = !o.no_device;
    int e = load_table(pi, o.tune_path);
    if (e) {
      delete p;
      return e;
    }
    build_plan(pi, rows, cols, count);
    if (o.max_workspace > 0 && pi.ws_bytes > (size_t)o.max_workspace) {
      size_t need = pi.ws_bytes;
      delete p;
      return fail(DMUON_ENOMEM, "workspace needs %zu bytes, cap is %lld", need, (long long)o.max_workspace);
    }
    if (pi.device) {
      hipError_t he = hipGetDevice(&pi.device_id);
      if (he != hipSuccess) {
        delete p;
        return fail(DMUON_EHIP, "hipGetDevice: %s", hipGetErrorString(he));
      }
      char* w = nullptr;
      e = alloc_workspace(pi.ws_bytes, &w);
      if (e != DMUON_OK) {
        delete p;
        return e;
      }
      pi.ws = w;
      pi.owns_ws = true;
    }
    log_plan("plan", pi);
    *out = p;
    return DMUON_OK;
  } catch (...) {
    return fail(DMUON_ENOMEM, "host allocation failed");
  }
}

int dmuon_plan_destroy(dmuon_plan_t* plan) {
  if (!plan) return DMUON_OK;
  int rc = DMUON_OK;
  if (plan->impl.owns_ws && plan->impl.ws) {
    hipError_t e = hipFree(plan->impl.ws);
    if (e != hipSuccess) rc = dmuon::fail(DMUON_EHIP, "hipFree: %s", hipGetErrorString(e));
  }
  delete plan;
  return rc;
}

int64_t dmuon_plan_describe(const dmuon_plan_t* plan, char* buf, size_t len) {
  using namespace dmuon;
  if (!plan) return fail(DMUON_EINVAL, "plan is NULL");
  const std::string s = describe_plan(plan->impl);
  if (buf && len > 0) {
    size_t k = std::min(len - 1, s.size());
    std::memcpy(buf, s.data(), k);
    buf[k] = 0;
  }
  return (int64_t)s.size();
}

int dmuon_step(const dmuon_plan_t* plan, void* const* params, const void* const* grads, void* const* momenta,
               float lr, float weight_decay, float mu, int nesterov, int steps, float a, float b, float c,
               void* stream) {
  using namespace dmuon;
  if (!plan) return fail(DMUON_EPLAN, "plan is NULL");
  const PlanImpl& p = plan->impl;
  if (!p.device || !p.ws) return fail(DMUON_EPLAN, "plan was made with no_device and cannot run");
  if (!params || !grads || !momenta) return fail(DMUON_EINVAL, "params/grads/momenta is NULL");
  int e = check_coeffs(steps, a, b, c);
  if (e) return e;
  if (!std::isfinite(lr) || !std::isfinite(weight_decay) || !std::isfinite(mu))
    return fail(DMUON_EINVAL, "lr, weight_decay and mu must be finite");
  for (int64_t i = 0; i < p.count; ++i)
    if (!params[i] || !grads[i] || !momenta[i])
      return fail(DMUON_EINVAL, "null pointer for matrix %lld", (long long)i);
  {
    const RangeScan range = scan_recurrence(a, b, c, steps);
    Prec unused;
    for (const auto& bk : p.buckets) {
      e = bucket_prec(p, bk, range, &unused);
      if (e) return e;
    }
  }
  int dev = -1;
  hipError_t he = hipGetDevice(&dev);
  if (he != hipSuccess) return fail(DMUON_EHIP, "hipGetDevice: %s", hipGetErrorString(he));
  if (dev != p.device_id) return fail(DMUON_EPLAN, "plan belongs to device %d, current device is %d", p.device_id, dev);
  RunSpec rs;
  rs.mode = RunSpec::STEP;
  rs.steps = steps;
  rs.a = a;
  rs.b = b;
  rs.c = c;
  rs.io = params;
  rs.grads = grads;
  rs.momenta = momenta;
  rs.lr = lr;
  rs.wd = weight_decay;
  rs.mu = mu;
  rs.nesterov = nesterov ? 1 : 0;
  try {
    return run(p, p.ws, rs, static_cast<hipStream_t>(stream));
  } catch (...) {
    return fail(DMUON_ENOMEM, "host allocation failed");
  }
}

int dmuon_plan_ns(const dmuon_plan_t* plan, void* const* mats, int steps, float a, float b, float c,
                  void* stream) {
  using namespace dmuon;
  if (!plan) return fail(DMUON_EPLAN, "plan is NULL");
  const PlanImpl& p = plan->impl;
  if (!p.device || !p.ws) return fail(DMUON_EPLAN, "plan was made with no_device and cannot run");
  if (!mats) return fail(DMUON_EINVAL, "mats is NULL");
  int e = check_coeffs(steps, a, b, c);
  if (e) return e;
  for (int64_t i = 0; i < p.count; ++i)
    if (!mats[i]) return fail(DMUON_EINVAL, "null pointer for matrix %lld", (long long)i);
  {
    const RangeScan range = scan_recurrence(a, b, c, steps);
    Prec unused;
    for (const auto& bk : p.buckets) {
      e = bucket_prec(p, bk, range, &unused);
      if (e) return e;
    }
  }
  int dev = -1;
  hipError_t he = hipGetDevice(&dev);
  if (he != hipSuccess) return fail(DMUON_EHIP, "hipGetDevice: %s", hipGetErrorString(he));
  if (dev != p.device_id) return fail(DMUON_EPLAN, "plan belongs to device %d, current device is %d", p.device_id, dev);
  RunSpec rs;
  rs.mode = RunSpec::NS;
  rs.steps = steps;
  rs.a = a;
  rs.b = b;
  rs.c = c;
  rs.io = mats;
  try {
    return run(p, p.ws, rs, static_cast<hipStream_t>(stream));
  } catch (...) {
    return fail(DMUON_ENOMEM, "host allocation failed");
  }
}

int dmuon_adamw_step(void* const* params, const void* const* grads, void* const* exp_avg,
                     void* const* exp_avg_sq, const int64_t* numel, int64_t count, int dtype, float lr,
                     float beta1, float beta2, float eps, float weight_decay, int64_t step, void* stream) {
  using namespace dmuon;
  if (!params || !grads || !exp_avg || !exp_avg_sq || !numel)
    return fail(DMUON_EINVAL, "params/grads/exp_avg/exp_avg_sq/numel is NULL");
  if (count <= 0) return fail(DMUON_EINVAL, "count must be positive (got %lld)", (long long)count);
  if (dtype != DMUON_BF16 && dtype != DMUON_F32) return fail(DMUON_EINVAL, "unknown dtype %d", dtype);
  if (step < 1) return fail(DMUON_EINVAL, "step counts from 1 (got %lld)", (long long)step);
  if (!(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f))
    return fail(DMUON_EINVAL, "betas must lie in [0, 1) (got %g, %g)", (double)beta1, (double)beta2);
  if (!(eps >= 0.0f) || !std::isfinite(eps) || !std::isfinite(lr) || !std::isfinite(weight_decay))
    return fail(DMUON_EINVAL, "lr and weight_decay must be finite and eps finite and >= 0");
  for (int64_t i = 0; i < count; ++i) {
    if (!params[i] || !grads[i] || !exp_avg[i] || !exp_avg_sq[i])
      return fail(DMUON_EINVAL, "null pointer for tensor %lld", (long long)i);
    if (numel[i] <= 0 || numel[i] > ((int64_t)1 << 40))
      return fail(DMUON_EINVAL, "numel[%lld] = %lld is out of range", (long long)i, (long long)numel[i]);
  }
  const int es = elem_size(dtype);
  // bias corrections in double, handed to the kernel as fp32 factors
  const double bc1 = 1.0 - std::pow((double)beta1, (double)step);
  const double bc2 = 1.0 - std::pow((double)beta2, (double)step);
  AdamwArgs proto{};
  proto.esize = es;
  proto.beta1 = beta1;
  proto.beta2 = beta2;
  proto.omb1 = (float)(1.0 - (double)beta1);
  proto.omb2 = (float)(1.0 - (double)beta2);
  proto.eps = eps;
  proto.decay = (float)(1.0 - (double)lr * (double)weight_decay);
  proto.step_size = (float)((double)lr / bc1);
  proto.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(bc2));
  hipStream_t st = static_cast<hipStream_t>(stream);
  for (int64_t s0 = 0; s0 < count; s0 += kMaxTab) {
    const int64_t s1 = std::min<int64_t>(count, s0 + kMaxTab);
    AdamwArgs a = proto;
    a.ntens = (int32_t)(s1 - s0);
    a.blk0[0] = 0;
    double bytes = 0.0;
    for (int64_t i = s0; i < s1; ++i) {
      const int k = (int)(i - s0);
      a.w[k] = reinterpret_cast<uint64_t>(params[i]);
      a.g[k] = reinterpret_cast<uint64_t>(grads[i]);
      a.m[k] = reinterpret_cast<uint64_t>(exp_avg[i]);
      a.v[k] = reinterpret_cast<uint64_t>(exp_avg_sq[i]);
      a.numel[k] = numel[i];
      a.blk0[k + 1] = a.blk0[k] + (numel[i] + kAdamChunk - 1) / kAdamChunk;
      if (((a.w[k] | a.g[k] | a.m[k] | a.v[k]) & 15u) == 0) a.vec_mask |= 1ull << k;
      bytes += (double)numel[i] * (3.0 * es + 16.0);
    }
    const char* name = es == 2 ? "adamw_kernel<2>" : "adamw_kernel<4>";
    HIP_TRY(timed(name, 0.0, bytes, st, [&] { return launch_adamw(a, st); }));
  }
  return DMUON_OK;
}

int dmuon_release_workspace(void) {
  using namespace dmuon;
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lock(g_cache_mu);
  auto it = g_cache.find(dev);
  if (it == g_cache.end()) return DMUON_OK;
  DeviceCache& dc = it->second;
  if (!dc.ws && dc.retired.empty()) return DMUON_OK;
  // enqueued work on any stream may still use the buffers
  HIP_TRY(hipDeviceSynchronize());
  int rc = DMUON_OK;
  auto release = [&](char* p) {
    const hipError_t e = hipFree(p);
    if (e != hipSuccess && rc == DMUON_OK) rc = fail(DMUON_EHIP, "hipFree: %s", hipGetErrorString(e));
  };
  for (auto& r : dc.retired) release(r.first);
  dc.retired.clear();
  if (dc.ws) release(dc.ws);
  dc.ws = nullptr;
  dc.bytes = 0;
  return rc;
}

int dmuon_workspace_info(int64_t* live_bytes, int64_t* retired_bytes, int32_t* retired_count) {
  using namespace dmuon;
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lock(g_cache_mu);
  int64_t live = 0, ret = 0;
  int32_t cnt = 0;
  auto it = g_cache.find(dev);
  if (it != g_cache.end()) {
    live = it->second.ws ? (int64_t)it->second.bytes : 0;
    for (auto& r : it->second.retired) ret += (int64_t)r.second;
    cnt = (int32_t)it->second.retired.size();
  }
  if (live_bytes) *live_bytes = live;
  if (retired_bytes) *retired_bytes = ret;
  if (retired_count) *retired_count = cnt;
  return DMUON_OK;
}

int dmuon_timing_enable(int enable) {
  std::lock_guard<std::mutex> lk(dmuon::g_tmu);
  dmuon::g_timing = enable != 0;
  return DMUON_OK;
}

int64_t dmuon_timing_report(char* buf, size_t len) {
  using namespace dmuon;
  std::vector<TimingRec> recs;
  {
    std::lock_guard<std::mutex> lk(g_tmu);
    recs.swap(g_trecs);
  }
  struct Agg {
    int64_t n = 0;
    double ms = 0, flops = 0, bytes = 0;
  };
  std::vector<std::pair<std::string, Agg>> aggs;
  int rc = DMUON_OK;
  for (auto& r : recs) {
    float ms = 0.0f;
    hipError_t e = hipEventSynchronize(r.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess && rc == DMUON_OK) rc = fail(DMUON_EHIP, "timing event: %s", hipGetErrorString(e));
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
    auto it = std::find_if(aggs.begin(), aggs.end(), [&](const auto& x) { return x.first == r.name; });
    if (it == aggs.end()) {
      aggs.push_back({r.name, Agg{}});
      it = aggs.end() - 1;
    }
    it->second.n += 1;
    it->second.ms += ms;
    it->second.flops += r.flops;
    it->second.bytes += r.bytes;
  }
  if (rc != DMUON_OK) return rc;
  std::string s = "{\"kernels\": [";
  char tmp[512];
  for (size_t i = 0; i < aggs.size(); ++i) {
    const Agg& a = aggs[i].second;
    snprintf(tmp, sizeof tmp,
             "%s{\"kernel\": \"%s\", \"launches\": %lld, \"total_ms\": %.6f, \"avg_ms\": %.6f, "
             "\"flops\": %.6e, \"bytes\": %.6e}",
             i ? ", " : "", aggs[i].first.c_str(), (long long)a.n, a.ms, a.ms / (double)a.n, a.flops, a.bytes);
    s += tmp;
  }
  s += "]}";
  if (buf && len > 0) {
    size_t k = std::min(len - 1, s.size());
    std::memcpy(buf, s.data(), k);
    buf[k] = 0;
  }
  return (int64_t)s.size();
}

int dmuon_profile_costs(const int64_t* rows, const int64_t* cols, int32_t nshapes, const int32_t* batches,
                        int32_t npts, int steps, float a, float b, float c, int32_t warmup, int32_t repeats,
                        double* times, void* stream) {
  using namespace dmuon;
  if (!rows || !cols || !batches || !times) return fail(DMUON_EINVAL, "NULL argument");
  if (nshapes <= 0 || npts <= 0) return fail(DMUON_EINVAL, "nshapes and npts must be positive");
  if (warmup < 0 || repeats < 1) return fail(DMUON_EINVAL, "warmup must be >= 0 and repeats >= 1");
  if (steps < 0) return fail(DMUON_EINVAL, "steps must be >= 0 (got %d)", steps);
  if (!std::isfinite(a) || !std::isfinite(b) || !std::isfinite(c)) return fail(DMUON_EINVAL, "coefficients must be finite");
  for (int p = 0; p < npts; ++p)
    if (batches[p] < 1 || batches[p] > 4096 || (p > 0 && batches[p] <= batches[p - 1]))
      return fail(DMUON_EINVAL, "batch sizes must be in [1, 4096] and strictly increasing");
  for (int s = 0; s < nshapes; ++s)
    if (rows[s] <= 0 || cols[s] <= 0 || rows[s] > (1 << 20) || cols[s] > (1 << 20))
      return fail(DMUON_EINVAL, "shape %d: rows and cols must be in [1, 2^20]", s);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  HIP_TRY(hipEventCreate(&e0));
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return fail(DMUON_EHIP, "hipEventCreate failed");
  }
  int rc = DMUON_OK;
  char* buf = nullptr;
  for (int s = 0; s < nshapes && rc == DMUON_OK; ++s) {
    const int64_t elems = rows[s] * cols[s];
    const size_t mbytes = round_up((size_t)elems * 2, kAlign);
    const size_t bytes = mbytes * (size_t)batches[npts - 1];
    if (hipMalloc(&buf, bytes) != hipSuccess) {
      rc = fail(DMUON_ENOMEM, "profiling buffer of %zu bytes", bytes);
      buf = nullptr;
      break;
    }
    for (int64_t i = 0; i < batches[npts - 1] && rc == DMUON_OK; ++i) {
      hipError_t e = launch_fill_bf16(reinterpret_cast<uint16_t*>(buf + i * mbytes), elems, (uint32_t)(s * 7919 + i + 1), st);
      if (e != hipSuccess) rc = fail(DMUON_EHIP, "fill: %s", hipGetErrorString(e));
    }
    std::vector<void*> ptrs((size_t)batches[npts - 1]);
    for (size_t i = 0; i < ptrs.size(); ++i) ptrs[i] = buf + i * mbytes;
    for (int p = 0; p < npts && rc == DMUON_OK; ++p) {
      const int64_t k = batches[p];
      for (int w = 0; w < warmup && rc == DMUON_OK; ++w)
        rc = dmuon_ns_batched(ptrs.data(), rows[s], cols[s], k, steps, a, b, c, stream);
      std::vector<float> ms;
      for (int r = 0; r < repeats && rc == DMUON_OK; ++r) {
        float t = 0.0f;
        if (hipEventRecord(e0, st) != hipSuccess) rc = fail(DMUON_EHIP, "hipEventRecord failed");
        if (rc == DMUON_OK) rc = dmuon_ns_batched(ptrs.data(), rows[s], cols[s], k, steps, a, b, c, stream);
        if (rc == DMUON_OK && (hipEventRecord(e1, st) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
                               hipEventElapsedTime(&t, e0, e1) != hipSuccess))
          rc = fail(DMUON_EHIP, "profiling events failed");
        ms.push_back(t);
      }
      if (rc == DMUON_OK) {
        std::sort(ms.begin(), ms.end());
        const size_t h = ms.size() / 2;
        times[(int64_t)s * npts + p] = (ms.size() % 2) ? ms[h] : 0.5 * ((double)ms[h - 1] + (double)ms[h]);
      }
    }
    (void)hipStreamSynchronize(st);
    (void)hipFree(buf);
    buf = nullptr;
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return rc;
}

int dmuon_tune(const int64_t* rows, const int64_t* cols, int64_t count, int steps, float a, float b, float c,
               int32_t warmup, int32_t repeats, const char* out_path, void* stream) {
  using namespace dmuon;
  if (!rows || !cols || !out_path || !*out_path) return fail(DMUON_EINVAL, "rows/cols/out_path is NULL");
  if (count <= 0) return fail(DMUON_EINVAL, "count must be positive (got %lld)", (long long)count);
  if (warmup < 0 || repeats < 1) return fail(DMUON_EINVAL, "warmup must be >= 0 and repeats >= 1");
  int e = check_coeffs(steps, a, b, c);
  if (e) return e;
  for (int64_t i = 0; i < count; ++i)
    if (rows[i] <= 0 || cols[i] <= 0 || rows[i] > (1 << 20) || cols[i] > (1 << 20))
      return fail(DMUON_EINVAL, "shape %lld: rows and cols must be in [1, 2^20]", (long long)i);
  hipStream_t st = static_cast<hipStream_t>(stream);
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  hipDeviceProp_t prop;
  HIP_TRY(hipGetDeviceProperties(&prop, dev));
  try {
    // the buckets as a plan with the built-in table forms them
    PlanImpl base;
    base.table = builtin_table();
    build_plan(base, rows, cols, count);
    struct Cand {
      int rec, fin;
      double ms;
    };
    struct Result {
      int64_t m, count;
      std::vector<int64_t> members;
      std::vector<Cand> cands;
      int best = -1;
    };
    std::vector<Result> results;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    HIP_TRY(hipEventCreate(&e0));
    HIP_TRY(hipEventCreate(&e1));
    int rc = DMUON_OK;
    const int tiles[3] = {64, 128, 256};
    for (const RecBucket& bk : base.buckets) {
      if (rc != DMUON_OK) break;
      Result res;
      res.m = bk.m;
      res.count = bk.count;
      for (int gi : bk.groups)
        for (int64_t mbr : base.groups[gi].members) res.members.push_back(mbr);
      std::vector<int64_t> br, bc;
      for (int64_t mbr : res.members) {
        br.push_back(rows[mbr]);
        bc.push_back(cols[mbr]);
      }
      // the bucket's matrices, deterministic pseudo-random bf16
      std::vector<size_t> off;
      size_t total = 0;
      for (size_t i = 0; i < br.size(); ++i) {
        off.push_back(total);
        total += round_up((size_t)(br[i] * bc[i]) * 2, kAlign);
      }
      char* mats = nullptr;
      if (hipMalloc(&mats, total) != hipSuccess) {
        (void)hipGetLastError();
        rc = fail(DMUON_ENOMEM, "tuning buffer of %zu bytes", total);
        break;
      }
      std::vector<void*> ptrs;
      for (size_t i = 0; i < br.size(); ++i) ptrs.push_back(mats + off[i]);
      std::vector<std::tuple<int, std::vector<int>>> seen;  // effective tiles already timed
      for (int rt : tiles) {
        for (int ft : tiles) {
          if (rc != DMUON_OK) break;
          PlanImpl p;
          p.table = {{1 << 30, kAnyBatch, rt, ft, ft}};
          p.table_source = "candidate";
          build_plan(p, br.data(), bc.data(), (int64_t)br.size());
          std::vector<int> eff;
          for (const Group& g : p.groups) {
            eff.push_back(g.tile_syrk);
            eff.push_back(g.tile_fin);
          }
          const int er = p.buckets[0].tile;
          bool dup = false;
          for (auto& x : seen) dup = dup || (std::get<0>(x) == er && std::get<1>(x) == eff);
          if (dup) continue;
          seen.emplace_back(er, eff);
          char* ws = nullptr;
          rc = alloc_workspace(p.ws_bytes, &ws);
          if (rc != DMUON_OK) break;
          RunSpec rs;
          rs.mode = RunSpec::NS;
          rs.steps = steps;
          rs.a = a;
          rs.b = b;
          rs.c = c;
          rs.io = ptrs.data();
          std::vector<float> ms;
          for (size_t i = 0; i < br.size() && rc == DMUON_OK; ++i)
            if (launch_fill_bf16(reinterpret_cast<uint16_t*>(mats + off[i]), br[i] * bc[i],
                                 (uint32_t)(7919 * i + 13), st) != hipSuccess)
              rc = fail(DMUON_EHIP, "fill failed");
          for (int w = 0; w < warmup && rc == DMUON_OK; ++w) rc = run(p, ws, rs, st);
          for (int r = 0; r < repeats && rc == DMUON_OK; ++r) {
            float t = 0.0f;
            if (hipEventRecord(e0, st) != hipSuccess) rc = fail(DMUON_EHIP, "hipEventRecord failed");
            if (rc == DMUON_OK) rc = run(p, ws, rs, st);
            if (rc == DMUON_OK && (hipEventRecord(e1, st) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
                                   hipEventElapsedTime(&t, e0, e1) != hipSuccess))
              rc = fail(DMUON_EHIP, "tuning events failed");
            ms.push_back(t);
          }
          (void)hipStreamSynchronize(st);
          (void)hipFree(ws);
          if (rc != DMUON_OK) break;
          std::sort(ms.begin(), ms.end());
          const size_t h = ms.size() / 2;
          const double med = (ms.size() % 2) ? ms[h] : 0.5 * ((double)ms[h - 1] + (double)ms[h]);
          res.cands.push_back({er, eff.empty() ? ft : eff[1], med});
        }
      }
      (void)hipStreamSynchronize(st);
      (void)hipFree(mats);
      if (rc != DMUON_OK) break;
      for (size_t i = 0; i < res.cands.size(); ++i)
        if (res.best < 0 || res.cands[i].ms < res.cands[(size_t)res.best].ms) res.best = (int)i;
      results.push_back(res);
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (rc != DMUON_OK) return rc;
    // one entry per bucket, ordered by (m, count)
    std::sort(results.begin(), results.end(),
              [](const Result& x, const Result& y) { return std::tie(x.m, x.count) < std::tie(y.m, y.count); });
    std::string js = "{\"arch\": \"";
    js += prop.gcnArchName;
    js += "\", \"device\": \"";
    for (const char* q = prop.name; *q; ++q)
      if (*q != '"' && *q != '\\') js += *q;
    char tmp[256];
    snprintf(tmp, sizeof tmp, "\", \"steps\": %d, \"coeffs\": [%.9g, %.9g, %.9g], \"warmup\": %d, \"repeats\": %d, ",
             steps, (double)a, (double)b, (double)c, warmup, repeats);
    js += tmp;
    js += "\"entries\": [";
    for (size_t i = 0; i < results.size(); ++i) {
      const Result& r = results[i];
      const Cand& bst = r.cands[(size_t)r.best];
      snprintf(tmp, sizeof tmp, "%s{\"max_m\": %lld, \"max_batch\": %lld, \"rec\": %d, \"syrk\": %d, \"final\": %d}",
               i ? ", " : "", (long long)r.m, (long long)r.count, bst.rec, bst.fin, bst.fin);
      js += tmp;
    }
    js += "], \"measured\": [";
    for (size_t i = 0; i < results.size(); ++i) {
      const Result& r = results[i];
      snprintf(tmp, sizeof tmp, "%s{\"m\": %lld, \"count\": %lld, \"candidates\": [", i ? ", " : "",
               (long long)r.m, (long long)r.count);
      js += tmp;
      for (size_t k = 0; k < r.cands.size(); ++k) {
        snprintf(tmp, sizeof tmp, "%s{\"rec\": %d, \"final\": %d, \"ms\": %.4f}", k ? ", " : "", r.cands[k].rec,
                 r.cands[k].fin, r.cands[k].ms);
        js += tmp;
      }
      js += "]}";
    }
    js += "]}\n";
    FILE* f = std::fopen(out_path, "wb");
    if (!f) return fail(DMUON_EINVAL, "cannot write '%s'", out_path);
    const bool ok = std::fwrite(js.data(), 1, js.size(), f) == js.size();
    if (std::fclose(f) != 0 || !ok) return fail(DMUON_EINVAL, "writing '%s' failed", out_path);
    return DMUON_OK;
  } catch (...) {
    return fail(DMUON_ENOMEM, "host allocation failed");
  }
}

const char* dmuon_last_error(void) { return dmuon::g_last_error.c_str(); }

const char* dmuon_version(void) { return "dmuon-mi355x 0.1.0 (gfx950)"; }

}  // extern "C"
