// Owner assignment for distributed Muon: every matrix gets exactly one owner
// rank, which runs its Newton-Schulz update; owners are chosen to minimise the
// predicted makespan (the largest per-rank time) from a per-shape cost table
// measured at a few batch sizes.
//
// Method: DMuon (gist.science technical summary, section 2.3: a
// makespan-minimising integer program over owner choices, with a greedy
// heuristic when the search space is too large; costs come from profiling each
// distinct shape rather than from flop counts).  The exact solver here is a
// branch and bound over per-rank batch counts, which reaches the same optimum
// as the integer program.  Host-only code.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <numeric>
#include <vector>

#include "dmuon.h"
#include "errors.h"

namespace dmuon {
namespace {

constexpr int64_t kDefaultNodes = 1000000;
constexpr int64_t kAutoExactMax = 64;  // AUTO runs the exact search up to this many matrices

// Matrices of one shape that share an owner run as one batch.  T[k] is the
// predicted time of a batch of k of them: the piecewise-linear curve through
// (0, 0) and the measured points, extended past the last point with the last
// segment's slope.
std::vector<double> batch_times(const int32_t* batches, int npts, const double* times, int64_t kmax) {
  std::vector<double> x(1, 0.0), y(1, 0.0);
  for (int p = 0; p < npts; ++p) {
    x.push_back((double)batches[p]);
    y.push_back(times[p]);
  }
  std::vector<double> T((size_t)kmax + 1, 0.0);
  for (int64_t k = 1; k <= kmax; ++k) {
    size_t j = 1;
    while (j + 1 < x.size() && x[j] < (double)k) ++j;
    const double t = y[j - 1] + (y[j] - y[j - 1]) * ((double)k - x[j - 1]) / (x[j] - x[j - 1]);
    T[(size_t)k] = std::max(t, 0.0);
  }
  return T;
}

struct Problem {
  int R = 1, S = 0;
  std::vector<int64_t> n;               // matrices per shape
  std::vector<std::vector<double>> T;   // T[s][k], k = 0..n[s]
  std::vector<double> min_ratio;        // min over k of T[s][k] / k: a per-matrix lower bound
  std::vector<int> order;               // shapes, heaviest total first
};

using Counts = std::vector<std::vector<int64_t>>;  // [rank][shape]

double makespan_of(const Problem& P, const Counts& c) {
  double mx = 0.0;
  for (int r = 0; r < P.R; ++r) {
    double l = 0.0;
    for (int s = 0; s < P.S; ++s) l += P.T[s][(size_t)c[r][s]];
    mx = std::max(mx, l);
  }
  return mx;
}

// One matrix at a time, shapes in order of decreasing single-matrix time: each
// goes to the rank whose load after taking it is smallest (lowest rank on ties).
double greedy(const Problem& P, Counts& c) {
  c.assign(P.R, std::vector<int64_t>(P.S, 0));
  std::vector<double> load(P.R, 0.0);
  std::vector<int> shapes(P.S);
  std::iota(shapes.begin(), shapes.end(), 0);
  std::stable_sort(shapes.begin(), shapes.end(), [&](int a, int b) {
    const double ta = P.n[a] > 0 ? P.T[a][1] : 0.0, tb = P.n[b] > 0 ? P.T[b][1] : 0.0;
    return ta > tb;
  });
  for (int s : shapes) {
    for (int64_t i = 0; i < P.n[s]; ++i) {
      int best = 0;
      double bl = 0.0;
      for (int r = 0; r < P.R; ++r) {
        const double l = load[r] + P.T[s][(size_t)c[r][s] + 1] - P.T[s][(size_t)c[r][s]];
        if (r == 0 || l < bl) {
          best = r;
          bl = l;
        }
      }
      load[best] = bl;
      ++c[best][s];
    }
  }
  return makespan_of(P, c);
}

// Depth-first search over the counts each rank takes of each shape (shapes in
// P.order, ranks in index order), pruned by the incumbent makespan and by the
// average-load bound.  Ranks with identical counts on every shape placed so
// far are interchangeable, so their counts of the next shape are kept
// non-increasing.
struct Search {
  const Problem& P;
  int64_t limit;
  int64_t nodes = 0;
  bool aborted = false;
  double best;
  Counts best_c, c;
  std::vector<double> load;
  std::vector<double> rest;          // rest[i]: lower bound on the work of shapes order[i..]
  std::vector<std::vector<char>> tie;  // tie[i][r]: rank r matches rank r - 1 on shapes order[0..i)
  double tol;

  Search(const Problem& p, int64_t lim, double incumbent, const Counts& inc)
      : P(p), limit(lim), best(incumbent), best_c(inc) {
    c.assign(P.R, std::vector<int64_t>(P.S, 0));
    load.assign(P.R, 0.0);
    rest.assign(P.S + 1, 0.0);
    for (int i = P.S - 1; i >= 0; --i) {
      const int s = P.order[i];
      rest[i] = rest[i + 1] + (double)P.n[s] * P.min_ratio[s];
    }
    tie.assign(P.S + 1, std::vector<char>(P.R, 1));
    tol = 1e-12 * std::max(1.0, incumbent);
  }

  double sum_load() const {
    double t = 0.0;
    for (double l : load) t += l;
    return t;
  }

  void place(int si, int r, int64_t rem) {
    if (aborted) return;
    if (++nodes > limit) {
      aborted = true;
      return;
    }
    if (si == P.S) {
      const double mk = *std::max_element(load.begin(), load.end());
      if (mk < best - tol) {
        best = mk;
        best_c = c;
      }
      return;
    }
    const int s = P.order[si];
    if (r == 0) {
      // ties for this shape: ranks equal on every shape placed so far
      if (si > 0) {
        const int sp = P.order[si - 1];
        for (int q = 1; q < P.R; ++q) tie[si][q] = tie[si - 1][q] && c[q][sp] == c[q - 1][sp];
      }
      const double mx = *std::max_element(load.begin(), load.end());
      const double lb = std::max(mx, (sum_load() + rest[si]) / P.R);
      if (lb >= best - tol) return;
    } else {
      const double lb = (sum_load() + (double)rem * P.min_ratio[s] + rest[si + 1]) / P.R;
      if (lb >= best - tol) return;
    }
    const bool last = r == P.R - 1;
    int64_t kmax = rem;
    if (r > 0 && tie[si][r]) kmax = std::min(kmax, c[r - 1][s]);
    const int64_t kmin = last ? rem : 0;
    if (kmin > kmax) return;
    for (int64_t k = kmax; k >= kmin; --k) {
      const double add = P.T[s][(size_t)k];
      if (load[r] + add >= best - tol) continue;
      load[r] += add;
      c[r][s] = k;
      if (last)
        place(si + 1, 0, si + 1 < P.S ? P.n[P.order[si + 1]] : 0);
      else
        place(si, r + 1, rem - k);
      c[r][s] = 0;
      load[r] -= add;
      if (aborted) return;
    }
  }
};

}  // namespace
}  // namespace dmuon

extern "C" int dmuon_assign_owners(const int32_t* shape_of, int64_t count, const int32_t* batches, int32_t npts,
                                   const double* times, int32_t nshapes, int32_t ranks, int32_t method,
                                   int64_t node_limit, int32_t* owner, double* makespan, int32_t* optimal) {
  using namespace dmuon;
  try {
    if (!shape_of || !batches || !times || !owner) return fail(DMUON_EINVAL, "NULL argument");
    if (count <= 0) return fail(DMUON_EINVAL, "count must be positive (got %lld)", (long long)count);
    if (npts <= 0 || nshapes <= 0) return fail(DMUON_EINVAL, "npts and nshapes must be positive");
    if (ranks <= 0 || ranks > (1 << 20)) return fail(DMUON_EINVAL, "ranks must be in [1, 2^20] (got %d)", ranks);
    if (method != DMUON_ASSIGN_AUTO && method != DMUON_ASSIGN_EXACT && method != DMUON_ASSIGN_GREEDY)
      return fail(DMUON_EINVAL, "unknown assignment method %d", method);
    for (int p = 0; p < npts; ++p) {
      if (batches[p] < 1 || (p > 0 && batches[p] <= batches[p - 1]))
        return fail(DMUON_EINVAL, "batch sizes must be >= 1 and strictly increasing");
    }
    for (int64_t i = 0; i < (int64_t)nshapes * npts; ++i)
      if (!std::isfinite(times[i]) || times[i] < 0.0) return fail(DMUON_EINVAL, "times must be finite and >= 0");
    Problem P;
    P.R = ranks;
    P.S = nshapes;
    P.n.assign(nshapes, 0);
    for (int64_t i = 0; i < count; ++i) {
      if (shape_of[i] < 0 || shape_of[i] >= nshapes)
        return fail(DMUON_EINVAL, "shape_of[%lld] = %d is out of range", (long long)i, shape_of[i]);
      ++P.n[shape_of[i]];
    }
    P.T.resize(nshapes);
    P.min_ratio.assign(nshapes, 0.0);
    for (int s = 0; s < nshapes; ++s) {
      P.T[s] = batch_times(batches, npts, times + (int64_t)s * npts, P.n[s] + 1);
      double mr = P.n[s] > 0 ? INFINITY : 0.0;
      for (int64_t k = 1; k <= P.n[s]; ++k) mr = std::min(mr, P.T[s][(size_t)k] / (double)k);
      P.min_ratio[s] = mr;
    }
    P.order.resize(nshapes);
    std::iota(P.order.begin(), P.order.end(), 0);
    std::stable_sort(P.order.begin(), P.order.end(), [&](int a, int b) {
      return P.T[a][(size_t)P.n[a]] > P.T[b][(size_t)P.n[b]];
    });

    Counts c;
    double mk = greedy(P, c);
    int opt = 0;
    const bool exact = method == DMUON_ASSIGN_EXACT || (method == DMUON_ASSIGN_AUTO && count <= kAutoExactMax);
    if (exact) {
      Search S(P, node_limit > 0 ? node_limit : kDefaultNodes, mk, c);
      S.place(0, 0, P.n[P.order[0]]);
      if (S.best < mk) {
        mk = S.best;
        c = S.best_c;
      }
      opt = S.aborted ? 0 : 1;
    }
    // matrices of shape s in index order: the first c[0][s] to rank 0, and so on
    std::vector<int> rank_of_next(nshapes, 0);
    std::vector<int64_t> left(nshapes, 0);
    for (int s = 0; s < nshapes; ++s) left[s] = c[0][s];
    for (int64_t i = 0; i < count; ++i) {
      const int s = shape_of[i];
      while (left[s] == 0) left[s] = c[++rank_of_next[s]][s];
      owner[i] = rank_of_next[s];
      --left[s];
    }
    if (makespan) *makespan = mk;
    if (optimal) *optimal = opt;
    return DMUON_OK;
  } catch (...) {
    return fail(DMUON_ENOMEM, "host allocation failed");
  }
}
