"""Plain oracle for the owner assignment of distributed DMuon.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix (gist.science/pt, technical summary section 2.3): every
matrix gets one owner rank; costs vary strongly with the matrix shape, so the
owners are chosen by an integer program that minimises the predicted makespan
(the largest per-rank load), from costs profiled per distinct shape at several
batch sizes; a greedy heuristic stands in when the search space is too large.

Readings taken where the pages leave a step open:

* matrices of one shape that share an owner run as one batch, so a rank's load
  is the sum over shapes of T_s(k_s), T_s(k) the time of a batch of k;
* T_s is the piecewise-linear curve through (0, 0) and the profiled points,
  continued past the last point with the last segment's slope, clamped at 0.

Two independent exact solvers: exhaustive enumeration of the per-rank counts
(tiny cases) and the integer program written out for ``scipy.optimize.milp``.
"""

from __future__ import annotations

import itertools

import numpy as np


def batch_time(batches, times_s, k: int) -> float:
    """T_s(k): linear interpolation through (0, 0) and (batches[p], times_s[p])."""
    if k <= 0:
        return 0.0
    xs = [0.0] + [float(b) for b in batches]
    ys = [0.0] + [float(t) for t in times_s]
    j = 1
    while j < len(xs) - 1 and xs[j] < k:
        j += 1
    x0, x1, y0, y1 = xs[j - 1], xs[j], ys[j - 1], ys[j]
    return max(0.0, y0 + (y1 - y0) * (k - x0) / (x1 - x0))


def counts_of(owner, shape_of, nshapes: int, ranks: int):
    """counts[r][s]: matrices of shape s owned by rank r."""
    c = [[0] * nshapes for _ in range(ranks)]
    for o, s in zip(owner, shape_of):
        c[o][s] += 1
    return c


def rank_loads(owner, shape_of, batches, times, ranks: int):
    """Predicted load of every rank for an assignment."""
    c = counts_of(owner, shape_of, len(times), ranks)
    return [sum(batch_time(batches, times[s], c[r][s]) for s in range(len(times))) for r in range(ranks)]


def makespan(owner, shape_of, batches, times, ranks: int) -> float:
    return max(rank_loads(owner, shape_of, batches, times, ranks))


def _compositions(n: int, parts: int):
    """All ways to write n as an ordered sum of `parts` non-negative integers."""
    if parts == 1:
        yield (n,)
        return
    for k in range(n + 1):
        for rest in _compositions(n - k, parts - 1):
            yield (k,) + rest


def brute_force_makespan(shape_of, batches, times, ranks: int) -> float:
    """Minimal makespan by trying every per-rank count of every shape."""
    nshapes = len(times)
    n = [0] * nshapes
    for s in shape_of:
        n[s] += 1
    best = float("inf")
    per_shape = [list(_compositions(n[s], ranks)) for s in range(nshapes)]
    for choice in itertools.product(*per_shape):
        loads = [sum(batch_time(batches, times[s], choice[s][r]) for s in range(nshapes)) for r in range(ranks)]
        best = min(best, max(loads))
    return best


def milp_makespan(shape_of, batches, times, ranks: int) -> float:
    """Minimal makespan from the integer program (scipy's HiGHS MILP).

    Variables: y[r, s, k] in {0, 1} selects how many matrices (k) of shape s
    rank r owns; C is the makespan.  Constraints: one k per (r, s); the counts
    of each shape add up to its number of matrices; every rank's load
    sum_{s, k} T_s(k) y[r, s, k] is at most C.  Objective: minimise C."""
    from scipy.optimize import LinearConstraint, milp

    nshapes = len(times)
    n = [0] * nshapes
    for s in shape_of:
        n[s] += 1
    index = {}
    for r in range(ranks):
        for s in range(nshapes):
            for k in range(n[s] + 1):
                index[(r, s, k)] = len(index)
    nv = len(index) + 1  # last variable: C
    cost = np.zeros(nv)
    cost[-1] = 1.0
    rows, lo, hi = [], [], []
    for r in range(ranks):
        for s in range(nshapes):
            row = np.zeros(nv)
            for k in range(n[s] + 1):
                row[index[(r, s, k)]] = 1.0
            rows.append(row), lo.append(1.0), hi.append(1.0)
    for s in range(nshapes):
        row = np.zeros(nv)
        for r in range(ranks):
            for k in range(n[s] + 1):
                row[index[(r, s, k)]] = float(k)
        rows.append(row), lo.append(float(n[s])), hi.append(float(n[s]))
    for r in range(ranks):
        row = np.zeros(nv)
        for s in range(nshapes):
            for k in range(n[s] + 1):
                row[index[(r, s, k)]] = batch_time(batches, times[s], k)
        row[-1] = -1.0
        rows.append(row), lo.append(-np.inf), hi.append(0.0)
    integrality = np.ones(nv)
    integrality[-1] = 0
    bounds_lo = np.zeros(nv)
    bounds_hi = np.ones(nv)
    bounds_hi[-1] = np.inf
    from scipy.optimize import Bounds

    res = milp(cost, constraints=LinearConstraint(np.array(rows), lo, hi), integrality=integrality,
               bounds=Bounds(bounds_lo, bounds_hi), options={"mip_rel_gap": 0.0})
    if not res.success:
        raise RuntimeError(res.message)
    return float(res.x[-1])
