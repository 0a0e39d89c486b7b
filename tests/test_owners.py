"""Owner assignment: the oracle against its pins, and dmuon_assign_owners
(host-only C ABI) against the oracle's exact optima.

The pages (gist.science/pt, technical summary section 2.3) fix the objective
-- the smallest predicted makespan over owner assignments, with costs profiled
per shape and batch size -- and name an integer program with a greedy
fallback.  The oracle solves the same problem twice, by exhaustive enumeration
and by the integer program, and both are pinned to hand-solved instances.
"""

import math
import os

import numpy as np
import pytest

import matrix_orthogonalising_optimizer_amd as dm
from oracle import owners as O


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dm.library_path()):
        pytest.fail("libdmuon.so is not built: run __graft_entry__.build()")
    return dm.load_library()


# ---------------------------------------------------------------- oracle pins
def test_batch_time_is_the_piecewise_linear_curve():
    b, t = [1, 4], [2.0, 5.0]
    assert O.batch_time(b, t, 0) == 0.0
    assert O.batch_time(b, t, 1) == 2.0
    assert O.batch_time(b, t, 2) == pytest.approx(3.0)   # on the segment (1, 2) -> (4, 5)
    assert O.batch_time(b, t, 4) == 5.0
    assert O.batch_time(b, t, 6) == pytest.approx(7.0)   # past the last point: slope 1
    assert O.batch_time([2], [3.0], 1) == pytest.approx(1.5)  # through the origin
    assert O.batch_time([1, 2], [4.0, 1.0], 5) == 0.0     # a falling curve clamps at 0


def test_partition_instance_by_hand():
    # six single-matrix shapes of cost 3, 1, 1, 2, 2, 1 on two ranks: 10 / 2 = 5
    times = [[3.0], [1.0], [1.0], [2.0], [2.0], [1.0]]
    so = list(range(6))
    assert O.brute_force_makespan(so, [1], times, 2) == pytest.approx(5.0)
    assert O.milp_makespan(so, [1], times, 2) == pytest.approx(5.0)


def test_identical_linear_items_by_hand():
    # 7 matrices of cost 2 on 3 ranks: ceil(7 / 3) * 2
    so = [0] * 7
    assert O.brute_force_makespan(so, [1], [[2.0]], 3) == pytest.approx(6.0)
    assert O.milp_makespan(so, [1], [[2.0]], 3) == pytest.approx(6.0)


def test_batching_instance_by_hand():
    # one shape, 4 matrices, T(1..4) = 4, 6, 7, 8; two ranks: (4, 0) -> 8,
    # (3, 1) -> max(7, 4) = 7, (2, 2) -> 6
    so = [0] * 4
    times = [[4.0, 6.0, 8.0]]
    assert O.brute_force_makespan(so, [1, 2, 4], times, 2) == pytest.approx(6.0)
    assert O.milp_makespan(so, [1, 2, 4], times, 2) == pytest.approx(6.0)


def random_instance(rng, count, nshapes, ranks, npts, linear=False):
    so = [int(x) for x in rng.integers(0, nshapes, size=count)]
    batches = [1] if linear else sorted(set(int(x) for x in rng.integers(1, 9, size=npts)) | {1})
    times = []
    for _ in range(nshapes):
        t1 = float(rng.uniform(0.5, 10.0))
        if linear:
            times.append([t1])
        else:
            # mostly concave (batching amortises), sometimes not
            ts, prev = [], 0.0
            for bsz in batches:
                v = t1 * bsz ** float(rng.uniform(0.4, 1.1))
                ts.append(max(v, prev * 0.9))
                prev = ts[-1]
            times.append(ts)
    return so, batches, times


@pytest.mark.parametrize("seed", range(8))
def test_oracle_solvers_agree(seed):
    rng = np.random.default_rng(500 + seed)
    so, b, t = random_instance(rng, int(rng.integers(2, 7)), int(rng.integers(1, 4)), int(rng.integers(1, 4)), 3)
    ranks = int(rng.integers(1, 4))
    assert O.milp_makespan(so, b, t, ranks) == pytest.approx(O.brute_force_makespan(so, b, t, ranks), rel=1e-9)


# ---------------------------------------------------------------- the C ABI
def check_assignment(owners, so, b, t, ranks, mk):
    assert len(owners) == len(so)
    assert all(0 <= o < ranks for o in owners)
    assert O.makespan(owners, so, b, t, ranks) == pytest.approx(mk, rel=1e-9, abs=1e-12)


@pytest.mark.parametrize("seed", range(30))
def test_exact_matches_brute_force(lib, seed):
    rng = np.random.default_rng(1000 + seed)
    count, ranks = int(rng.integers(1, 9)), int(rng.integers(1, 4))
    so, b, t = random_instance(rng, count, int(rng.integers(1, 4)), ranks, int(rng.integers(1, 4)))
    owners, mk, opt = dm.assign_owners(so, b, t, ranks, method="exact")
    assert opt
    check_assignment(owners, so, b, t, ranks, mk)
    assert mk == pytest.approx(O.brute_force_makespan(so, b, t, ranks), rel=1e-9, abs=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_exact_matches_integer_program(lib, seed):
    rng = np.random.default_rng(2000 + seed)
    so, b, t = random_instance(rng, 16, 4, 4, 3)
    owners, mk, opt = dm.assign_owners(so, b, t, 4, method="exact")
    assert opt
    check_assignment(owners, so, b, t, 4, mk)
    assert mk == pytest.approx(O.milp_makespan(so, b, t, 4), rel=1e-7)


@pytest.mark.parametrize("seed", range(10))
def test_greedy_is_within_the_lpt_bound_for_linear_costs(lib, seed):
    # with batch-independent per-matrix costs the greedy is longest-processing-
    # time-first, whose makespan is at most (4/3 - 1/(3R)) of the optimum
    rng = np.random.default_rng(3000 + seed)
    ranks = int(rng.integers(2, 4))
    so, b, t = random_instance(rng, int(rng.integers(3, 9)), int(rng.integers(2, 5)), ranks, 1, linear=True)
    owners, mk, opt = dm.assign_owners(so, b, t, ranks, method="greedy")
    assert not opt
    check_assignment(owners, so, b, t, ranks, mk)
    best = O.brute_force_makespan(so, b, t, ranks)
    assert best - 1e-12 <= mk <= (4.0 / 3.0 - 1.0 / (3 * ranks)) * best + 1e-9


def test_exact_improves_on_greedy_where_batching_matters(lib):
    # two shapes; batching makes splitting the big shape costly.  Greedy puts
    # the first A on rank 0 and the first B on rank 1, then keeps splitting.
    so = [0, 0, 0, 0, 1, 1]
    b, t = [1, 4], [[10.0, 12.0], [6.0, 24.0]]
    g, mg, _ = dm.assign_owners(so, b, t, 2, method="greedy")
    e, me, opt = dm.assign_owners(so, b, t, 2, method="exact")
    assert opt and me <= mg
    assert me == pytest.approx(O.brute_force_makespan(so, b, t, 2))
    check_assignment(e, so, b, t, 2, me)


def test_node_limit_returns_the_incumbent(lib):
    rng = np.random.default_rng(77)
    so, b, t = random_instance(rng, 40, 5, 6, 3)
    _, mg, _ = dm.assign_owners(so, b, t, 6, method="greedy")
    owners, mk, opt = dm.assign_owners(so, b, t, 6, method="exact", node_limit=1)
    assert not opt and mk == pytest.approx(mg)
    check_assignment(owners, so, b, t, 6, mk)


def test_auto_on_the_vla_mix(lib):
    # 200 matrices in four shapes on 8 ranks: AUTO takes the greedy path.
    # Costs from the algorithmic flop count at 1 PFLOP/s plus 20 us per launch.
    from matrix_orthogonalising_optimizer_amd import synth
    import bench
    shapes = synth.WORKLOADS["vla_mix_200"][0]
    distinct = sorted(set(shapes))
    so = [distinct.index(s) for s in shapes]
    b = [1, 8, 64]
    t = [[0.02 + k * bench.ns_flops(r, c, 5) / 1e12 for k in b] for r, c in distinct]
    owners, mk, opt = dm.assign_owners(so, b, t, 8)
    check_assignment(owners, so, b, t, 8, mk)
    # lower bound: every shape's total work at its cheapest per-matrix rate, spread evenly
    lb = sum(so.count(s) * min(O.batch_time(b, t[s], k) / k for k in range(1, so.count(s) + 1))
             for s in range(len(distinct))) / 8
    assert lb <= mk <= 1.5 * lb
    assert dm.assign_owners(so, b, t, 8) == (owners, mk, opt)  # deterministic


def test_single_rank_and_more_ranks_than_matrices(lib):
    so, b, t = [0, 1, 1], [1, 2], [[3.0, 5.0], [1.0, 1.5]]
    owners, mk, opt = dm.assign_owners(so, b, t, 1)
    assert owners == [0, 0, 0] and mk == pytest.approx(4.5) and opt
    owners, mk, opt = dm.assign_owners(so, b, t, 5)
    assert opt and mk == pytest.approx(3.0)
    check_assignment(owners, so, b, t, 5, mk)


def test_assign_validates_arguments(lib):
    import ctypes
    i32 = ctypes.c_int32
    so = (i32 * 2)(0, 1)
    bt = (i32 * 2)(1, 2)
    tm = (ctypes.c_double * 4)(1.0, 2.0, 1.0, 2.0)
    out = (i32 * 2)()
    f = lib.dmuon_assign_owners
    assert f(so, 2, bt, 2, tm, 2, 2, 0, 0, out, None, None) == dm.OK
    assert f(None, 2, bt, 2, tm, 2, 2, 0, 0, out, None, None) == dm.EINVAL
    assert f(so, 0, bt, 2, tm, 2, 2, 0, 0, out, None, None) == dm.EINVAL
    assert f(so, 2, bt, 2, tm, 2, 0, 0, 0, out, None, None) == dm.EINVAL      # ranks
    assert f(so, 2, bt, 2, tm, 2, 2, 9, 0, out, None, None) == dm.EINVAL      # method
    assert f(so, 2, bt, 2, tm, 1, 2, 0, 0, out, None, None) == dm.EINVAL      # shape index 1 of 1
    bad = (i32 * 2)(2, 2)
    assert f(so, 2, bad, 2, tm, 2, 2, 0, 0, out, None, None) == dm.EINVAL     # not increasing
    neg = (ctypes.c_double * 4)(1.0, -2.0, 1.0, 2.0)
    assert f(so, 2, bt, 2, neg, 2, 2, 0, 0, out, None, None) == dm.EINVAL
    nan = (ctypes.c_double * 4)(1.0, math.nan, 1.0, 2.0)
    assert f(so, 2, bt, 2, nan, 2, 2, 0, 0, out, None, None) == dm.EINVAL
    assert "finite" in lib.dmuon_last_error().decode()


# ---------------------------------------------------------------- profiling (GPU)
@pytest.mark.gpu
def test_profile_costs_feed_the_assignment():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dm.load_library()
    shapes = [(128, 256), (512, 256), (256, 1024)]
    batches = [1, 2, 4]
    times = dm.profile_costs(shapes, batches, repeats=3)
    assert len(times) == 3 and all(len(r) == 3 for r in times)
    assert all(math.isfinite(x) and x > 0 for r in times for x in r)
    so = [0] * 5 + [1] * 3 + [2] * 4
    owners, mk, opt = dm.assign_owners(so, batches, times, 3)
    assert opt
    check_assignment(owners, so, batches, times, 3, mk)
    with pytest.raises(dm.DmuonError):
        dm.profile_costs(shapes, [2, 1])
