"""GPU parity on the benchmark's own inputs and plans (through the C ABI).

The benchmark times dmuon_step over dense seeded Gaussian gradients in the
weight shapes of its workloads.  Here the same gradients (the first draw of
the workload's seed, synth.workload) go through a plan of the same shapes in
the same order and with the same tile table (the measured table shipped with
the package, when there is one), so every launch has the configuration the
benchmark times:
the same buckets, tiles, storage, multi-problem launches and lockstep
recurrences.  Only the step's scalars differ: W = 0, lr = 1 and no weight
decay, so that the stored parameter is -s(rows, cols) O, where O is the
orthogonalised Nesterov update (gist.science technical summary, section 2.2:
Gram-space recurrence, symmetric products, batching of like shapes; sections
1 and 5: Newton-Schulz applied to the momentum-aggregated gradient).  O is
compared with the fp64 oracle's Muon step on the same input, one or more
sampled matrices per distinct shape, at the bf16 MFMA tolerance (relative
Frobenius error 2e-2).  The errors are printed.

Momentum starts at zero with mu = 0.95, as in the benchmark: the first step's
update is (1 + mu) G, whose normalised map equals that of G up to eps.
"""

import numpy as np
import pytest

import oracle
import matrix_orthogonalising_optimizer_amd as dm
from matrix_orthogonalising_optimizer_amd import synth
from matrix_orthogonalising_optimizer_amd.autotune import shipped_table
from gpu_util import TOL_BF16_MFMA, rel, to_dev, to_host

pytestmark = pytest.mark.gpu

MU = 0.95


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dm.load_library()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def step_outputs(shapes, G):
    """Run one dmuon_step of the benchmark's plan with W = 0, lr = 1, wd = 0;
    return (plan description, device parameters, device momenta)."""
    import torch
    tg = [to_dev(g, "bf16") for g in G]
    tw = [torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
    tb = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    with dm.Plan(shapes, tune_path=shipped_table()) as plan:
        desc = plan.describe()
        plan.step(tw, tg, tb, lr=1.0, weight_decay=0.0, mu=MU)
        torch.cuda.synchronize()
    del tg
    return desc, tw, tb


def check_member(i, shape, g, w, b):
    """O of matrix i from the stored parameter, against the oracle."""
    W0 = np.zeros(shape)
    _, bn, O = oracle.muon_step(W0, g, np.zeros(shape), lr=1.0, weight_decay=0.0, mu=MU)
    assert rel(to_host(b), bn) <= 1e-6, (i, shape)
    got = -to_host(w) / oracle.shape_scale(*shape)
    assert np.all(np.isfinite(got)), (i, shape)
    e = rel(got, O)
    print(f"matrix {i} {shape[0]}x{shape[1]}: relative error {e:.3e}", flush=True)
    assert e <= TOL_BF16_MFMA, (i, shape, e)
    return e


def test_llama7b_layer_dense_gradients():
    """4 x 4096^2 and 3 x (11008 x 4096 / 4096 x 11008): one m = 4096 recurrence
    bucket of 7, Gram and final products of the three shape groups in
    multi-problem launches.  Every matrix is checked."""
    G, _ = synth.workload("llama7b_layer")
    shapes = [g.shape for g in G]
    desc, tw, tb = step_outputs(shapes, G)
    rec = desc["recurrence"]
    assert len(rec) == 1 and rec[0]["m"] == 4096 and rec[0]["count"] == 7, rec
    print(f"7B layer plan: {rec}", flush=True)
    errs = [check_member(i, s, G[i], tw[i], tb[i]) for i, s in enumerate(shapes)]
    print(f"7B layer: max relative error {max(errs):.3e}", flush=True)


def test_vla_mix_full_plan_sampled():
    """All 200 matrices through the benchmark's plan: 256^2, 1024^2 and
    1024 x 4096 (which share the m = 1024 recurrence bucket) and 2048 x 8192;
    buckets with the same tile run their recurrences in lockstep launches.
    Three members of every shape group (first, middle, last) are checked
    against the oracle."""
    G, _ = synth.workload("vla_mix_200")
    shapes = [g.shape for g in G]
    desc, tw, tb = step_outputs(shapes, G)
    by_m = {b["m"]: b for b in desc["recurrence"]}
    assert sorted(by_m) == [256, 1024, 2048], by_m.keys()
    assert by_m[1024]["count"] == 100 and by_m[256]["count"] == 50 and by_m[2048]["count"] == 50
    print(f"VLA plan: {desc['recurrence']}", flush=True)
    groups = {}
    for i, s in enumerate(shapes):
        groups.setdefault(s, []).append(i)
    errs = []
    for s, idx in groups.items():
        for i in sorted({idx[0], idx[len(idx) // 2], idx[-1]}):
            errs.append(check_member(i, s, G[i], tw[i], tb[i]))
    print(f"VLA mix: max relative error {max(errs):.3e}", flush=True)


def test_mlp70b_dense_gradient():
    """The 70B MLP plan (8 x 8192 x 28672) on one dense seeded gradient,
    repeated in all eight slots: every output must equal the first bitwise
    (batch members are independent), and the first matches the oracle."""
    import torch
    G1, _ = synth.workload("mlp70b_8x8192x28672", count=1)
    shapes = synth.WORKLOADS["mlp70b_8x8192x28672"][0]
    g = G1[0]
    tg = to_dev(g, "bf16")
    tgs = [tg] + [tg.clone() for _ in shapes[1:]]
    tw = [torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
    tb = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    with dm.Plan(shapes, tune_path=shipped_table()) as plan:
        rec = plan.describe()["recurrence"]
        assert len(rec) == 1 and rec[0]["m"] == 8192 and rec[0]["count"] == 8
        plan.step(tw, tgs, tb, lr=1.0, weight_decay=0.0, mu=MU)
        torch.cuda.synchronize()
    del tgs, tg
    for i in range(1, len(shapes)):
        assert torch.equal(tw[i], tw[0]), i
    check_member(0, shapes[0], g, tw[0], tb[0])


def test_llama7b_layer_plan_ns():
    """The NS call the benchmark's --mode ns times on the 7B layer:
    dmuon_plan_ns over the same seven gradients in one plan (one m = 4096
    recurrence bucket of 7).  One matrix per distinct shape is compared with
    the oracle's Gram NS of its input."""
    import torch
    G, _ = synth.workload("llama7b_layer")
    shapes = [g.shape for g in G]
    ts = [to_dev(g, "bf16") for g in G]
    with dm.Plan(shapes, tune_path=shipped_table()) as plan:
        rec = plan.describe()["recurrence"]
        assert len(rec) == 1 and rec[0]["m"] == 4096 and rec[0]["count"] == 7, rec
        plan.ns(ts)
        torch.cuda.synchronize()
    seen = set()
    for i, s in enumerate(shapes):
        if s in seen:
            continue
        seen.add(s)
        got = to_host(ts[i])
        assert np.all(np.isfinite(got)), (i, s)
        e = rel(got, oracle.ns_gram(G[i].astype(np.float64)))
        print(f"plan ns matrix {i} {s[0]}x{s[1]}: relative error {e:.3e}", flush=True)
        assert e <= TOL_BF16_MFMA, (i, s, e)
