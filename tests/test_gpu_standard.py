"""GPU parity of the standard-form iteration (plan form "standard", and AUTO's
choice for plain bf16 products on near-square buckets) against the fp64
oracle.  The oracle's standard and Gram forms are equal to 1e-10 (pinned in
test_oracle.py), so either is the reference."""

import numpy as np
import pytest

import oracle
import matrix_orthogonalising_optimizer_amd as dm
from matrix_orthogonalising_optimizer_amd import synth
from gpu_util import TOL_BF16_MFMA, rel, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dm.load_library()


def ns_via_step(shapes, G, precision, form, steps=5, coeffs=oracle.QUINTIC):
    """NS(G) through dmuon_step: W = 0, lr = 1, no decay, no momentum, shape
    factor 1, so the stored parameter is -NS(G)."""
    import torch
    tw = [torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
    tb = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    tg = [to_dev(g, "bf16") for g in G]
    with dm.Plan(shapes, precision=precision, form=form, scale_mode="none") as plan:
        assert all(b["form"] == "standard" for b in plan.describe()["recurrence"] if not b["fp32"])
        plan.step(tw, tg, tb, lr=1.0, weight_decay=0.0, mu=0.0, steps=steps, coeffs=coeffs)
    torch.cuda.synchronize()
    return [-to_host(w) for w in tw]


SHAPES = [(256, 256), (512, 768), (768, 512), (300, 300), (256, 1280)]


@pytest.mark.parametrize("precision", ["f16", "bf16"])
def test_standard_form_matches_oracle(precision):
    rng = np.random.default_rng(401)
    G = [synth.gaussian(rng, s, 0.02, "bf16") for s in SHAPES]
    out = ns_via_step(SHAPES, G, precision, "standard")
    for s, g, o in zip(SHAPES, G, out):
        assert rel(o, oracle.ns_standard(g)) <= TOL_BF16_MFMA, (s, precision)


@pytest.mark.parametrize("steps", [1, 2])
def test_standard_form_few_steps(steps):
    # odd and even step counts end in different buffers of the iterate
    rng = np.random.default_rng(409 + steps)
    shapes = [(384, 512), (512, 384)]
    G = [synth.gaussian(rng, s, 0.02, "bf16") for s in shapes]
    out = ns_via_step(shapes, G, "f16", "standard", steps=steps)
    for s, g, o in zip(shapes, G, out):
        assert rel(o, oracle.ns_standard(g, steps=steps)) <= TOL_BF16_MFMA, (s, steps)


def test_standard_form_full_step_with_momentum():
    import torch
    rng = np.random.default_rng(419)
    shapes = [(512, 512), (640, 512)]
    W = [synth.gaussian(rng, s, 0.02, "bf16") for s in shapes]
    G = [synth.gaussian(rng, s, 0.02, "bf16") for s in shapes]
    B = [rng.standard_normal(s, dtype=np.float32) * np.float32(0.01) for s in shapes]
    tw = [to_dev(w, "bf16") for w in W]
    tg = [to_dev(g, "bf16") for g in G]
    tb = [to_dev(b, "f32") for b in B]
    lr, wd, mu = 0.02, 0.1, 0.95
    with dm.Plan(shapes, form="standard") as plan:
        plan.step(tw, tg, tb, lr=lr, weight_decay=wd, mu=mu)
    torch.cuda.synchronize()
    for i, s in enumerate(shapes):
        Wn, bn, O = oracle.muon_step(W[i], G[i], B[i], lr=lr, weight_decay=wd, mu=mu)
        assert rel(to_host(tb[i]), bn) <= 1e-6
        sc = oracle.shape_scale(*s)
        bound = 2.0 ** -8 * np.linalg.norm(Wn) + lr * sc * TOL_BF16_MFMA * np.linalg.norm(O)
        assert np.linalg.norm(to_host(tw[i]) - Wn) <= bound, s


def test_auto_picks_standard_for_bf16_square_and_stays_accurate():
    # plain bf16 products: the Gram form misses 2e-2 on square matrices, the
    # standard form that AUTO picks there does not
    rng = np.random.default_rng(421)
    shapes = [(512, 512)]
    G = [synth.gaussian(rng, s, 0.02, "bf16") for s in shapes]
    d = dm.Plan(shapes, precision="bf16", device=False).describe()
    assert d["recurrence"][0]["form"] == "standard"
    t = to_dev(G[0], "bf16")
    dm.ns_batched([t], precision="bf16")
    import torch
    torch.cuda.synchronize()
    assert rel(to_host(t), oracle.ns_standard(G[0])) <= TOL_BF16_MFMA


def test_standard_and_gram_forms_agree():
    rng = np.random.default_rng(431)
    shapes = [(512, 1024), (1024, 512)]
    G = [synth.gaussian(rng, s, 0.02, "bf16") for s in shapes]
    a = ns_via_step(shapes, G, "f16", "standard")
    import torch
    tw = [torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
    tb = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    with dm.Plan(shapes, form="gram", scale_mode="none") as plan:
        plan.step(tw, [to_dev(g, "bf16") for g in G], tb, lr=1.0, weight_decay=0.0, mu=0.0)
    torch.cuda.synchronize()
    for x, w in zip(a, tw):
        assert rel(x, -to_host(w)) <= 2 * TOL_BF16_MFMA / 4
