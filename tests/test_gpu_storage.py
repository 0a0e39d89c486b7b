"""Lower-triangle storage of the symmetric states: the products read the
upper part of a row panel transposed from the stored lower blocks instead of
a mirrored copy.  The same values reach the same MFMAs in the same order, so
the results must equal those of full storage bit for bit; accuracy against
the fp64 oracle is covered for the default (lower) storage by the other
parity tests and checked here once more."""

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


def step_with(storage, shapes, W, G, B, steps=5):
    import torch
    tw = [to_dev(w, "bf16") for w in W]
    tg = [to_dev(g, "bf16") for g in G]
    tb = [to_dev(b, "f32") for b in B]
    with dm.Plan(shapes, storage=storage) as plan:
        d = plan.describe()["recurrence"]
        plan.step(tw, tg, tb, lr=0.02, weight_decay=0.1, mu=0.95, steps=steps)
    torch.cuda.synchronize()
    return d, tw, tb


@pytest.mark.parametrize("shapes", [
    [(512, 1024), (1024, 512), (512, 512)],      # tile 256, both orientations
    [(256, 768), (768, 256), (256, 256)],        # tile 128
    [(768, 1280), (1280, 768)],                  # 3 x 3 tiles: all three K ranges
])
def test_lower_storage_matches_full_bitwise(shapes):
    import torch
    rng = np.random.default_rng(sum(r * 7 + c for r, c in shapes))
    W = [synth.gaussian(rng, s, 0.02, "bf16") for s in shapes]
    G = [synth.gaussian(rng, s, 0.02, "bf16") for s in shapes]
    B = [rng.standard_normal(s, dtype=np.float32) * np.float32(0.01) for s in shapes]
    dl, wl, bl = step_with("auto", shapes, W, G, B)
    df, wf, bf = step_with("full", shapes, W, G, B)
    assert all(b["storage"] == "lower" for b in dl), dl
    assert all(b["storage"] == "full" for b in df)
    for s, a, b in zip(shapes, wl, wf):
        assert torch.equal(a, b), s
    for s, a, b in zip(shapes, bl, bf):
        assert torch.equal(a, b), s


@pytest.mark.parametrize("steps", [1, 2, 5])
def test_lower_storage_matches_oracle(steps):
    # NS alone (W = 0, lr = 1, no decay or momentum, shape factor 1): the
    # stored parameter is -NS(G)
    import torch
    shapes = [(768, 1280), (1280, 768)]
    rng = np.random.default_rng(4421 + steps)
    G = [synth.gaussian(rng, s, 0.02, "bf16") for s in shapes]
    tw = [torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
    tb = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    with dm.Plan(shapes, scale_mode="none") as plan:
        assert plan.describe()["recurrence"][0]["storage"] == "lower"
        plan.step(tw, [to_dev(g, "bf16") for g in G], tb, lr=1.0, weight_decay=0.0, mu=0.0, steps=steps)
    torch.cuda.synchronize()
    for s, g, w in zip(shapes, G, tw):
        assert rel(-to_host(w), oracle.ns_gram(g, steps=steps)) <= TOL_BF16_MFMA, (s, steps)
