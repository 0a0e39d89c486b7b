"""GPU parity of similar-shape padded batching (plan option pad_ratio) against
the fp64 oracle on the unpadded matrices: zero rows add zero eigenvalues that
never mix with the others, so results equal the unpadded ones."""

import numpy as np
import pytest

import oracle
import matrix_orthogonalising_optimizer_amd as dm
from matrix_orthogonalising_optimizer_amd import synth
from gpu_util import TOL_BF16_MFMA, rel, to_dev, to_host

pytestmark = pytest.mark.gpu

SHAPES = [(240, 512), (256, 640), (300, 300), (512, 200), (1000, 1000), (2048, 1024)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dm.load_library()


@pytest.mark.parametrize("form", ["gram", "standard"])
@pytest.mark.parametrize("steps", [1, 5])
def test_padded_plan_matches_oracle(form, steps):
    import torch
    rng = np.random.default_rng(503 + steps)
    G = [synth.gaussian(rng, s, 0.02, "bf16") for s in SHAPES]
    tw = [torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in SHAPES]
    tb = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in SHAPES]
    tg = [to_dev(g, "bf16") for g in G]
    with dm.Plan(SHAPES, form=form, pad_ratio=0.25, scale_mode="none") as plan:
        d = plan.describe()
        assert any(b["m"] > g["m"] for g in d["gemm"] for b in [d["recurrence"][g["rec"]]])
        for _ in range(2):  # the second call reuses the workspace: padded rows must be zero again
            for t in tw:
                t.zero_()
            plan.step(tw, tg, tb, lr=1.0, weight_decay=0.0, mu=0.0, steps=steps)
    torch.cuda.synchronize()
    for s, g, w in zip(SHAPES, G, tw):
        assert rel(-to_host(w), oracle.ns_gram(g, steps=steps)) <= TOL_BF16_MFMA, (s, form, steps)
