"""The implicit workspace of the plan-free calls, and a NaN-poisoned workspace.

1. A workspace that the cache outgrows is retired, never freed while a HIP
   graph may still address it; only dmuon_release_workspace frees it.  The
   checks here read the library's bookkeeping (dmuon_workspace_info): no
   captured graph is replayed after growth.
2. Growth while the caller's stream is being captured is refused before
   anything is enqueued.
3. With DMUON_POISON_WORKSPACE=1 every new workspace is filled with 0xFF
   bytes (NaN in fp32, fp16 and bf16).  Lower-stored symmetric states leave
   their upper triangle unwritten (gist.science technical summary, section
   2.2: only the lower triangle of the symmetric products is computed), so a
   kernel that read it, or any other workspace memory before writing it,
   would turn results into NaN.  Poisoned and clean runs must agree bitwise.
"""

import numpy as np
import pytest

import matrix_orthogonalising_optimizer_amd as dm
from matrix_orthogonalising_optimizer_amd import synth
from gpu_util import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dm.load_library()


def test_outgrown_workspace_is_retired_not_freed():
    import torch
    torch.cuda.synchronize()
    dm.release_workspace()
    assert dm.workspace_info() == {"live_bytes": 0, "retired_bytes": 0, "retired_count": 0}
    rng = np.random.default_rng(811)
    small = [to_dev(synth.gaussian(rng, (128, 384), 0.02, "bf16"), "bf16") for _ in range(2)]
    big = [to_dev(synth.gaussian(rng, (512, 1024), 0.02, "bf16"), "bf16") for _ in range(2)]
    dm.ns_batched(small)
    i1 = dm.workspace_info()
    assert i1["live_bytes"] > 0 and i1["retired_count"] == 0
    dm.ns_batched(big)
    i2 = dm.workspace_info()
    assert i2["retired_count"] == 1 and i2["retired_bytes"] == i1["live_bytes"]
    assert i2["live_bytes"] >= i1["live_bytes"] * 3 // 2
    dm.ns_batched(small)  # fits: no growth
    assert dm.workspace_info() == i2
    torch.cuda.synchronize()
    dm.release_workspace()
    assert dm.workspace_info() == {"live_bytes": 0, "retired_bytes": 0, "retired_count": 0}
    dm.ns_batched(small)  # allocates again
    torch.cuda.synchronize()
    assert dm.workspace_info()["live_bytes"] > 0


def test_growth_during_capture_is_refused():
    import torch
    torch.cuda.synchronize()
    dm.release_workspace()
    rng = np.random.default_rng(812)
    mats = [to_dev(synth.gaussian(rng, (256, 512), 0.02, "bf16"), "bf16") for _ in range(2)]
    before = [m.clone() for m in mats]
    x = torch.zeros(16, device="cuda")
    g = torch.cuda.CUDAGraph()
    err = None
    with torch.cuda.graph(g):
        x.add_(1.0)
        try:
            dm.ns_batched(mats)
        except dm.DmuonError as e:
            err = e
    torch.cuda.synchronize()
    assert err is not None and err.code == dm.EUNSUPPORTED, err
    assert "captured" in str(err)
    assert dm.workspace_info()["live_bytes"] == 0
    g.replay()
    torch.cuda.synchronize()
    for a, b in zip(mats, before):
        assert torch.equal(a, b)  # nothing was enqueued or recorded


def _two_steps(shapes, kw, W, G, B):
    import torch
    tw = [to_dev(w, "bf16") for w in W]
    tb = [to_dev(b, "f32") for b in B]
    with dm.Plan(shapes, **kw) as plan:
        desc = plan.describe()
        for G_k in G:
            plan.step(tw, [to_dev(g, "bf16") for g in G_k], tb, lr=0.02, weight_decay=0.1, mu=0.95)
        torch.cuda.synchronize()
    return desc, tw, tb


@pytest.mark.parametrize("shapes,kw", [
    ([(512, 1024), (1024, 512), (512, 512)], {}),          # lower storage, 256 tiles
    ([(256, 768), (768, 256), (256, 256)], {}),            # lower storage, 128 tiles
    ([(768, 1280), (1280, 768)], {}),                      # three K ranges
    ([(128, 512), (100, 300), (96, 96), (300, 700)], {}),  # fused, fp32 and ragged buckets
    ([(200, 600), (220, 660), (640, 200)], {"pad_ratio": 0.25}),  # zero-padded bucket
    ([(256, 256), (300, 500)], {"form": "standard"}),
])
def test_poisoned_workspace_changes_nothing(shapes, kw, monkeypatch):
    import torch
    rng = np.random.default_rng(813 + len(shapes))
    W = [synth.gaussian(rng, s, 0.02, "bf16") for s in shapes]
    G = [[synth.gaussian(rng, s, 0.02, "bf16") for s in shapes] for _ in range(2)]
    B = [np.zeros(s, np.float32) for s in shapes]
    monkeypatch.setenv("DMUON_POISON_WORKSPACE", "0")
    dc, wc, bc = _two_steps(shapes, kw, W, G, B)
    monkeypatch.setenv("DMUON_POISON_WORKSPACE", "1")
    dp, wp, bp = _two_steps(shapes, kw, W, G, B)
    assert dc == dp
    if not kw:
        assert any(b["storage"] == "lower" for b in dp["recurrence"]) or any(b["fused"] for b in dp["recurrence"])
    for i, (a, b) in enumerate(zip(wc, wp)):
        assert bool(torch.isfinite(b.float()).all()), (i, shapes[i])
        assert torch.equal(a, b), (i, shapes[i])
    for a, b in zip(bc, bp):
        assert torch.equal(a, b)
