"""Multi-problem launches: the Gram products of all shape groups of a bucket,
and their final products, run as a few launches of up to four problems each
(problems of one launch may differ in every dimension).  Checked against the
fp64 oracle, including buckets with more groups than one launch holds and
groups whose caller pointers overflow one launch's table."""

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


def check_step(shapes, seed, sample=None, **plan_kw):
    import torch
    rng = np.random.default_rng(seed)
    W = [synth.gaussian(rng, s, 0.02, "bf16") for s in shapes]
    G = [synth.gaussian(rng, s, 0.02, "bf16") for s in shapes]
    B = [rng.standard_normal(s, dtype=np.float32) * np.float32(0.01) for s in shapes]
    tw = [to_dev(w, "bf16") for w in W]
    tg = [to_dev(g, "bf16") for g in G]
    tb = [to_dev(b, "f32") for b in B]
    lr, wd, mu = 0.02, 0.1, 0.95
    with dm.Plan(shapes, **plan_kw) as plan:
        desc = plan.describe()
        plan.step(tw, tg, tb, lr=lr, weight_decay=wd, mu=mu)
    torch.cuda.synchronize()
    idx = range(len(shapes)) if sample is None else sample
    for i in idx:
        s = shapes[i]
        Wn, bn, O = oracle.muon_step(W[i], G[i], B[i], lr=lr, weight_decay=wd, mu=mu)
        assert rel(to_host(tb[i]), bn) <= 1e-6, (i, s)
        bound = 2.0 ** -8 * np.linalg.norm(Wn) + lr * oracle.shape_scale(*s) * TOL_BF16_MFMA * np.linalg.norm(O)
        assert np.linalg.norm(to_host(tw[i]) - Wn) <= bound, (i, s)
    return desc


def test_groups_of_one_bucket_share_launches():
    # one m = 512 bucket of four shape groups, both orientations
    shapes = [(512, 512), (512, 1024), (1024, 512), (512, 768), (512, 512), (768, 512)]
    d = check_step(shapes, 611)
    assert len(d["recurrence"]) == 1 and len(d["gemm"]) == 5


def test_more_groups_than_one_launch_holds():
    # six groups in the m = 384 bucket (tile 128): two Gram launches
    shapes = [(384, 384), (384, 512), (512, 384), (384, 640), (640, 384), (384, 896)]
    d = check_step(shapes, 613)
    assert len(d["recurrence"]) == 1 and len(d["gemm"]) == 6


def test_caller_pointer_table_overflow_splits_launches():
    # 2 x 40 wide matrices of one bucket: their final products need 80 caller
    # pointers, more than one launch carries
    shapes = [(256, 512)] * 40 + [(256, 768)] * 40
    check_step(shapes, 617, sample=[0, 39, 40, 79])


def test_padded_bucket_with_several_groups():
    shapes = [(448, 1024), (480, 960), (512, 512), (496, 1488)]
    d = check_step(shapes, 619, pad_ratio=0.25)
    assert len(d["recurrence"]) == 1


def test_standard_form_groups_share_launches():
    shapes = [(512, 512), (512, 768), (768, 512), (512, 640)]
    d = check_step(shapes, 623, form="standard")
    assert all(b["form"] == "standard" for b in d["recurrence"])
