"""GPU parity of the fused AdamW step (dmuon_adamw_step) against the fp64 oracle.

AdamW is the baseline optimizer of the pages' overhead comparison
(gist.science technical summary, section 4).  Three consecutive steps run on
the GPU and in the oracle from the same initial weights and gradient
sequence; the oracle carries its own fp64 state between steps.

Bounds: the moments are fp32 on the GPU, rounded a few times per step.  The
rounding error of m scales with its terms, not with m itself (m = beta1 m +
(1 - beta1) g can cancel to nearly zero), so it is bounded by 1e-5 of the
same recursion run on |g| (all terms positive); v has no cancellation and is
bounded relative to itself.  Both bounds sit far below a misplaced beta or
bias correction, which moves the moments by O(0.1) of their size.  A bf16
weight is rounded once per step and the error of earlier steps is carried
along (times 1 - lr wd), so the bound is a running sum over the steps of one
bf16 ulp of that step's weight, 1e-5 of the update term and the update's
share of m's error bound (a weight that passes near zero has a much smaller
ulp than the error it carries).  fp32 weights: the same sum with 1e-6 of |W|
in place of the ulp.
"""

import numpy as np
import pytest

import oracle
import matrix_orthogonalising_optimizer_amd as dm
from matrix_orthogonalising_optimizer_amd import synth
from gpu_util import to_dev, to_host

pytestmark = pytest.mark.gpu

LR, B1, B2, EPS, WD = 1e-3, 0.9, 0.95, 1e-8, 0.1


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dm.load_library()


def ulp_bf16(x):
    a = np.abs(np.asarray(x, np.float64))
    return 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -126))) - 7)


def run_steps(shapes, dtype, steps=3, offset=0, seed=1):
    """Run `steps` AdamW steps on the GPU and in the oracle; check each step.
    offset > 0 places every tensor `offset` elements into a larger buffer, so
    that no pointer is 16-byte aligned (element-wise path)."""
    import torch
    rng = np.random.default_rng(seed)
    W0 = [synth.gaussian(rng, s, 0.05, dtype) for s in shapes]
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32

    def alloc(x, dt):
        flat = torch.zeros(int(np.prod(x.shape)) + offset, dtype=dt, device="cuda")
        v = flat[offset:].view(x.shape)
        v.copy_(torch.from_numpy(np.ascontiguousarray(x, np.float32)).to("cuda").to(dt))
        return v

    tw = [alloc(w, tdt) for w in W0]
    tm = [alloc(np.zeros(s, np.float32), torch.float32) for s in shapes]
    tv = [alloc(np.zeros(s, np.float32), torch.float32) for s in shapes]
    W = [w.astype(np.float64) for w in W0]
    M = [np.zeros(s) for s in shapes]
    V = [np.zeros(s) for s in shapes]
    Mag = [np.zeros(s) for s in shapes]  # the m recursion on |g|: scale of m's rounding error
    Eb = [np.zeros(s) for s in shapes]   # running error bound of the weight
    for t in range(1, steps + 1):
        G = [synth.gaussian(rng, s, 10.0 ** -rng.integers(1, 4), dtype) for s in shapes]
        tg = [alloc(g, tdt) for g in G]
        dm.adamw_step(tw, tg, tm, tv, lr=LR, step=t, betas=(B1, B2), eps=EPS, weight_decay=WD)
        torch.cuda.synchronize()
        for i, s in enumerate(shapes):
            Wn, M[i], V[i] = oracle.adamw_step(W[i], G[i], M[i], V[i], step=t, lr=LR, beta1=B1, beta2=B2,
                                               eps=EPS, weight_decay=WD)
            upd = np.abs(Wn - W[i] * (1 - LR * WD))
            W[i] = Wn
            Mag[i] = B1 * Mag[i] + (1 - B1) * np.abs(G[i])
            m_tol = 1e-5 * Mag[i]
            assert not (np.abs(to_host(tm[i]) - M[i]) > m_tol).any(), (t, i, s, "m")
            np.testing.assert_allclose(to_host(tv[i]), V[i], rtol=1e-5, atol=0.0)
            # m's error bound carried through the update term
            upd_m = LR * (m_tol / (1 - B1 ** t)) / (np.sqrt(V[i] / (1 - B2 ** t)) + EPS)
            got = to_host(tw[i])
            rounding = ulp_bf16(Wn) if dtype == "bf16" else 1e-6 * np.abs(Wn) + 1e-12
            Eb[i] = (1 - LR * WD) * Eb[i] + rounding + 1e-5 * upd + upd_m
            bad = np.abs(got - Wn) > Eb[i]
            assert not bad.any(), (t, i, s, int(bad.sum()))
    return tw


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_adamw_matches_oracle(dtype):
    # whole 16-byte groups, a ragged tail, a tensor smaller than one group,
    # one spanning several 8192-element blocks, a vector
    shapes = [(256, 512), (300, 77), (3, 5), (1000, 1003), (1, 9001)]
    run_steps(shapes, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_adamw_unaligned_tensors(dtype):
    run_steps([(64, 100), (37, 41)], dtype, offset=1, seed=2)


def test_adamw_more_tensors_than_one_launch_carries():
    run_steps([(16, 24 + i % 5) for i in range(150)], "bf16", steps=2, seed=3)


def test_adamw_aligned_equals_unaligned_bitwise():
    # the 16-byte and element-wise paths do the same arithmetic per element
    import torch
    a = run_steps([(128, 384), (50, 70)], "bf16", steps=2, seed=4)
    b = run_steps([(128, 384), (50, 70)], "bf16", steps=2, seed=4, offset=1)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
