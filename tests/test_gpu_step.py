"""GPU parity of dmuon_step (fused Muon update) against the fp64 oracle."""

import math

import numpy as np
import pytest

import oracle
import matrix_orthogonalising_optimizer_amd as dm
from matrix_orthogonalising_optimizer_amd import synth
from gpu_util import TOL_BF16_MFMA, TOL_F32, block_expect, rel, to_dev, to_host

pytestmark = pytest.mark.gpu

LR, WD, MU = 0.02, 0.1, 0.95


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dm.load_library()


def make_state(rng, shapes, dtype, w_sigma=0.02):
    W = [synth.gaussian(rng, s, w_sigma, dtype) for s in shapes]
    G = [synth.gaussian(rng, s, 0.02, dtype) for s in shapes]
    B = [rng.standard_normal(s, dtype=np.float32) * np.float32(0.01) for s in shapes]
    return W, G, B


def step_gpu(plan, W, G, B, dtype, **kw):
    import torch
    tw = [to_dev(x, dtype) for x in W]
    tg = [to_dev(x, dtype) for x in G]
    tb = [to_dev(x, "f32") for x in B]
    plan.step(tw, tg, tb, **kw)
    torch.cuda.synchronize()
    return [to_host(t) for t in tw], [to_host(t) for t in tb]


SHAPES = [(300, 700), (700, 300), (256, 256), (300, 700), (64, 1000)]


@pytest.mark.parametrize("nesterov", [True, False])
def test_step_f32_params(nesterov):
    rng = np.random.default_rng(61)
    W, G, B = make_state(rng, SHAPES, "f32")
    with dm.Plan(SHAPES, dtype="f32") as plan:
        Wg, Bg = step_gpu(plan, W, G, B, "f32", lr=LR, weight_decay=WD, mu=MU, nesterov=nesterov)
    for i, s in enumerate(SHAPES):
        Wn, bn, O = oracle.muon_step(W[i], G[i], B[i], lr=LR, weight_decay=WD, mu=MU, nesterov=nesterov)
        assert rel(Bg[i], bn) <= 1e-6
        dW_gpu = Wg[i] - W[i].astype(np.float64) * (1 - LR * WD)
        dW_ref = Wn - W[i].astype(np.float64) * (1 - LR * WD)
        assert rel(dW_gpu, dW_ref) <= TOL_F32, (i, s)


def test_step_bf16_update_isolated():
    # W = 0, no decay, lr = 1: the stored parameter is -s(rows, cols) O itself
    rng = np.random.default_rng(67)
    _, G, B = make_state(rng, SHAPES, "bf16")
    W = [np.zeros(s, np.float32) for s in SHAPES]
    with dm.Plan(SHAPES) as plan:
        Wg, Bg = step_gpu(plan, W, G, B, "bf16", lr=1.0, weight_decay=0.0, mu=MU)
    for i, s in enumerate(SHAPES):
        _, bn, O = oracle.muon_step(W[i], G[i], B[i], lr=1.0, weight_decay=0.0, mu=MU)
        assert rel(Bg[i], bn) <= 1e-6
        sc = oracle.shape_scale(*s)
        assert rel(-Wg[i] / sc, O) <= TOL_BF16_MFMA, (i, s)


def test_step_bf16_full_update():
    # bf16 parameters: error = bf16 rounding of W (half an ulp) + lr s |O error|
    rng = np.random.default_rng(71)
    W, G, B = make_state(rng, SHAPES, "bf16")
    with dm.Plan(SHAPES) as plan:
        Wg, Bg = step_gpu(plan, W, G, B, "bf16", lr=LR, weight_decay=WD, mu=MU)
    for i, s in enumerate(SHAPES):
        Wn, bn, O = oracle.muon_step(W[i], G[i], B[i], lr=LR, weight_decay=WD, mu=MU)
        sc = oracle.shape_scale(*s)
        bound = 2.0 ** -8 * np.linalg.norm(Wn) + LR * sc * TOL_BF16_MFMA * np.linalg.norm(O)
        assert np.linalg.norm(Wg[i] - Wn) <= bound, (i, s)


def test_step_zero_steps_and_scale_none():
    rng = np.random.default_rng(73)
    shapes = [(120, 40), (40, 120)]
    W, G, B = make_state(rng, shapes, "f32")
    with dm.Plan(shapes, dtype="f32", scale_mode="none") as plan:
        Wg, Bg = step_gpu(plan, W, G, B, "f32", lr=LR, weight_decay=WD, mu=MU, steps=0)
    for i, s in enumerate(shapes):
        Wn, bn, O = oracle.muon_step(W[i], G[i], B[i], lr=LR, weight_decay=WD, mu=MU, steps=0,
                                     scale_mode="none")
        assert rel(Wg[i], Wn) <= 1e-6


def test_two_consecutive_steps_llama_layer_structured():
    # the 7B-layer workload at full size: permuted block-diagonal gradients, zero
    # weights, so that each step's output is known block by block
    import torch
    rng = np.random.default_rng(79)
    shapes = synth.LLAMA7B_LAYER
    plan = dm.Plan(shapes)
    tw = [torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
    tb = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    bufs = [np.zeros(s) for s in shapes]
    for step in range(2):
        structs = [synth.permuted_blocks(rng, *s, 8, 0.02, "bf16") for s in shapes]
        tg = [to_dev(st[0], "bf16") for st in structs]
        for t in tw:
            t.zero_()
        plan.step(tw, tg, tb, lr=1.0, weight_decay=0.0, mu=MU)
        torch.cuda.synchronize()
        for i, (s, st) in enumerate(zip(shapes, structs)):
            M, rp, cp, rs, cs = st
            bufs[i] = MU * bufs[i] + M
            assert rel(to_host(tb[i]), bufs[i]) <= 1e-6
            if step == 0:
                # u = (1 + mu) G: same blocks, so NS(u) = NS(G) up to eps
                want, mask = block_expect(M, rp, cp, rs, cs)
                got = -to_host(tw[i]) / oracle.shape_scale(*s)
                assert rel(got, want) <= TOL_BF16_MFMA, (step, s)
                assert np.all(got[~mask] == 0)
    plan.close()


def test_step_matches_ns_batched_path():
    # the fused step and ns_batched run the same product kernels: W = -O when the
    # gradient is the whole update (buf = 0, mu = 0, lr = 1, wd = 0).  The norms
    # are summed in a different order by the two input kernels, so allow the
    # last bit of the scale to differ (one bf16 ulp per element at most).
    import torch
    rng = np.random.default_rng(83)
    shapes = [(256, 640), (640, 256)]
    G = [synth.gaussian(rng, s, 0.02, "bf16") for s in shapes]
    tw = [torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
    tb = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    tg = [to_dev(g, "bf16") for g in G]
    with dm.Plan(shapes, scale_mode="none") as plan:
        plan.step(tw, tg, tb, lr=1.0, weight_decay=0.0, mu=0.0)
    tn = [to_dev(g, "bf16") for g in G]
    for t in tn:
        dm.ns_batched([t])
    torch.cuda.synchronize()
    for w, n in zip(tw, tn):
        assert rel(to_host(-w), to_host(n)) <= 5e-3
