"""GPU parity of the fused one-launch kernel for short sides <= 128 against
the fp64 oracle (through the C ABI).

The kernel runs 16-bit Gram buckets of short side <= 128 with fp16 state
(DMUON_PREC_F16, or AUTO for wide members): Gram product, recurrence and
final product in one workgroup per matrix.  Tolerance: the 2e-2 relative
Frobenius bar of 16-bit MFMA operands.  Shapes cover both padded sizes (64 and
128), X resident in registers (n up to 512 at 128 rows, 1024 at 64) and
streamed (longer rows), ragged rows and columns, misaligned pointers and more
members than one launch carries.
"""

import numpy as np
import pytest

import oracle
import matrix_orthogonalising_optimizer_amd as dm
from matrix_orthogonalising_optimizer_amd import synth
from gpu_util import TOL_BF16_MFMA, rel, to_dev, to_host

pytestmark = pytest.mark.gpu

LR, WD, MU = 0.02, 0.1, 0.95


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dm.load_library()
    yield
    torch.cuda.synchronize()


def run_ns(mats, precision="f16", steps=5, coeffs=oracle.QUINTIC):
    import torch
    ts = [to_dev(m, "bf16") for m in mats]
    dm.ns_batched(ts, steps=steps, coeffs=coeffs, precision=precision)
    torch.cuda.synchronize()
    return [to_host(t) for t in ts]


def runs_fused(shape, precision="f16"):
    d = dm.Plan([shape], precision=precision, device=False).describe()
    return d["recurrence"][0]["fused"]


# (rows, cols): padded 128 and 64, resident and streamed X, ragged sizes
SHAPES = [(128, 512), (100, 300), (64, 256), (33, 2000), (1, 9), (7, 13), (96, 200), (120, 1000),
          (60, 1100), (128, 136), (65, 130), (64, 1024)]


@pytest.mark.parametrize("shape", SHAPES)
def test_fused_ns_against_oracle(shape):
    assert runs_fused(shape)
    rng = np.random.default_rng(sum(shape))
    mats = [synth.gaussian(rng, shape, 0.02, "bf16") for _ in range(3)]
    got = run_ns(mats)
    for g, m in zip(got, mats):
        assert g.shape == m.shape
        assert rel(g, oracle.ns_gram(m)) <= TOL_BF16_MFMA, shape


def test_c2_batch_runs_fused_under_auto():
    mats, dtype = synth.workload("bf16_64x128x512")
    assert runs_fused((128, 512), precision="auto")
    got = run_ns(mats, precision="auto")
    errs = [rel(g, oracle.ns_gram(m)) for g, m in zip(got, mats)]
    assert max(errs) <= TOL_BF16_MFMA, max(errs)


def test_fused_matches_grouped_path():
    # the same arithmetic as the grouped fp16 kernels up to summation order:
    # W = 0, no decay, lr = 1, no momentum, no shape factor -> W' = -O
    import torch
    shapes = [(128, 512)] * 3 + [(64, 256)] * 2 + [(100, 300)]
    rng = np.random.default_rng(5)
    G = [synth.gaussian(rng, s, 0.02, "bf16") for s in shapes]
    res = {}
    for fused in ("auto", "off"):
        with dm.Plan(shapes, precision="f16", scale_mode="none", fused=fused) as plan:
            assert all(b["fused"] == (fused == "auto") for b in plan.describe()["recurrence"])
            W = [torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
            B = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
            plan.step(W, [to_dev(g, "bf16") for g in G], B, lr=1.0, weight_decay=0.0, mu=0.0, nesterov=False)
            torch.cuda.synchronize()
            res[fused] = [-to_host(w) for w in W]
    for i, g in enumerate(G):
        want = oracle.ns_gram(g)
        assert rel(res["auto"][i], want) <= TOL_BF16_MFMA
        assert rel(res["off"][i], want) <= TOL_BF16_MFMA
        # both carry the same fp16 state and scales: far closer to each other than to the bar
        assert rel(res["auto"][i], res["off"][i]) <= 5e-3, i


# (rows, cols): both padded sizes, one to sixteen final-product chunks (the
# last one ragged or not), ragged rows
SPLIT_SHAPES = [(128, 512), (100, 300), (128, 136), (65, 130), (120, 1000), (64, 256), (33, 2000), (7, 13)]


@pytest.mark.parametrize("shape", SPLIT_SHAPES)
def test_split_launches_match_one_launch_and_oracle(shape):
    # the fused map as two launches (Gram product and recurrence, then the
    # final product per 128 columns from the stored Q image) and as one: the
    # same arithmetic in the same order, so the same bits, and at the
    # oracle's bar.  W = 0, lr = 1, no momentum or decay, no shape factor:
    # W' = -O
    import torch
    n = 3
    rng = np.random.default_rng(sum(shape) + 7)
    G = [synth.gaussian(rng, shape, 0.02, "bf16") for _ in range(n)]
    res = {}
    for fused in ("split", "one"):
        with dm.Plan([shape] * n, precision="f16", scale_mode="none", fused=fused) as plan:
            desc = plan.describe()
            assert desc["recurrence"][0]["fused"]
            assert desc["gemm"][0]["split"] is (fused == "split")
            W = [torch.zeros(shape, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
            B = [torch.zeros(shape, dtype=torch.float32, device="cuda") for _ in range(n)]
            plan.step(W, [to_dev(g, "bf16") for g in G], B, lr=1.0, weight_decay=0.0, mu=0.0, nesterov=False)
            torch.cuda.synchronize()
            res[fused] = [-to_host(w) for w in W]
    for i, g in enumerate(G):
        assert np.array_equal(res["split"][i], res["one"][i]), (shape, i)
        assert rel(res["split"][i], oracle.ns_gram(g)) <= TOL_BF16_MFMA, (shape, i)


@pytest.mark.parametrize("nesterov", [True, False])
def test_fused_step_against_oracle(nesterov):
    # two consecutive steps on a mix of small wide shapes: momentum, update,
    # weight decay and the shape factor (1 for rows <= cols)
    import torch
    shapes = [(128, 512), (128, 512), (64, 256), (100, 300), (33, 700)]
    rng = np.random.default_rng(83)
    W = [synth.gaussian(rng, s, 0.02, "bf16") for s in shapes]
    B = [rng.standard_normal(s, dtype=np.float32) * np.float32(0.01) for s in shapes]
    Gs = [[synth.gaussian(rng, s, 0.02, "bf16") for s in shapes] for _ in range(2)]
    with dm.Plan(shapes) as plan:
        assert all(b["fused"] for b in plan.describe()["recurrence"])
        tw = [to_dev(x, "bf16") for x in W]
        tb = [to_dev(x, "f32") for x in B]
        Wr = [x.astype(np.float64) for x in W]
        Br = [x.astype(np.float64) for x in B]
        for G in Gs:
            plan.step(tw, [to_dev(g, "bf16") for g in G], tb, lr=LR, weight_decay=WD, mu=MU, nesterov=nesterov)
            torch.cuda.synchronize()
            Wg, Bg = [to_host(t) for t in tw], [to_host(t) for t in tb]
            for i, s in enumerate(shapes):
                Wn, bn, O = oracle.muon_step(Wr[i], G[i], Br[i], lr=LR, weight_decay=WD, mu=MU,
                                             nesterov=nesterov)
                assert rel(Bg[i], bn) <= 1e-6
                # bf16 rounding of W (half an ulp) + lr |O error| (shape factor 1)
                bound = 2.0 ** -8 * np.linalg.norm(Wn) + LR * TOL_BF16_MFMA * np.linalg.norm(O)
                assert np.linalg.norm(Wg[i] - Wn) <= bound, (i, s)
                # continue from what the GPU holds (its bf16 W, its fp32 buffer)
                Wr[i], Br[i] = Wg[i], Bg[i]


def test_more_members_than_one_launch():
    # 270 members: two launches of 256 (one workgroup per CU) and 14
    rng = np.random.default_rng(89)
    mats = [synth.gaussian(rng, (64, 128), 0.02, "bf16") for _ in range(270)]
    got = run_ns(mats)
    for g, m in zip(got, mats):
        assert rel(g, oracle.ns_gram(m)) <= TOL_BF16_MFMA


def test_batch_tensor_equals_list_bitwise():
    # one contiguous (300, 64, 128) tensor (two launches of 256 and 44)
    # against the same matrices as a list of separate tensors
    import torch
    rng = np.random.default_rng(91)
    mats = [synth.gaussian(rng, (64, 128), 0.02, "bf16") for _ in range(300)]
    batch = torch.stack([to_dev(m, "bf16") for m in mats])
    singles = [to_dev(m, "bf16") for m in mats]
    dm.ns_batched(batch)
    dm.ns_batched(singles)
    torch.cuda.synchronize()
    for i, (m, t) in enumerate(zip(mats, singles)):
        assert torch.equal(batch[i], t), i
    for i in (0, 255, 256, 299):
        assert rel(to_host(batch[i]), oracle.ns_gram(mats[i])) <= TOL_BF16_MFMA, i


@pytest.mark.parametrize("shape,n", [((128, 512), 64), ((300, 520), 4)])
def test_step_batch_tensors_equal_lists_bitwise(shape, n):
    # the fused kernel (128 x 512) and the grouped kernels (300 x 520): three
    # batch tensors give bitwise the parameters and momenta of the same step
    # over lists of separate tensors
    import torch
    rng = np.random.default_rng(92)
    G = [synth.gaussian(rng, shape, 0.02, "bf16") for _ in range(n)]
    W = [synth.gaussian(rng, shape, 0.02, "bf16") for _ in range(n)]
    B = [rng.standard_normal(shape, dtype=np.float32) * np.float32(0.01) for _ in range(n)]
    with dm.Plan([shape] * n) as plan:
        wb, gb = torch.stack([to_dev(x, "bf16") for x in W]), torch.stack([to_dev(x, "bf16") for x in G])
        bb = torch.stack([to_dev(x, "f32") for x in B])
        wl, gl, bl = [to_dev(x, "bf16") for x in W], [to_dev(x, "bf16") for x in G], [to_dev(x, "f32") for x in B]
        plan.step(wb, gb, bb, lr=LR, weight_decay=WD, mu=MU)
        plan.step(wl, gl, bl, lr=LR, weight_decay=WD, mu=MU)
        torch.cuda.synchronize()
    for i in range(n):
        assert torch.equal(wb[i], wl[i]) and torch.equal(bb[i], bl[i]), i


def test_step_with_more_members_than_one_momentum_launch():
    # 150 members: one fused launch, whose momentum pass runs as three
    # launches of 64, 64 and 22.  W = 0, lr = 1 and no decay, so the stored
    # parameter is -O (shape factor 1); the momentum buffer and every O are
    # checked against the oracle.
    import torch
    shape, n = (64, 128), 150
    rng = np.random.default_rng(90)
    G = [synth.gaussian(rng, shape, 0.02, "bf16") for _ in range(n)]
    B = [rng.standard_normal(shape, dtype=np.float32) * np.float32(0.01) for _ in range(n)]
    with dm.Plan([shape] * n) as plan:
        assert all(b["fused"] for b in plan.describe()["recurrence"])
        tw = [torch.zeros(shape, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
        tb = [to_dev(x, "f32") for x in B]
        plan.step(tw, [to_dev(g, "bf16") for g in G], tb, lr=1.0, weight_decay=0.0, mu=MU)
        torch.cuda.synchronize()
    for i in range(n):
        _, bn, O = oracle.muon_step(np.zeros(shape), G[i], B[i].astype(np.float64), lr=1.0, weight_decay=0.0, mu=MU)
        assert rel(to_host(tb[i]), bn) <= 1e-6, i
        assert rel(-to_host(tw[i]), O) <= TOL_BF16_MFMA, i


def test_misaligned_and_odd_pitch():
    # matrices at odd element offsets of one buffer, odd column count: every
    # load and store takes the element-wise path
    import torch
    shape = (50, 131)
    rng = np.random.default_rng(97)
    mats = [synth.gaussian(rng, shape, 0.02, "bf16") for _ in range(3)]
    n = shape[0] * shape[1]
    buf = torch.zeros(3 * n + 8, dtype=torch.bfloat16, device="cuda")
    views = []
    for i, m in enumerate(mats):
        off = 1 + i * (n + 1)
        v = buf[off:off + n].view(shape)
        v.copy_(to_dev(m, "bf16"))
        views.append(v)
    guard = [buf[0].item()] + [buf[1 + i * (n + 1) + n].item() for i in range(2)]
    dm.ns_batched(views, precision="f16")
    torch.cuda.synchronize()
    for v, m in zip(views, mats):
        assert rel(to_host(v), oracle.ns_gram(m)) <= TOL_BF16_MFMA
    # the elements between the matrices are untouched
    assert [buf[0].item()] + [buf[1 + i * (n + 1) + n].item() for i in range(2)] == guard


@pytest.mark.parametrize("steps", [1, 2, 3, 7])
def test_fused_step_counts(steps):
    rng = np.random.default_rng(101)
    mats = [synth.gaussian(rng, (96, 400), 0.02, "bf16") for _ in range(2)]
    got = run_ns(mats, steps=steps)
    for g, m in zip(got, mats):
        assert rel(g, oracle.ns_gram(m, steps)) <= TOL_BF16_MFMA


def test_fused_cubic_reaches_polar_factor():
    # 30 cubic steps on a full-rank 96 x 200 matrix: the polar factor U V^T
    rng = np.random.default_rng(29)
    m, n = 96, 200
    U, _ = np.linalg.qr(rng.standard_normal((m, m)))
    V, _ = np.linalg.qr(rng.standard_normal((n, m)))
    M = synth.bf16_round(((U * np.linspace(0.3, 1.0, m)) @ V.T).astype(np.float32))
    assert runs_fused((m, n))
    got = run_ns([M], steps=30, coeffs=(1.5, -0.5, 0.0))[0]
    assert rel(got, oracle.ns_gram(M, 30, (1.5, -0.5, 0.0))) <= TOL_BF16_MFMA
    assert rel(got @ got.T, np.eye(m)) <= 5e-2


def test_steps_beyond_the_fused_limit_fall_back():
    # more than 64 steps: the grouped fp16 kernels run the bucket (a mild
    # cubic keeps Q's scale at 2^0, so fp16 state is allowed)
    rng = np.random.default_rng(103)
    M = synth.gaussian(rng, (64, 256), 0.02, "bf16")
    co = (1.03, -0.03, 0.0)
    got = run_ns([M], steps=70, coeffs=co)[0]
    assert rel(got, oracle.ns_gram(M, 70, co)) <= TOL_BF16_MFMA


def test_long_cubic_leaves_fp16_state():
    # 70 steps of (1.5, -0.5, 0): Q's scale would flush the converged
    # directions out of fp16, so F16 is refused and AUTO runs bf16 state
    rng = np.random.default_rng(109)
    M = synth.gaussian(rng, (64, 256), 0.02, "bf16")
    co = (1.5, -0.5, 0.0)
    with pytest.raises(dm.DmuonError) as e:
        run_ns([M], steps=70, coeffs=co)
    assert e.value.code == dm.EUNSUPPORTED
    got = run_ns([M], precision="auto", steps=70, coeffs=co)[0]
    assert rel(got, oracle.ns_gram(M, 70, co)) <= TOL_BF16_MFMA


def test_zero_matrix_and_determinism():
    rng = np.random.default_rng(107)
    z = np.zeros((80, 333), np.float32)
    assert np.all(run_ns([z])[0] == 0)
    M = synth.gaussian(rng, (128, 512), 0.02, "bf16")
    a, b = run_ns([M])[0], run_ns([M])[0]
    assert np.array_equal(a, b)
