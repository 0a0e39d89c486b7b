"""GPU parity of dmuon_ns_batched against the fp64 oracle (through the C ABI).

Tolerances are relative Frobenius errors: 2e-2 for 16-bit MFMA operands with
fp32 accumulation, 1e-4 for the fp32 MFMA path.
"""

import math

import numpy as np
import pytest

import oracle
import matrix_orthogonalising_optimizer_amd as dm
from matrix_orthogonalising_optimizer_amd import synth
from gpu_util import TOL_BF16_MFMA, TOL_F32, block_expect, rel, to_dev, to_host

pytestmark = pytest.mark.gpu

QUINTIC = oracle.QUINTIC


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dm.load_library()
    yield
    torch.cuda.synchronize()


def run_ns(mats, dtype, precision="auto", steps=5, coeffs=QUINTIC):
    import torch
    ts = [to_dev(m, dtype) for m in mats]
    dm.ns_batched(ts, steps=steps, coeffs=coeffs, precision=precision)
    torch.cuda.synchronize()
    return [to_host(t) for t in ts]


def test_c1_fp32_256x1024():
    mats, dtype = synth.workload("fp32_256x1024")
    got = run_ns(mats, "f32", "f32")[0]
    want = oracle.ns_gram(mats[0])
    assert rel(got, want) <= TOL_F32
    # the standard form agrees too
    assert rel(got, oracle.ns_standard(mats[0])) <= TOL_F32


def test_c2_batch_64x128x512():
    mats, dtype = synth.workload("bf16_64x128x512")
    assert dtype == "bf16" and len(mats) == 64
    got = run_ns(mats, "bf16")
    errs = [rel(g, oracle.ns_gram(m)) for g, m in zip(got, mats)]
    assert max(errs) <= TOL_BF16_MFMA, max(errs)


SHAPES = [(64, 64), (100, 300), (300, 100), (257, 513), (640, 1100), (1100, 640), (33, 2000),
          (2000, 33), (1, 9), (9, 1), (128, 128), (500, 500), (1024, 1024), (520, 260)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("precision", ["auto", "f32"])
def test_shapes_against_oracle(shape, precision):
    rng = np.random.default_rng(hash(shape) % 2**32)
    dtype = "f32" if precision == "f32" else "bf16"
    mats = [synth.gaussian(rng, shape, 0.02, dtype) for _ in range(2)]
    got = run_ns(mats, dtype, precision)
    tol = TOL_F32 if precision == "f32" else TOL_BF16_MFMA
    for g, m in zip(got, mats):
        assert g.shape == m.shape
        assert rel(g, oracle.ns_gram(m)) <= tol


@pytest.mark.parametrize("shape", [(256, 256), (300, 400), (1024, 1024)])
def test_forced_f16_on_square_shapes(shape):
    # the fp16 path on its own, on square shapes above the fp32 cut-over
    rng = np.random.default_rng(19)
    mats = [synth.gaussian(rng, shape, 0.02, "bf16")]
    got = run_ns(mats, "bf16", "f16")[0]
    assert rel(got, oracle.ns_gram(mats[0])) <= TOL_BF16_MFMA


@pytest.mark.parametrize("shape", [(64, 64), (100, 300), (300, 100)])
def test_bf16_inputs_on_fp32_path(shape):
    rng = np.random.default_rng(13)
    mats = [synth.gaussian(rng, shape, 0.02, "bf16") for _ in range(3)]
    got = run_ns(mats, "bf16", "f32")
    for g, m in zip(got, mats):
        # fp32 arithmetic; the result is rounded to bf16 (relative 2^-9 per entry)
        assert rel(g, oracle.ns_gram(m)) <= 4e-3


@pytest.mark.parametrize("shape", [(128, 512), (300, 1100), (1100, 300), (1024, 4096)])
def test_plain_bf16_mode_on_wide_shapes(shape):
    # plain bf16 operands meet the bar on matrices with m well below n
    rng = np.random.default_rng(17)
    mats = [synth.gaussian(rng, shape, 0.02, "bf16")]
    got = run_ns(mats, "bf16", "bf16")[0]
    assert rel(got, oracle.ns_gram(mats[0])) <= TOL_BF16_MFMA


@pytest.mark.parametrize("steps", [0, 1, 2, 3, 7, 12])
@pytest.mark.parametrize("precision", ["f16", "f32"])
def test_step_counts(steps, precision):
    rng = np.random.default_rng(23)
    dtype = "f32" if precision == "f32" else "bf16"
    mats = [synth.gaussian(rng, (200, 450), 0.02, dtype)]
    got = run_ns(mats, dtype, precision, steps=steps)[0]
    tol = TOL_F32 if precision == "f32" else TOL_BF16_MFMA
    assert rel(got, oracle.ns_gram(mats[0], steps)) <= tol


@pytest.mark.parametrize("precision", ["f16", "bf16", "f32"])
def test_zero_matrix_gives_zeros(precision):
    dtype = "f32" if precision == "f32" else "bf16"
    got = run_ns([np.zeros((96, 160), np.float32)], dtype, precision)[0]
    assert np.all(got == 0)


@pytest.mark.parametrize("precision", ["f16", "f32"])
def test_cubic_coefficients_reach_polar_factor(precision):
    # 30 cubic steps, full rank: converges to the polar factor U V^T
    rng = np.random.default_rng(29)
    m, n = 96, 200
    U, _ = np.linalg.qr(rng.standard_normal((m, m)))
    V, _ = np.linalg.qr(rng.standard_normal((n, m)))
    M = ((U * np.linspace(0.3, 1.0, m)) @ V.T).astype(np.float32)
    dtype = "f32" if precision == "f32" else "bf16"
    if dtype == "bf16":
        M = synth.bf16_round(M)
    got = run_ns([M], dtype, precision, steps=30, coeffs=(1.5, -0.5, 0.0))[0]
    tol = TOL_F32 if precision == "f32" else TOL_BF16_MFMA
    assert rel(got, oracle.ns_gram(M, 30, (1.5, -0.5, 0.0))) <= tol
    assert rel(got @ got.T, np.eye(m)) <= (1e-3 if precision == "f32" else 5e-2)


@pytest.mark.parametrize("shape", [(300, 520), (700, 900), (1024, 1536)])
def test_cubic_coefficients_tiled_products(shape):
    # (1.5, -0.5, 0) has no square term: the tiled polynomial kernels (128
    # and 256 tiles, full and lower storage) then clear the accumulator and
    # add c1 A~ themselves instead of scaling A~ A~ + (c1 / c2) A~
    rng = np.random.default_rng(32)
    M = synth.gaussian(rng, shape, 1.0, "bf16")
    got = run_ns([M], "bf16", "f16", steps=12, coeffs=(1.5, -0.5, 0.0))[0]
    e = rel(got, oracle.ns_gram(M, 12, (1.5, -0.5, 0.0)))
    print(f"cubic {shape}: relative error {e:.3e}", flush=True)
    assert e <= TOL_BF16_MFMA


@pytest.mark.parametrize("precision", ["f16", "f32"])
def test_exact_null_space_with_long_iteration(precision):
    # A signed-permuted diagonal matrix with 48 zero rows: its Gram matrix has
    # exact zero eigenvalues, on which Q grows like a^T = 1.5^30 (beyond fp16).
    # An overflow there would give NaN through inf * 0; the fp16 path stores Q
    # divided by a per-step power of two.  The result is known entry by entry.
    rng = np.random.default_rng(30)
    m, n, r = 96, 200, 48
    d = np.zeros(m)
    d[:r] = synth.bf16_round(np.linspace(0.3, 1.0, r).astype(np.float32))
    d *= rng.choice([-1.0, 1.0], m)
    D = np.zeros((m, n), np.float32)
    D[np.arange(m), np.arange(m)] = d
    rp, cp = rng.permutation(m), rng.permutation(n)
    M = D[rp][:, cp]
    dtype = "f32" if precision == "f32" else "bf16"
    got = run_ns([M], dtype, precision, steps=30, coeffs=(1.5, -0.5, 0.0))[0]
    assert np.all(np.isfinite(got))
    s = np.abs(d) / (np.linalg.norm(d) + oracle.DEFAULT_EPS)
    for _ in range(30):
        s = 1.5 * s - 0.5 * s ** 3
    W = np.zeros((m, n))
    W[np.arange(m), np.arange(m)] = np.sign(d) * s
    want = W[rp][:, cp]
    tol = TOL_F32 if precision == "f32" else TOL_BF16_MFMA
    assert rel(got, want) <= tol
    assert rel(got, oracle.ns_gram(M, 30, (1.5, -0.5, 0.0))) <= tol


@pytest.mark.parametrize("shape", [(200, 330), (330, 200)])
def test_identity_coefficients(shape):
    rng = np.random.default_rng(31)
    M = synth.gaussian(rng, shape, 1.0, "f32")
    got = run_ns([M], "f32", "f32", steps=3, coeffs=(1.0, 0.0, 0.0))[0]
    want = M / (np.linalg.norm(M.astype(np.float64)) + oracle.DEFAULT_EPS)
    assert rel(got, want) <= 1e-6


@pytest.mark.parametrize("shape", [(96, 200), (200, 96)])
def test_signed_selection_closed_form(shape):
    X = synth.signed_selection(np.random.default_rng(37), *shape)
    got = run_ns([X], "bf16", "f16")[0]
    k = min(shape)
    s = 1.0 / (math.sqrt(k) + oracle.DEFAULT_EPS)
    for _ in range(5):
        s = QUINTIC[0] * s + QUINTIC[1] * s ** 3 + QUINTIC[2] * s ** 5
    assert rel(got, s * X) <= TOL_BF16_MFMA


def test_misaligned_pointer_path():
    import torch
    rng = np.random.default_rng(41)
    M = synth.gaussian(rng, (150, 333), 0.02, "bf16")
    base = torch.zeros(1 + M.size, dtype=torch.bfloat16, device="cuda")
    view = base[1:].view(150, 333)  # storage offset 1: 2-byte aligned only
    view.copy_(to_dev(M, "bf16"))
    assert view.data_ptr() % 16 != 0
    dm.ns_batched([view])
    torch.cuda.synchronize()
    assert rel(to_host(view), oracle.ns_gram(M)) <= TOL_BF16_MFMA
    assert float(base[0]) == 0.0  # nothing written before the matrix


def test_deterministic_and_batch_equals_singles():
    import torch
    rng = np.random.default_rng(43)
    mats = [synth.gaussian(rng, (384, 700), 0.02, "bf16") for _ in range(5)]
    a = [to_dev(m, "bf16") for m in mats]
    b = [to_dev(m, "bf16") for m in mats]
    dm.ns_batched(a)
    for t in b:
        dm.ns_batched([t])
    c = [to_dev(m, "bf16") for m in mats]
    dm.ns_batched(c)
    torch.cuda.synchronize()
    for x, y, z in zip(a, b, c):
        assert torch.equal(x, y) and torch.equal(x, z)
    # batch order permutes outputs bitwise
    d = [to_dev(m, "bf16") for m in mats[::-1]]
    dm.ns_batched(d)
    torch.cuda.synchronize()
    for x, y in zip(a, d[::-1]):
        assert torch.equal(x, y)


@pytest.mark.parametrize("dtype,shape,n", [("f32", (200, 330), 3), ("bf16", (384, 700), 70)])
def test_batch_tensor_equals_list(dtype, shape, n):
    # one contiguous (n, rows, cols) tensor against the same matrices as a
    # list: the fp32 path, and a bf16 batch of more matrices than one grouped
    # launch carries; bitwise equal, and one member against the oracle
    import torch
    rng = np.random.default_rng(44)
    mats = [synth.gaussian(rng, shape, 0.02, dtype) for _ in range(n)]
    batch = torch.stack([to_dev(m, dtype) for m in mats])
    singles = [to_dev(m, dtype) for m in mats]
    dm.ns_batched(batch, precision="f32" if dtype == "f32" else "auto")
    dm.ns_batched(singles, precision="f32" if dtype == "f32" else "auto")
    torch.cuda.synchronize()
    for i, t in enumerate(singles):
        assert torch.equal(batch[i], t), i
    tol = TOL_F32 if dtype == "f32" else TOL_BF16_MFMA
    assert rel(to_host(batch[n - 1]), oracle.ns_gram(mats[n - 1])) <= tol


def test_large_batch_spans_pointer_chunks():
    # more matrices than one launch carries pointers for
    rng = np.random.default_rng(47)
    mats = [synth.gaussian(rng, (64, 96), 0.02, "bf16") for _ in range(150)]
    got = run_ns(mats, "bf16")
    errs = [rel(g, oracle.ns_gram(m)) for g, m in zip(got, mats)]
    assert max(errs) <= TOL_BF16_MFMA


@pytest.mark.parametrize("shape", [(4096, 4096), (11008, 4096), (4096, 11008)])
def test_llama_layer_full_size_structured(shape):
    # full size, permuted block-diagonal input: every output tile is touched and
    # the oracle result is known block by block
    import torch
    rng = np.random.default_rng(53)
    M, rp, cp, rs, cs = synth.permuted_blocks(rng, *shape, 16, 0.02, "bf16")
    want, mask = block_expect(M, rp, cp, rs, cs)
    t = to_dev(M, "bf16")
    dm.ns_batched([t])
    torch.cuda.synchronize()
    got = to_host(t)
    assert rel(got, want) <= TOL_BF16_MFMA
    assert np.all(got[~mask] == 0)


def test_c5_mlp70b_full_size_structured():
    import torch
    rng = np.random.default_rng(59)
    M, rp, cp, rs, cs = synth.permuted_blocks(rng, 8192, 28672, 32, 0.02, "bf16")
    want, mask = block_expect(M, rp, cp, rs, cs)
    t = to_dev(M, "bf16")
    dm.ns_batched([t])
    torch.cuda.synchronize()
    got = to_host(t)
    assert rel(got, want) <= TOL_BF16_MFMA
    assert np.all(got[~mask] == 0)


def test_c4_vla_mix_sampled():
    # the mixed workload through a plan-free call per shape; oracle on one
    # matrix per shape (matrices are independent)
    import torch
    mats, _ = synth.workload("vla_mix_200")
    by_shape = {}
    for i, m in enumerate(mats):
        by_shape.setdefault(m.shape, []).append(i)
    for shape, idx in by_shape.items():
        ts = [to_dev(mats[i], "bf16") for i in idx]
        dm.ns_batched(ts)
        torch.cuda.synchronize()
        i0 = idx[0]
        assert rel(to_host(ts[0]), oracle.ns_gram(mats[i0])) <= TOL_BF16_MFMA, shape
        i1 = idx[-1]
        if shape[0] <= 1024:
            assert rel(to_host(ts[-1]), oracle.ns_gram(mats[i1])) <= TOL_BF16_MFMA, shape


# dmuon_plan_ns: one plan over several shapes.  The m = 300 recurrence bucket
# takes both orientations (300 x 520 and its transpose) and a wider matrix
# (300 x 900) in shared launches; 128 x 512 runs the fused small-matrix
# kernel; 96 x 96 (near square, small) the fp32 path under AUTO.
PLAN_NS_SHAPES = [(300, 520), (520, 300), (300, 900), (128, 512), (128, 512), (96, 96)]


def test_plan_ns_mixed_shapes_against_oracle():
    import torch
    rng = np.random.default_rng(311)
    mats = [synth.gaussian(rng, s, 0.02, "bf16") for s in PLAN_NS_SHAPES]
    ts = [to_dev(m, "bf16") for m in mats]
    with dm.Plan(PLAN_NS_SHAPES) as plan:
        d = plan.describe()
        assert sorted(b["m"] for b in d["recurrence"]) == [96, 128, 300]
        plan.ns(ts)
        torch.cuda.synchronize()
    errs = [rel(to_host(t), oracle.ns_gram(m)) for t, m in zip(ts, mats)]
    print("plan ns relative errors " + " ".join(f"{e:.2e}" for e in errs), flush=True)
    assert max(errs) <= TOL_BF16_MFMA


def test_plan_ns_batch_tensor_equals_ns_batched():
    # a plan of one shape: its NS call on a (count, rows, cols) tensor gives
    # the bits of dmuon_ns_batched on the same matrices (the same plan)
    import torch
    rng = np.random.default_rng(312)
    shape, n = (256, 768), 5
    x = torch.stack([to_dev(synth.gaussian(rng, shape, 0.02, "bf16"), "bf16") for _ in range(n)])
    y = x.clone()
    with dm.Plan([shape] * n) as plan:
        plan.ns(x)
    dm.ns_batched([y[i] for i in range(n)])
    torch.cuda.synchronize()
    assert torch.equal(x, y)


@pytest.mark.parametrize("opts", [
    dict(storage="full"),                    # both triangles of the states stored
    dict(pad_ratio=0.5),                     # 200 and 256 share one padded bucket
    dict(form="standard"),                   # the standard iteration per bucket
    dict(precision="f32"),                   # fp32 MFMA throughout
    dict(fused="off"),                       # short sides <= 128 on the grouped kernels
])
def test_plan_ns_options_against_oracle(opts):
    # dmuon_plan_ns under every plan option that changes the launches: the
    # same mixed shapes (both orientations, a padded pair, a small bucket)
    # against the oracle at the option's tolerance
    import torch
    shapes = [(200, 520), (256, 520), (520, 256), (96, 400)]
    rng = np.random.default_rng(313)
    mats = [synth.gaussian(rng, s, 0.02, "bf16") for s in shapes]
    ts = [to_dev(m, "bf16") for m in mats]
    with dm.Plan(shapes, **opts) as plan:
        plan.ns(ts)
        torch.cuda.synchronize()
    # fp32 arithmetic with bf16 results: the rounding of the output (relative
    # 2^-9 per entry) bounds the error, as for the plan-free fp32 path
    tol = 4e-3 if opts.get("precision") == "f32" else TOL_BF16_MFMA
    errs = [rel(to_host(t), oracle.ns_gram(m)) for t, m in zip(ts, mats)]
    print(f"plan ns {opts}: relative errors " + " ".join(f"{e:.2e}" for e in errs), flush=True)
    assert max(errs) <= tol
