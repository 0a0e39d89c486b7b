"""Diagonal tiles of the symmetric products at tile 256 (GPU, through the C ABI).

A lower tile on the diagonal of a symmetric output runs its own block layout:
the four waves share the tile's 36 lower 32 x 32 blocks (ten each, four
computed twice and stored once), and where both operands are one matrix (the
Gram and polynomial products) the B fragments come from the A stages, whose
B stages are then never loaded.  State widths that are exact multiples of 256
take that path, and at 512 and 768 most tiles are diagonal (2 of 3, 3 of 6).
Results are checked against the fp64 oracle (the recurrence of the Gram
form; DMuon, gist.science technical summary section 2.2) at the 16-bit MFMA
tolerance, and lower against full storage bit for bit.
"""

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
    yield
    torch.cuda.synchronize()


def plan_ns(shapes, mats, storage="auto", coeffs=oracle.QUINTIC, steps=5):
    import torch
    ts = [to_dev(m, "bf16") for m in mats]
    with dm.Plan(shapes, storage=storage) as plan:
        rec = plan.describe()["recurrence"]
        plan.ns(ts, steps=steps, coeffs=coeffs)
    torch.cuda.synchronize()
    return rec, [to_host(t) for t in ts]


@pytest.mark.parametrize("shapes", [
    [(512, 512), (512, 512)],
    [(512, 1536), (1536, 512)],          # both orientations share the 512 bucket
    [(768, 768), (768, 1536)],
    [(512, 512), (768, 768), (512, 1024)],  # two buckets in lockstep launches
])
def test_diagonal_heavy_states_against_oracle(shapes):
    rng = np.random.default_rng(sum(r * 3 + c for r, c in shapes))
    mats = [synth.gaussian(rng, s, 0.02, "bf16") for s in shapes]
    rec, got = plan_ns(shapes, mats)
    assert all(b["tile"] == 256 for b in rec), rec
    errs = [rel(g, oracle.ns_gram(m)) for g, m in zip(got, mats)]
    print("relative errors", ["%.2e" % e for e in errs])
    assert max(errs) <= TOL_BF16_MFMA


@pytest.mark.parametrize("shapes", [[(512, 512), (512, 1536)], [(768, 1536), (1536, 768)]])
def test_diagonal_heavy_lower_equals_full(shapes):
    rng = np.random.default_rng(7 + len(shapes))
    mats = [synth.gaussian(rng, s, 0.02, "bf16") for s in shapes]
    rl, low = plan_ns(shapes, mats, storage="auto")
    rf, full = plan_ns(shapes, mats, storage="full")
    assert all(b["storage"] == "lower" for b in rl) and all(b["storage"] == "full" for b in rf)
    for a, b in zip(low, full):
        assert np.array_equal(a, b)


def test_diagonal_heavy_cubic_reaches_polar_factor():
    # cubic NS (1.5, -0.5, 0) has no square term: the polynomial kernel then
    # clears its accumulator and adds c1 A~ alone, on the diagonal tiles too;
    # 30 steps on a full-rank input converge to the polar factor U V^T
    rng = np.random.default_rng(23)
    m, n = 512, 1024
    U, _ = np.linalg.qr(rng.standard_normal((m, m)))
    V, _ = np.linalg.qr(rng.standard_normal((n, m)))
    M = synth.bf16_round(((U * np.linspace(0.3, 1.0, m)) @ V.T).astype(np.float32))
    coeffs = (1.5, -0.5, 0.0)
    rec, got = plan_ns([(m, n)], [M], coeffs=coeffs, steps=30)
    assert rec[0]["tile"] == 256, rec
    e = rel(got[0], oracle.ns_gram(M, 30, coeffs))
    print(f"cubic {m}x{n}: relative error {e:.3e}", flush=True)
    assert e <= TOL_BF16_MFMA
    assert rel(got[0] @ got[0].T, np.eye(m)) <= 5e-2


def test_single_diagonal_tile_states(tmp_path):
    # states one 256-tile wide (a tune table forcing 256 tiles): every tile
    # of the Gram, polynomial and symmetric products is a diagonal tile
    table = tmp_path / "tile256.json"
    table.write_text('{"entries": [{"max_m": 1073741824, "rec": 256, "syrk": 256, "final": 256}]}')
    shapes = [(256, 256), (256, 1024), (1024, 256)]
    rng = np.random.default_rng(41)
    mats = [synth.gaussian(rng, s, 0.02, "bf16") for s in shapes]
    import torch
    ts = [to_dev(m, "bf16") for m in mats]
    with dm.Plan(shapes, tune_path=str(table)) as plan:
        rec = plan.describe()["recurrence"]
        plan.ns(ts)
    torch.cuda.synchronize()
    assert [b["tile"] for b in rec] == [256], rec
    errs = [rel(to_host(t), oracle.ns_gram(m)) for t, m in zip(ts, mats)]
    print("relative errors", ["%.2e" % e for e in errs])
    assert max(errs) <= TOL_BF16_MFMA
