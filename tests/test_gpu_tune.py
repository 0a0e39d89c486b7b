"""GPU checks of the measured tile table (dmuon_tune) and of the tile
configurations a table can select.

The pages search tile shapes and pipeline configurations per matrix shape and
cache the best (gist.science technical summary, section 2.4).  dmuon_tune
times the tile candidates of every recurrence bucket on the device and writes
the table the planner reads.  Checked here:

- the table written for a small mixed workload has one entry per bucket (its
  short side and batch size), tiles from the candidate set, and a timing for
  every candidate, the entry being the fastest;
- a plan built from that table uses its tiles, and its Muon step matches the
  fp64 oracle;
- hand-written tables that force each tile size (64, 128, 256) for every
  product of both buckets give steps that match the oracle too, so whichever
  configuration a device measures fastest is a correct one.

Shapes: 300 x 520 (twice) and its transpose 520 x 300 share the m = 300
bucket (ragged at every tile size); 512 x 1024 (twice) is the m = 512 bucket
(whole tiles, lower storage at tiles 128 and 256).  The step runs with W = 0,
lr = 1 and no decay, so the stored parameter is -s(rows, cols) O, and O is
compared with the oracle's orthogonalised Nesterov update at the 16-bit MFMA
tolerance.
"""

import json

import numpy as np
import pytest

import oracle
import matrix_orthogonalising_optimizer_amd as dm
from matrix_orthogonalising_optimizer_amd import synth
from gpu_util import TOL_BF16_MFMA, rel, to_dev, to_host

pytestmark = pytest.mark.gpu

SHAPES = [(300, 520), (300, 520), (520, 300), (512, 1024), (512, 1024)]
TILES = (64, 128, 256)
MU = 0.95


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dm.load_library()


@pytest.fixture(scope="module")
def grads():
    rng = np.random.default_rng(41)
    return [synth.gaussian(rng, s, 0.02, "bf16") for s in SHAPES]


def step_errors(G, tune_path):
    """One step of a plan built with `tune_path`: (description, relative error of each O)."""
    import torch
    tg = [to_dev(g, "bf16") for g in G]
    tw = [torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in SHAPES]
    tb = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in SHAPES]
    with dm.Plan(SHAPES, tune_path=tune_path) as plan:
        desc = plan.describe()
        plan.step(tw, tg, tb, lr=1.0, weight_decay=0.0, mu=MU)
        torch.cuda.synchronize()
    errs = []
    for i, s in enumerate(SHAPES):
        _, _, O = oracle.muon_step(np.zeros(s), G[i], np.zeros(s), lr=1.0, weight_decay=0.0, mu=MU)
        got = -to_host(tw[i]) / oracle.shape_scale(*s)
        assert np.all(np.isfinite(got)), (i, s)
        errs.append(rel(got, O))
    return desc, errs


def test_tune_writes_a_table_the_plan_uses(tmp_path, grads):
    path = tmp_path / "table.json"
    table = dm.tune(SHAPES, str(path), warmup=1, repeats=3)
    assert table["steps"] == 5
    entries = {e["max_m"]: e for e in table["entries"]}
    assert sorted(entries) == [300, 512], table["entries"]
    assert entries[300]["max_batch"] == 3 and entries[512]["max_batch"] == 2
    measured = {r["m"]: r for r in table["measured"]}
    for m, e in entries.items():
        assert e["rec"] in TILES and e["syrk"] in TILES and e["final"] in TILES, e
        cands = measured[m]["candidates"]
        assert len(cands) >= 2 and all(c["ms"] > 0 for c in cands), cands
        best = min(cands, key=lambda c: c["ms"])
        assert (e["rec"], e["final"]) == (best["rec"], best["final"]), (e, best)
        print(f"m = {m}: {len(cands)} candidates, best rec {best['rec']} final {best['final']} "
              f"{best['ms']:.4f} ms", flush=True)
    desc, errs = step_errors(grads, str(path))
    assert desc["tune_table"] == str(path)
    for b in desc["recurrence"]:
        assert b["tile"] == entries[b["m"]]["rec"], b
    for g in desc["gemm"]:
        m = min(g["rows"], g["cols"])
        assert g["tile_syrk"] == entries[m]["syrk"] and g["tile_final"] == entries[m]["final"], g
    print("tuned table: relative errors " + " ".join(f"{e:.2e}" for e in errs), flush=True)
    assert max(errs) <= TOL_BF16_MFMA


@pytest.mark.parametrize("tile", TILES)
def test_every_tile_size_matches_the_oracle(tmp_path, grads, tile):
    path = tmp_path / f"tile{tile}.json"
    path.write_text(json.dumps({"entries": [{"max_m": 1 << 20, "rec": tile, "syrk": tile, "final": tile}]}))
    desc, errs = step_errors(grads, str(path))
    for b in desc["recurrence"]:
        assert b["tile"] == tile, b
    storage = {b["m"]: b["storage"] for b in desc["recurrence"]}
    print(f"tile {tile}: storage {storage}, relative errors " + " ".join(f"{e:.2e}" for e in errs), flush=True)
    assert max(errs) <= TOL_BF16_MFMA
