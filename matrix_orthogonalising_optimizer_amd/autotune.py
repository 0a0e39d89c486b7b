"""Measure the tile table on this GPU and write it as JSON.

Usage: python -m matrix_orthogonalising_optimizer_amd.autotune [--out PATH] [--workloads a,b,...]

For each named workload, dmuon_tune times every tile configuration of every
recurrence bucket of that workload's shape list on the current device and
picks the fastest (the pages' per-shape search, cached for later steps:
gist.science technical summary, section 2.4).  The per-workload tables are
merged into one file: entries sorted by (max_m, max_batch), the largest
bucket of each short side widened to any batch size.  Plans read the file
through ``Plan(..., tune_path=PATH)`` or the DMUON_TUNE_TABLE environment
variable; ``shipped_table()`` names the table committed with the package
for this architecture.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_WORKLOADS = ("bf16_64x128x512", "llama7b_layer", "vla_mix_200", "mlp70b_8x8192x28672")


def shipped_table(arch: str = "gfx950"):
    """Path of the measured table committed with the package, or None."""
    p = os.path.join(HERE, "tune", f"{arch}.json")
    return p if os.path.exists(p) else None


def merge(tables):
    """One table from several dmuon_tune outputs (same device and coefficients)."""
    entries = {}
    measured = []
    meta = {}
    for name, t in tables:
        for k in ("arch", "device", "steps", "coeffs", "warmup", "repeats"):
            meta.setdefault(k, t.get(k))
        for e in t["entries"]:
            entries[(e["max_m"], e["max_batch"])] = e
        for m in t.get("measured", []):
            measured.append(dict(m, workload=name))
    keys = sorted(entries)
    out = []
    for i, k in enumerate(keys):
        e = dict(entries[k])
        if i + 1 == len(keys) or keys[i + 1][0] != k[0]:
            e.pop("max_batch")          # the largest bucket of this short side: any batch
        out.append(e)
    return dict(meta, entries=out, workloads=[n for n, _ in tables], measured=measured)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--out", default=os.path.join(HERE, "tune", "gfx950.json"))
    ap.add_argument("--workloads", default=",".join(DEFAULT_WORKLOADS))
    ap.add_argument("--repeats", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    args = ap.parse_args(argv)

    import torch
    import matrix_orthogonalising_optimizer_amd as dm
    from matrix_orthogonalising_optimizer_amd import synth

    dm.load_library()
    torch.cuda.set_device(0)
    tables = []
    with tempfile.TemporaryDirectory() as d:
        for name in args.workloads.split(","):
            shapes = synth.WORKLOADS[name][0]
            if synth.WORKLOADS[name][1] != "bf16":
                continue
            t = dm.tune(shapes, os.path.join(d, name + ".json"), warmup=args.warmup, repeats=args.repeats)
            print(f"{name}: {json.dumps(t['entries'])}", flush=True)
            tables.append((name, t))
    table = merge(tables)
    os.makedirs(os.path.dirname(os.path.abspath(args.out)), exist_ok=True)
    with open(args.out, "w") as fh:
        json.dump(table, fh, indent=1)
        fh.write("\n")
    print(f"wrote {args.out}", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
