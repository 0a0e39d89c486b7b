#!/usr/bin/env python3
"""Throughput of the fused Muon step (batched Gram Newton-Schulz) on one MI355X.

One step = one dmuon_step over the whole workload: Nesterov momentum, Frobenius
normalisation, the Gram product, the 5-step m x m recurrence, the final product
and the parameter update, for every matrix.  Inputs are seeded synthetic
Gaussian matrices resident in HBM before timing starts.

Prints one JSON line with the throughput (matrices/s), the algorithmic TFLOP/s,
the roofline of the dominant kernel and the fp64 CPU oracle timed on a bounded
sample of the same workload.  The throughput comes from K timed steps with no
instrumentation; the per-kernel figures from a second pass of K steps in which
the library brackets every launch with HIP events on its stream (the events
add host work between launches, which would otherwise inflate the step time
of small workloads, but not to any kernel's own duration).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Gram-NS matrices/sec and effective TFLOP/s (% bf16 MFMA peak), 1 MI355X"
PEAK_16BIT = 2516.6e12   # dense bf16/fp16 MFMA, 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_F32 = 157.3e12      # dense fp32 MFMA
HBM_PEAK = 8.0e12        # bytes/s
COEFFS = (3.4445, -4.7750, 2.0315)


def ns_flops(rows: int, cols: int, steps: int) -> float:
    """Algorithmic flops of one matrix: symmetric products count one triangle.

    Gram product m(m+1)n, 4T-3 symmetric m x m products m^2(m+1) each, final
    product 2 m^2 n (m = short side, n = long side)."""
    if steps == 0:
        return 0.0
    m, n = min(rows, cols), max(rows, cols)
    return m * (m + 1) * n + (4 * steps - 3) * m * m * (m + 1) + 2.0 * m * m * n


def kernel_source_sha256() -> str:
    """sha256 of the product kernels' sources with comments and runs of
    white space removed: an edit of comments alone keeps committed counter
    summaries valid, any change of code does not."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in ("gemm_impl.h", "kernels.h"):
        with open(os.path.join(ROOT, "matrix_orthogonalising_optimizer_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def profiled_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summaries, or None when none matches this kernel source and workload."""
    d = os.path.join(ROOT, "profiles")
    if not os.path.isdir(d):
        return None
    sha = kernel_source_sha256()
    for name in sorted(os.listdir(d)):
        if not name.endswith(".traffic.txt"):
            continue
        kv = {}
        with open(os.path.join(d, name)) as fh:
            for line in fh:
                if "=" in line:
                    k, v = line.rstrip("\n").split("=", 1)
                    kv[k] = v
        if kv.get("kernel") == kernel and kv.get("workload") == workload and kv.get("kernel_source_sha256") == sha:
            return float(kv["traffic_bytes_per_launch"])
    return None


def resolve_tune_table(choice: str):
    """Tune-table path for the plans (None = the library's built-in table)."""
    if choice == "builtin":
        return None
    if choice == "shipped":
        from matrix_orthogonalising_optimizer_amd.autotune import shipped_table
        return shipped_table()
    return choice


def arithmetic_of(kernels) -> str:
    """Arithmetic type(s) the products ran in, from the kernel instances that
    ran: a product kernel is named gemm_kernel<operand, state, ...> and its
    state type is the precision of the bucket (the Gram product of a 16-bit
    bucket multiplies the bf16 input exactly on bf16 MFMA and writes the
    bucket's fp16 state); the fused small-matrix kernel runs fp16 operands."""
    names = {"_Float16": "f16", "float": "f32"}
    kinds = set()
    for k in kernels:
        n = k["kernel"]
        if n.startswith("gemm_kernel<"):
            parts = n[len("gemm_kernel<"):].split(", ")
            kinds.add(names.get(parts[1], "bf16"))
        elif n.startswith("small_ns_kernel"):
            kinds.add("f16")
    return "+".join(sorted(kinds)) or "none"


def shapes_summary(shapes):
    out, seen = [], {}
    for s in shapes:
        seen[s] = seen.get(s, 0) + 1
    for s, c in seen.items():
        out.append(f"{c}x{s[0]}x{s[1]}")
    return ", ".join(out)


def cpu_baseline(shapes, dtype, steps, budget_s, seed):
    """Time the fp64 oracle's Muon step on one matrix per distinct shape.

    Shapes are sampled cheapest first until the time budget is spent; the rest
    are extrapolated with the measured flop rate.  Returns the dict for the
    JSON line."""
    import oracle
    from matrix_orthogonalising_optimizer_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    distinct = sorted(set(shapes), key=lambda s: ns_flops(*s, steps))
    counts = {s: shapes.count(s) for s in distinct}
    rng = np.random.default_rng(seed)
    timed, spent = {}, 0.0
    for s in distinct:
        if timed and spent > budget_s:
            break
        W = synth.gaussian(rng, s, 0.02, dtype)
        G = synth.gaussian(rng, s, 0.02, dtype)
        B = np.zeros(s, np.float32)
        t0 = time.perf_counter()
        oracle.muon_step(W, G, B, lr=0.02, weight_decay=0.1, mu=0.95, steps=steps, coeffs=COEFFS)
        dt = time.perf_counter() - t0
        timed[s] = dt
        spent += dt
    rate = sum(ns_flops(*s, steps) for s in timed) / max(sum(timed.values()), 1e-12)
    est = 0.0
    for s in distinct:
        est += counts[s] * (timed[s] if s in timed else ns_flops(*s, steps) / rate)
    sampled = ", ".join(f"1x{s[0]}x{s[1]} {timed[s]:.2f}s" for s in timed)
    rest = [s for s in distinct if s not in timed]
    note = f"oracle muon_step (fp64 NumPy) on one matrix per distinct shape: {sampled}"
    note += "; scaled by the shape counts"
    if rest:
        note += "; not run, extrapolated at the measured flop rate: " + ", ".join(f"{a}x{b}" for a, b in rest)
    try:
        host_cpus = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        host_cpus = os.cpu_count() or 1
    return {"value": len(shapes) / est, "unit": "matrices/s", "cores": int(threads), "kind": "oracle",
            "sample": note, "seconds_per_step_estimate": est,
            "blas_threads": int(threads), "host_cpus_available": int(host_cpus)}


def bucket_report(dm, desc, shapes, W, G, B, T, args, dtype):
    """Each recurrence bucket of the plan on its own: a plan of its members
    alone, timed like the whole step (warm-up, then K steps between events).
    Buckets of one plan share launches when they run together, so these
    stand-alone times need not add up to the whole step."""
    import torch
    out = []
    for b in desc["recurrence"]:
        idx = sorted(b["members"])
        sub = [shapes[i] for i in idx]
        Ws, Gs, Bs = [W[i] for i in idx], [G[i] for i in idx], [B[i] for i in idx]
        plan = dm.Plan(sub, dtype=dtype, precision=args.precision, tune_path=resolve_tune_table(args.tune_table))
        for _ in range(max(1, args.warmup)):
            plan.step(Ws, Gs, Bs, lr=0.02, weight_decay=0.1, mu=0.95, steps=T, coeffs=COEFFS)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            plan.step(Ws, Gs, Bs, lr=0.02, weight_decay=0.1, mu=0.95, steps=T, coeffs=COEFFS)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        plan.close()
        fl = sum(ns_flops(r, c, T) for r, c in sub)
        out.append({"m": b["m"], "shapes": shapes_summary(sub), "tile": b["tile"], "storage": b["storage"],
                    "fp32": b["fp32"], "fused": b["fused"], "ms_per_step": round(ms, 4),
                    "matrices_per_s": round(len(sub) / (ms * 1e-3), 2),
                    "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
                    "pct_bf16_peak": round(100.0 * fl / (ms * 1e-3) / PEAK_16BIT, 2)})
    return out


def adamw_timing(dm, W, G, args):
    """The fused AdamW step (dmuon_adamw_step) over the same parameters and
    gradients, fresh fp32 moments: warm-up, then K timed steps; the
    per-launch durations come from the library's HIP events."""
    import torch
    Wc = [w.clone() for w in W]
    M = [torch.zeros(w.shape, dtype=torch.float32, device=w.device) for w in W]
    V = [torch.zeros(w.shape, dtype=torch.float32, device=w.device) for w in W]
    t = 0

    def one():
        nonlocal t
        t += 1
        dm.adamw_step(Wc, G, M, V, lr=1e-3, step=t, betas=(0.9, 0.95), eps=1e-8, weight_decay=0.1)

    for _ in range(max(1, args.warmup)):
        one()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        one()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    dm.timing_enable(True)
    for _ in range(args.steps):
        one()
    torch.cuda.synchronize()
    dm.timing_enable(False)
    ks = dm.timing_report()["kernels"]
    k = max(ks, key=lambda x: x["total_ms"])
    achieved = k["bytes"] / (k["total_ms"] * 1e-3)
    del Wc, M, V
    return {"ms_per_step": round(ms, 4), "kernel": k["kernel"], "launches_per_step": k["launches"] / args.steps,
            "avg_launch_ms": round(k["avg_ms"], 4), "bytes_per_launch": k["bytes"] / k["launches"],
            "achieved_gbps": round(achieved / 1e9, 1), "hbm_frac": round(achieved / HBM_PEAK, 4)}


def adamw_line(dm, shapes, dtype, W, G, args):
    """The JSON line of --mode adamw: the fused AdamW step, HBM-bound."""
    r = adamw_timing(dm, W, G, args)
    nmat = len(shapes)
    return {
        "metric": "AdamW step matrices/sec (fused dmuon_adamw_step), 1 MI355X",
        "value": round(nmat / (r["ms_per_step"] * 1e-3), 3), "unit": "matrices/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": r["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32 math, " + dtype + " parameters", "data": "synthetic",
        "config": {"workload": args.workload, "matrices": nmat, "shapes": shapes_summary(shapes),
                   "mode": "dmuon_adamw_step", "betas": [0.9, 0.95], "global_batch": nmat,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": r["achieved_gbps"], "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": r["hbm_frac"], "traffic": None, "kernel": r["kernel"],
                     "launches_per_step": r["launches_per_step"], "avg_launch_ms": r["avg_launch_ms"],
                     "bytes_per_launch": r["bytes_per_launch"]},
    }


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama7b_layer")
    ap.add_argument("--mode", choices=["step", "ns", "adamw"], default="step",
                    help="step: dmuon_step (default); ns: dmuon_ns_batched per shape group; adamw: the fused "
                         "AdamW step on the same parameters")
    ap.add_argument("--ns-steps", type=int, default=5)
    ap.add_argument("--precision", default="auto", choices=["auto", "f16", "bf16", "f32"])
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tune-table", default="shipped",
                    help="tile table of the plans: 'shipped' (the measured table committed with the package "
                         "for gfx950, else the built-in one), 'builtin', or a JSON path")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one step captured in a HIP graph (the host then issues one "
                         "replay per step instead of the library calls)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(each matrix is independent work for one GPU: several GPUs would each run this "
              "path on the matrices they own)",
              file=sys.stderr)
        return 2

    import torch
    import matrix_orthogonalising_optimizer_amd as dm
    from matrix_orthogonalising_optimizer_amd import synth

    dm.load_library()
    torch.cuda.set_device(0)
    shapes, dtype, sigma, seed = synth.WORKLOADS[args.workload]
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    # gradients first: they are the workload's own matrices (synth.workload),
    # which the parity tests run through the same plan
    G_host, W_host, _ = synth.step_inputs(args.workload)
    G = [torch.from_numpy(x).to("cuda").to(tdt) for x in G_host]
    W = [torch.from_numpy(x).to("cuda").to(tdt) for x in W_host]
    del G_host, W_host
    B = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    T = args.ns_steps
    # a workload of one shape is passed as (count, rows, cols) batch tensors,
    # the way a caller holds a batch of like matrices (no per-matrix Python
    # work per call); the lists then hold views of them
    batched = len(set(shapes)) == 1
    if batched:
        Gb, Wb, Bb = torch.stack(G), torch.stack(W), torch.stack(B)
        G, W, B = list(Gb), list(Wb), list(Bb)
        torch.cuda.synchronize()

    if args.mode == "adamw":
        print(json.dumps(adamw_line(dm, shapes, dtype, W, G, args)), flush=True)
        return 0
    tune_path = resolve_tune_table(args.tune_table)
    if args.mode == "step":
        plan = dm.Plan(shapes, dtype=dtype, precision=args.precision, tune_path=tune_path)

        def one_step():
            if batched:
                plan.step(Wb, Gb, Bb, lr=0.02, weight_decay=0.1, mu=0.95, steps=T, coeffs=COEFFS)
            else:
                plan.step(W, G, B, lr=0.02, weight_decay=0.1, mu=0.95, steps=T, coeffs=COEFFS)
    elif batched:
        # one shape: the plan-free call on the batch tensor
        def one_step():
            dm.ns_batched(Gb, steps=T, coeffs=COEFFS, precision=args.precision)
    else:
        # several shapes: one plan, whose recurrence buckets share launches
        # across shapes of one short side (separate per-shape calls would not)
        plan = dm.Plan(shapes, dtype=dtype, precision=args.precision, tune_path=tune_path)

        def one_step():
            plan.ns(G, steps=T, coeffs=COEFFS)

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    eager_step = one_step
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            eager_step()
        torch.cuda.synchronize()
        one_step = graph.replay

    stream = torch.cuda.current_stream()
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(args.steps):
        one_step()
    t_end.record(stream)
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_end) / args.steps
    # per-kernel pass: the same K steps with every launch bracketed by events
    dm.timing_enable(True)
    k_start, k_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    k_start.record(stream)
    for _ in range(args.steps):
        eager_step()
    k_end.record(stream)
    torch.cuda.synchronize()
    dm.timing_enable(False)
    rep = dm.timing_report()
    ms_instrumented = k_start.elapsed_time(k_end) / args.steps

    nmat = len(shapes)
    flops = sum(ns_flops(r, c, T) for r, c in shapes)
    tflops = flops / (ms * 1e-3) / 1e12
    kernels = sorted(rep["kernels"], key=lambda k: -k["total_ms"])
    dom = kernels[0]
    # the dominant kernel's own arithmetic sets its peak
    peak = PEAK_F32 if arithmetic_of([dom]) == "f32" else PEAK_16BIT

    achieved = dom["flops"] / (dom["total_ms"] * 1e-3)
    traffic = profiled_traffic(dom["kernel"], args.workload) if args.mode == "step" else None
    roofline = {"bound": "mfma", "achieved": round(achieved / 1e12, 2), "peak": round(peak / 1e12, 1),
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic,
                "kernel": dom["kernel"], "launches_per_step": dom["launches"] / args.steps,
                "avg_launch_ms": round(dom["avg_ms"], 4),
                "flops_per_launch": dom["flops"] / dom["launches"]}
    breakdown = []
    for k in kernels:
        e = {"kernel": k["kernel"], "launches": k["launches"], "avg_ms": round(k["avg_ms"], 4),
             "share": round(k["total_ms"] / (ms_instrumented * args.steps), 4)}
        if k["flops"] > 0:
            e["tflops"] = round(k["flops"] / (k["total_ms"] * 1e-3) / 1e12, 1)
        if k["bytes"] > 0:
            e["gbps"] = round(k["bytes"] / (k["total_ms"] * 1e-3) / 1e9, 1)
        breakdown.append(e)

    line = {
        "metric": METRIC,
        "value": round(nmat / (ms * 1e-3), 3),
        "unit": "matrices/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": arithmetic_of(kernels),
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "matrices": nmat,
            "shapes": shapes_summary(shapes),
            "input_dtype": dtype,
            "mode": ("dmuon_step: momentum + Gram NS + update" if args.mode == "step"
                     else "dmuon_ns_batched" if batched else "dmuon_plan_ns"),
            "ns_steps": T,
            "coeffs": list(COEFFS),
            "precision": args.precision,
            "launch": "one HIP graph replay per step" if args.graph else "library calls per step",
            "inputs": "(count, rows, cols) batch tensors" if batched else "one tensor per matrix",
            "global_batch": nmat,
            "parallelism": "single GPU",
        },
        "tflops": round(tflops, 2),
        "pct_bf16_peak": round(100.0 * flops / (ms * 1e-3) / PEAK_16BIT, 2),
        "roofline": roofline,
        "kernel_timing": {"pass": "second run of the same steps, each launch bracketed by HIP events",
                          "ms_per_step_instrumented": round(ms_instrumented, 4)},
        "kernels": breakdown,
    }
    if args.mode == "step":
        desc = plan.describe()
        tt = desc["tune_table"]
        if isinstance(tt, str) and os.path.isabs(tt):
            real_root = os.path.realpath(ROOT)
            if os.path.realpath(tt).startswith(real_root + os.sep):
                tt = os.path.relpath(os.path.realpath(tt), real_root)
        line["config"]["tune_table"] = tt
        if len(desc["recurrence"]) > 1:
            line["buckets"] = bucket_report(dm, desc, shapes, W, G, B, T, args, dtype)
        # context: the element-wise optimizer the pages compare against, on
        # the same parameters and gradients
        aw = adamw_timing(dm, W, G, args)
        aw["dmuon_over_adamw"] = round(ms / aw["ms_per_step"], 2)
        line["adamw_context"] = aw
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(shapes, dtype, T, args.cpu_budget, seed + 1000)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
