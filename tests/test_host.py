"""Host-side checks of libdmuon that need no GPU.

The library is loaded (it must have been built), every symbol declared in
include/dmuon.h must be exported, and the planner, the tune-table reader and
argument validation are exercised through host-only plans.  Validation happens
before any HIP call, so the error paths run here without a device.
"""

import ctypes
import json
import os
import re

import pytest

import oracle
import matrix_orthogonalising_optimizer_amd as dm
from matrix_orthogonalising_optimizer_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dm.library_path()):
        pytest.fail("libdmuon.so is not built: run __graft_entry__.build()")
    return dm.load_library()


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "dmuon.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dmuon_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_symbols()
    assert "dmuon_ns_batched" in names and "dmuon_step" in names and "dmuon_plan" in names
    for n in names:
        assert hasattr(lib, n), n


def test_version(lib):
    assert "gfx950" in dm.version()


def plan_groups(desc):
    gemm = [((g["rows"], g["cols"]), g["members"]) for g in desc["gemm"]]
    rec = [(b["m"], sorted(b["members"])) for b in desc["recurrence"]]
    return gemm, rec


@pytest.mark.parametrize("name", ["llama7b_layer", "vla_mix_200", "mlp70b_8x8192x28672",
                                  "bf16_64x128x512", "fp32_256x1024"])
def test_planner_matches_oracle_buckets(lib, name):
    shapes = synth.WORKLOADS[name][0]
    dtype = "f32" if synth.WORKLOADS[name][1] == "f32" else "bf16"
    p = dm.Plan(shapes, dtype=dtype, device=False)
    desc = p.describe()
    gemm, rec = plan_groups(desc)
    want = oracle.plan_buckets(shapes)
    assert gemm == [(k, v) for k, v in want["gemm"]]
    assert rec == [(k, sorted(v)) for k, v in want["recurrence"]]
    assert desc["count"] == len(shapes) and desc["device"] is False


def test_planner_mixed_order_and_transposes(lib):
    shapes = [(300, 700), (700, 300), (300, 700), (64, 64), (300, 300)]
    desc = dm.Plan(shapes, device=False).describe()
    gemm, rec = plan_groups(desc)
    want = oracle.plan_buckets(shapes)
    assert gemm == [(k, v) for k, v in want["gemm"]]
    assert rec == [(k, sorted(v)) for k, v in want["recurrence"]]
    tr = {(g["rows"], g["cols"]): g["transposed"] for g in desc["gemm"]}
    assert tr == {(300, 700): False, (700, 300): True, (64, 64): False, (300, 300): False}


@pytest.mark.parametrize("m", [1, 64, 100, 256, 1000, 4096, 8192])
def test_only_lower_tiles_are_launched(lib, m):
    # symmetric products touch nt (nt + 1) / 2 of the nt^2 output tiles
    desc = dm.Plan([(m, m + 5)], device=False).describe()
    b = desc["recurrence"][0]
    nt = -(-m // b["tile"])
    assert b["lower_tiles"] == nt * (nt + 1) // 2
    g = desc["gemm"][0]
    nts = -(-m // g["tile_syrk"])
    assert g["syrk_tiles"] == nts * (nts + 1) // 2


def test_workspace_scales_with_batch(lib):
    d1 = dm.Plan([(1024, 4096)], device=False).describe()
    d2 = dm.Plan([(1024, 4096)] * 3, device=False).describe()
    assert 2.9 * d1["workspace_bytes"] <= d2["workspace_bytes"] <= 3.1 * d1["workspace_bytes"]


def test_workspace_cap_is_enforced(lib):
    with pytest.raises(dm.DmuonError) as e:
        dm.Plan([(4096, 4096)], device=False, max_workspace=1 << 20)
    assert e.value.code == dm.ENOMEM


def test_tune_table_file(lib, tmp_path):
    path = tmp_path / "tune.json"
    path.write_text(json.dumps({"entries": [
        {"max_m": 512, "rec": 64, "syrk": 128, "final": 64},
        {"max_m": 1 << 30, "rec": 128, "syrk": 256, "final": 128}]}))
    desc = dm.Plan([(300, 900), (2048, 2048)], device=False, tune_path=str(path)).describe()
    assert desc["tune_table"] == str(path)
    g = {(x["rows"], x["cols"]): x for x in desc["gemm"]}
    assert (g[(300, 900)]["tile_syrk"], g[(300, 900)]["tile_final"]) == (128, 64)
    assert (g[(2048, 2048)]["tile_syrk"], g[(2048, 2048)]["tile_final"]) == (256, 128)
    r = {b["m"]: b["tile"] for b in desc["recurrence"]}
    assert r == {300: 64, 2048: 128}


@pytest.mark.parametrize("text", ["{}", "{\"entries\": []}", "{\"entries\": [{\"max_m\": 5}]}",
                                  "{\"entries\": [{\"max_m\": 9, \"rec\": 96, \"syrk\": 64, \"final\": 64}]}",
                                  "{\"entries\": [{\"max_m\": 9, \"rec\": 64, \"syrk\": 64, \"final\": 64},"
                                  " {\"max_m\": 3, \"rec\": 64, \"syrk\": 64, \"final\": 64}]}"])
def test_bad_tune_table_is_rejected(lib, tmp_path, text):
    path = tmp_path / "bad.json"
    path.write_text(text)
    with pytest.raises(dm.DmuonError) as e:
        dm.Plan([(64, 64)], device=False, tune_path=str(path))
    assert e.value.code == dm.EINVAL


def test_missing_tune_table_is_rejected(lib, tmp_path):
    with pytest.raises(dm.DmuonError) as e:
        dm.Plan([(64, 64)], device=False, tune_path=str(tmp_path / "nope.json"))
    assert e.value.code == dm.EINVAL


@pytest.mark.parametrize("shape", [(0, 4), (4, 0), (-1, 3)])
def test_plan_rejects_bad_shapes(lib, shape):
    with pytest.raises(dm.DmuonError) as e:
        dm.Plan([shape], device=False)
    assert e.value.code == dm.EINVAL


def test_plan_rejects_bad_options(lib):
    with pytest.raises(dm.DmuonError) as e:
        dm.Plan([(8, 8)], dtype="f32", precision="f16", device=False)
    assert e.value.code == dm.EUNSUPPORTED
    # bf16 data may run on the fp32 path (inputs widened in the workspace)
    d = dm.Plan([(8, 8)], dtype="bf16", precision="f32", device=False).describe()
    assert d["recurrence"][0]["fp32"] is True
    rows = (ctypes.c_int64 * 1)(8)
    h = ctypes.c_void_p()
    assert lib.dmuon_plan(rows, rows, 0, 0, None, ctypes.byref(h)) == dm.EINVAL
    assert lib.dmuon_plan(rows, rows, 1, 7, None, ctypes.byref(h)) == dm.EINVAL
    assert lib.dmuon_plan(None, rows, 1, 0, None, ctypes.byref(h)) == dm.EINVAL
    assert lib.dmuon_plan(rows, rows, 1, 0, None, None) == dm.EINVAL


def test_fused_split_choice():
    # AUTO runs the fused map as two launches (recurrence, then the final
    # product per 128 columns) for groups of at most 64 matrices of short
    # side above 64; SPLIT always, ONE and OFF never; the split region (Q's
    # image and two scalars per matrix) is part of the workspace.  fp16 state
    # throughout (near-square shapes would take the fp32 path under AUTO
    # precision)
    cases = [((128, 512), 64, "auto", True), ((128, 512), 65, "auto", False), ((64, 256), 64, "auto", False),
             ((64, 256), 64, "split", True), ((70, 150), 8, "auto", True), ((7, 13), 2, "split", True),
             ((128, 512), 64, "one", False)]
    for shape, n, fused, split in cases:
        d = dm.Plan([shape] * n, device=False, fused=fused, precision="f16").describe()
        assert d["recurrence"][0]["fused"], (shape, fused)
        assert d["gemm"][0]["split"] is split, (shape, n, fused, d["gemm"][0])
    one = dm.Plan([(128, 512)] * 64, device=False, fused="one").describe()["workspace_bytes"]
    split = dm.Plan([(128, 512)] * 64, device=False, fused="split").describe()["workspace_bytes"]
    assert split - one >= 64 * (32768 + 16)
    off = dm.Plan([(128, 512)] * 64, device=False, fused="off").describe()
    assert not off["recurrence"][0]["fused"] and off["gemm"][0]["split"] is False


def test_plan_ns_argument_checks():
    # Plan.ns refuses a wrong count, shape, dtype or a host tensor before the
    # library is called (a host-only plan would refuse to run anyway)
    import torch
    plan = dm.Plan([(4, 8), (8, 4)], device=False)
    good = [torch.zeros(4, 8, dtype=torch.bfloat16), torch.zeros(8, 4, dtype=torch.bfloat16)]
    with pytest.raises(ValueError, match="a plan of 2"):
        plan.ns(good[:1])
    with pytest.raises(ValueError, match="GPU tensor"):
        plan.ns(good)
    with pytest.raises(ValueError, match="share one shape"):
        plan.ns(torch.zeros(2, 4, 8, dtype=torch.bfloat16))
    plan.close()


def test_batch_tensor_pointers_and_checks():
    # a (count, rows, cols) batch tensor: matrix i starts i * rows * cols
    # elements past the base; anything but a contiguous 3-D GPU tensor is
    # refused before the library is called
    import torch

    class Fake:
        is_cuda = True
        shape = (5, 3, 7)

        def dim(self):
            return 3

        def is_contiguous(self):
            return True

        def element_size(self):
            return 2

        def data_ptr(self):
            return 0x7F0000001000

    arr, rows, cols, count = dm._batch_ptrs(Fake(), "ns_batched")
    assert (rows, cols, count) == (3, 7, 5)
    assert [arr[i] for i in range(count)] == [0x7F0000001000 + i * 3 * 7 * 2 for i in range(count)]
    with pytest.raises(ValueError, match="contiguous 3-D GPU tensor"):
        dm.ns_batched(torch.zeros(4, 8, 16, dtype=torch.bfloat16))  # on the CPU
    f = Fake()
    f.is_contiguous = lambda: False
    with pytest.raises(ValueError, match="contiguous 3-D GPU tensor"):
        dm._batch_ptrs(f, "ns_batched")
    f = Fake()
    f.shape = (0, 3, 7)
    with pytest.raises(ValueError, match="empty batch"):
        dm._batch_ptrs(f, "ns_batched")


def test_step_batch_tensor_checks():
    # step takes three (count, rows, cols) batch tensors for a plan of one
    # shape; mixed forms, wrong shapes or dtypes, a plan of several shapes and
    # CPU tensors are refused before the library is called
    import torch
    plan = dm.Plan([(8, 16)] * 3, device=False)
    W = torch.zeros(3, 8, 16, dtype=torch.bfloat16)
    G, B = W.clone(), torch.zeros(3, 8, 16)
    kw = dict(lr=0.02, weight_decay=0.1, mu=0.95)
    with pytest.raises(ValueError, match="all as lists or all as 3-D batch tensors"):
        plan.step(W, list(G), B, **kw)
    with pytest.raises(ValueError, match="momenta has dtype"):
        plan.step(W, G, B.bfloat16(), **kw)
    with pytest.raises(ValueError, match=r"params has shape \(2, 8, 16\)"):
        plan.step(W[:2], G[:2], B[:2], **kw)
    with pytest.raises(ValueError, match="contiguous 3-D GPU tensor"):
        plan.step(W, G, B, **kw)
    with pytest.raises(ValueError, match="share one shape"):
        dm.Plan([(8, 16), (4, 4)], device=False).step(W, G, B, **kw)


def test_binding_rejects_bad_step_arguments(lib):
    # the binding checks shapes, dtypes, contiguity and placement before any
    # library call, naming the first offending matrix; CPU tensors reach the
    # last check (a plan made without a device never runs)
    import torch
    shapes = [(8, 16), (8, 16), (4, 4)]
    plan = dm.Plan(shapes, device=False)

    def mats(dtype, override=None):
        ts = [torch.zeros(s, dtype=dtype) for s in shapes]
        if override:
            ts[override[0]] = override[1]
        return ts

    W, G, B = mats(torch.bfloat16), mats(torch.bfloat16), mats(torch.float32)
    kw = dict(lr=0.02, weight_decay=0.1, mu=0.95)
    with pytest.raises(ValueError, match="one param, grad and momentum"):
        plan.step(W[:2], G, B, **kw)
    with pytest.raises(ValueError, match="matrix 2 does not have the planned shape"):
        plan.step(W, mats(torch.bfloat16, (2, torch.zeros(4, 5, dtype=torch.bfloat16))), B, **kw)
    with pytest.raises(ValueError, match="matrix 1 does not have the planned shape"):
        plan.step(W, G, mats(torch.float32, (1, torch.zeros(16, 8))), **kw)
    with pytest.raises(ValueError, match="matrix 1 has the wrong dtype"):
        plan.step(mats(torch.bfloat16, (1, torch.zeros(8, 16))), G, B, **kw)
    with pytest.raises(ValueError, match="matrix 0 has the wrong dtype"):
        plan.step(W, G, mats(torch.bfloat16), **kw)
    with pytest.raises(ValueError, match="matrix 0 must be a contiguous GPU tensor"):
        plan.step(W, G, B, **kw)
    with pytest.raises(ValueError, match="empty list"):
        dm.ns_batched([])
    with pytest.raises(ValueError, match="must live on the GPU"):
        dm.ns_batched([torch.zeros(8, 16, dtype=torch.bfloat16)])


def test_small_buckets_run_fp32_under_auto(lib):
    # 16-bit operands are not accurate enough on small square Gram matrices;
    # AUTO runs near-square m <= 128 on fp32 MFMA, wide m <= 128 (n >= 2 m)
    # and everything larger on 16-bit MFMA
    shapes = [(64, 64), (128, 512), (96, 191), (129, 129), (4096, 4096)]
    d = dm.Plan(shapes, device=False).describe()
    assert {b["m"]: b["fp32"] for b in d["recurrence"]} == {
        64: True, 128: False, 96: True, 129: False, 4096: False}
    d = dm.Plan([(64, 64)], precision="f16", device=False).describe()
    assert d["recurrence"][0]["fp32"] is False
    # one near-square member keeps the whole bucket on fp32
    d = dm.Plan([(100, 400), (100, 150)], device=False).describe()
    assert d["recurrence"][0]["fp32"] is True


def test_fused_kernel_eligibility(lib):
    # 16-bit Gram buckets of short side <= 128 whose members are all stored
    # rows <= cols run the one-launch kernel; transposed members, the
    # standard form, fp32 buckets and DMUON_FUSED_OFF do not
    def fused(shapes, **kw):
        d = dm.Plan(shapes, device=False, **kw).describe()
        return {b["m"]: b["fused"] for b in d["recurrence"]}
    assert fused([(128, 512), (64, 64), (4096, 4096)]) == {128: True, 64: False, 4096: False}
    assert fused([(64, 64)], precision="f16") == {64: True}
    assert fused([(128, 512), (512, 128)]) == {128: False}
    assert fused([(128, 512)], fused="off") == {128: False}
    assert fused([(128, 512)], form="standard") == {128: False}
    assert fused([(128, 512)], dtype="f32") == {128: False}
    assert fused([(129, 512)]) == {129: False}
    with pytest.raises(KeyError):
        dm.Plan([(8, 8)], device=False, fused="on")
    opts = dm._PlanOpts()
    lib.dmuon_plan_opts_default(ctypes.byref(opts))
    assert opts.fused == 0
    opts.fused = 7
    rows = (ctypes.c_int64 * 1)(8)
    h = ctypes.c_void_p()
    opts.no_device = 1
    assert lib.dmuon_plan(rows, rows, 1, 0, ctypes.byref(opts), ctypes.byref(h)) == dm.EINVAL


def test_step_on_host_only_plan_is_rejected(lib):
    p = dm.Plan([(8, 8)], device=False)
    arr = (ctypes.c_void_p * 1)(1)
    rc = lib.dmuon_step(p._h, arr, arr, arr, 0.02, 0.1, 0.95, 1, 5, 3.4445, -4.775, 2.0315, None)
    assert rc == dm.EPLAN
    assert lib.dmuon_step(None, arr, arr, arr, 0.02, 0.1, 0.95, 1, 5, 1.0, 0.0, 0.0, None) == dm.EPLAN


def test_ns_batched_validates_before_touching_the_device(lib):
    one = (ctypes.c_void_p * 1)(16)
    null = (ctypes.c_void_p * 1)(None)
    a, b, c = dm.QUINTIC
    f = lib.dmuon_ns_batched
    assert f(None, 4, 4, 1, 5, a, b, c, None) == dm.EINVAL
    assert f(one, 0, 4, 1, 5, a, b, c, None) == dm.EINVAL
    assert f(one, 4, -2, 1, 5, a, b, c, None) == dm.EINVAL
    assert f(one, 4, 4, 0, 5, a, b, c, None) == dm.EINVAL
    assert f(one, 4, 4, 1, -1, a, b, c, None) == dm.EINVAL
    assert f(null, 4, 4, 1, 5, a, b, c, None) == dm.EINVAL
    assert f(one, 4, 4, 1, 5, float("nan"), b, c, None) == dm.EINVAL
    assert "NULL" in lib.dmuon_last_error().decode() or "coeff" in lib.dmuon_last_error().decode()
    ex = lib.dmuon_ns_batched_ex
    assert ex(one, 4, 4, 1, 9, 0, 5, a, b, c, None) == dm.EINVAL          # dtype
    assert ex(one, 4, 4, 1, 0, 7, 5, a, b, c, None) == dm.EINVAL          # precision
    assert ex(one, 4, 4, 1, dm.F32, 1, 5, a, b, c, None) == dm.EUNSUPPORTED  # f32 data, f16 MFMA
    assert ex(one, 4, 4, 1, dm.F32, 2, 5, a, b, c, None) == dm.EUNSUPPORTED  # f32 data, bf16 MFMA
    # coefficients whose recurrence overflows fp16 cannot be forced onto the fp16 path
    assert ex(one, 512, 512, 1, dm.BF16, 1, 3, 40.0, 0.0, 0.0, None) == dm.EUNSUPPORTED
    assert "overflow" in lib.dmuon_last_error().decode()
    # so can long runs whose Q scale would flush the converged directions:
    # the cubic's null directions grow like 1.5^k, beyond 2^12 x 8192 from 43 steps
    assert ex(one, 64, 256, 1, dm.BF16, 1, 43, 1.5, -0.5, 0.0, None) == dm.EUNSUPPORTED
    assert ex(one, 64, 256, 1, dm.BF16, 1, 70, 1.5, -0.5, 0.0, None) == dm.EUNSUPPORTED


def test_plan_destroy_null_is_noop(lib):
    assert lib.dmuon_plan_destroy(None) == dm.OK


def test_form_choice_per_bucket(lib):
    shapes = [(300, 300), (512, 768), (768, 512), (64, 64), (256, 1024)]
    form = lambda **kw: {b["m"]: b["form"] for b in dm.Plan(shapes, device=False, **kw).describe()["recurrence"]}
    # fp16 products: the Gram form everywhere under AUTO
    assert set(form().values()) == {"gram"}
    # plain bf16 products: standard where every member has n <= 2 m
    assert form(precision="bf16") == {300: "standard", 512: "standard", 64: "standard", 256: "gram"}
    # forced standard: every 16-bit bucket; fp32 buckets (m <= 128 under AUTO precision) keep the Gram form
    assert form(form="standard") == {300: "standard", 512: "standard", 64: "gram", 256: "standard"}
    assert set(form(form="gram", precision="bf16").values()) == {"gram"}


def test_standard_form_workspace_holds_the_second_iterate(lib):
    g = dm.Plan([(512, 768)] * 2, device=False, form="gram").describe()["workspace_bytes"]
    s = dm.Plan([(512, 768)] * 2, device=False, form="standard").describe()["workspace_bytes"]
    assert s - g >= 2 * 512 * 768 * 2


def test_bad_form_is_rejected(lib):
    rows = (ctypes.c_int64 * 1)(8)
    opts = dm._PlanOpts()
    lib.dmuon_plan_opts_default(ctypes.byref(opts))
    assert opts.form == 0
    opts.form = 7
    opts.no_device = 1
    h = ctypes.c_void_p()
    assert lib.dmuon_plan(rows, rows, 1, 0, ctypes.byref(opts), ctypes.byref(h)) == dm.EINVAL


def test_padding_merges_similar_short_sides(lib):
    shapes = [(240, 512), (256, 640), (300, 300), (200, 900), (1000, 1000), (1024, 2048), (100, 100), (120, 400)]
    buckets = lambda r: {b["m"]: sorted(b["members"]) for b in
                         dm.Plan(shapes, device=False, pad_ratio=r).describe()["recurrence"]}
    # largest side first: 1024 opens 1024, 1000 joins; 300 opens round_up(300, 64) = 320;
    # 256 joins 320 (<= 1.25 * 256); 240 opens 256 (320 > 300); 200 would round to 256 > 250;
    # 120 x 400 (wide, a 16-bit bucket) opens 128; the fp32 bucket (100 x 100) is never padded
    assert buckets(0.25) == {256: [0], 320: [1, 2], 200: [3], 1024: [4, 5], 100: [6], 128: [7]}
    assert buckets(0.1) == {256: [0, 1], 320: [2], 200: [3], 1024: [4, 5], 100: [6], 128: [7]}
    assert buckets(0.0) == {240: [0], 256: [1], 300: [2], 200: [3], 1000: [4], 1024: [5], 100: [6], 120: [7]}
    with pytest.raises(dm.DmuonError):
        dm.Plan(shapes, device=False, pad_ratio=1.5)


def test_storage_choice_per_bucket(lib):
    # lower-triangle storage needs 16-bit Gram buckets whose every product
    # covers whole tiles of 128 or 256; full storage elsewhere or on request
    shapes = [(512, 1024), (1024, 512), (256, 768), (300, 700), (640, 1000), (96, 384), (1280, 768)]
    rec = {b["m"]: b for b in dm.Plan(shapes, device=False).describe()["recurrence"]}
    assert rec[512]["storage"] == "lower" and rec[512]["tile"] == 256
    assert rec[256]["storage"] == "lower" and rec[256]["tile"] == 128
    assert rec[768]["storage"] == "lower"      # 3 x 3 tiles of 256
    assert rec[300]["storage"] == "full"       # not a multiple of the tile
    assert rec[640]["storage"] == "full"       # 1000 columns: the final product is ragged
    assert rec[96]["storage"] == "full"        # 96 is not a multiple of the tile
    full = dm.Plan(shapes, device=False, storage="full").describe()["recurrence"]
    assert all(b["storage"] == "full" for b in full)
    std = dm.Plan([(512, 512)], device=False, form="standard").describe()["recurrence"]
    assert std[0]["storage"] == "full"         # no symmetric states


def test_bad_storage_is_rejected(lib):
    rows = (ctypes.c_int64 * 1)(8)
    opts = dm._PlanOpts()
    lib.dmuon_plan_opts_default(ctypes.byref(opts))
    assert opts.storage == 0
    opts.storage = 5
    opts.no_device = 1
    h = ctypes.c_void_p()
    assert lib.dmuon_plan(rows, rows, 1, 0, ctypes.byref(opts), ctypes.byref(h)) == dm.EINVAL


def test_fp32_buckets_shrink_tiles_to_fill_the_gpu(lib, tmp_path):
    # fp32 MFMA is 16x slower than 16-bit: with the built-in table an fp32
    # bucket whose launch would have fewer tiles than the GPU's 256 CUs uses
    # smaller tiles (down to 64); a tune-table file is taken as given
    def tiles(shapes, **kw):
        d = dm.Plan(shapes, dtype="f32", device=False, **kw).describe()
        return ([b["tile"] for b in d["recurrence"]],
                [(g["tile_syrk"], g["tile_final"]) for g in d["gemm"]])
    assert tiles([(256, 1024)]) == ([64], [(64, 64)])
    assert tiles([(1024, 1024)] * 2) == ([64], [(64, 64)])
    assert tiles([(4096, 4096)]) == ([128], [(128, 128)])   # 528 tiles of 128
    # 16-bit buckets keep the table's tiles
    d = dm.Plan([(256, 1024)], device=False).describe()
    assert d["recurrence"][0]["tile"] == 128
    path = tmp_path / "tune.json"
    path.write_text(json.dumps({"entries": [{"max_m": 1 << 30, "rec": 128, "syrk": 128, "final": 128}]}))
    assert tiles([(256, 1024)], tune_path=str(path)) == ([128], [(128, 128)])


def test_kernel_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    # the committed counter summaries stay valid across comment edits of the
    # kernel sources, and not across any change of code
    import shutil
    import bench
    src = os.path.join(os.path.dirname(os.path.abspath(dm.__file__)), "csrc")
    dst = tmp_path / "matrix_orthogonalising_optimizer_amd" / "csrc"
    dst.mkdir(parents=True)
    for f in ("gemm_impl.h", "kernels.h"):
        shutil.copy(os.path.join(src, f), dst / f)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    base = bench.kernel_source_sha256()
    with open(dst / "kernels.h", "a") as fh:
        fh.write("\n// a comment\n/* and a block\n   comment */\n\n")
    assert bench.kernel_source_sha256() == base
    with open(dst / "kernels.h", "a") as fh:
        fh.write("constexpr int kExtra = 1;\n")
    assert bench.kernel_source_sha256() != base


def test_plan_log_prints_the_description():
    # DMUON_LOG=1 prints each new plan's JSON description to stderr
    import subprocess
    import sys
    code = ("import matrix_orthogonalising_optimizer_amd as dm; "
            "dm.Plan([(64, 128), (4096, 4096)], device=False)")
    env = dict(os.environ, DMUON_LOG="1")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    line = [ln for ln in r.stderr.splitlines() if ln.startswith("dmuon plan: ")]
    assert len(line) == 1, r.stderr
    desc = json.loads(line[0][len("dmuon plan: "):])
    assert desc["count"] == 2 and [b["m"] for b in desc["recurrence"]] == [64, 4096]
    env["DMUON_LOG"] = "0"
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=120)
    assert "dmuon plan" not in r.stderr


def test_noalloc_entry_point_validates_before_any_device_call(lib):
    # argument errors are reported before the scratch is looked up
    arr = (ctypes.c_void_p * 1)()
    assert lib.dmuon_ns_batched_noalloc(None, 4, 4, 1, 5, 3.4445, -4.775, 2.0315, None) == dm.EINVAL
    assert lib.dmuon_ns_batched_noalloc(arr, 4, 4, 1, 5, 3.4445, -4.775, 2.0315, None) == dm.EINVAL  # NULL entry
    assert lib.dmuon_ns_batched_noalloc(arr, 0, 4, 1, 5, 3.4445, -4.775, 2.0315, None) == dm.EINVAL
    assert b"ptrs" in lib.dmuon_last_error() or b"positive" in lib.dmuon_last_error()


def test_tune_table_batch_classes(lib, tmp_path):
    # entries keyed by (max_m, max_batch): the first entry with m <= max_m
    # and bucket size <= max_batch applies; else the last entry
    path = tmp_path / "tune.json"
    path.write_text(json.dumps({"arch": "gfx950", "entries": [
        {"max_m": 256, "max_batch": 4, "rec": 64, "syrk": 64, "final": 64},
        {"max_m": 256, "rec": 128, "syrk": 128, "final": 128},
        {"max_m": 2048, "max_batch": 10, "rec": 128, "syrk": 256, "final": 256},
        {"max_m": 4096, "rec": 256, "syrk": 256, "final": 256}], "measured": [{"m": 1}]}))

    def rec_tiles(shapes):
        d = dm.Plan(shapes, device=False, tune_path=str(path)).describe()
        return {b["m"]: (b["tile"], b["count"]) for b in d["recurrence"]}

    assert rec_tiles([(256, 512)] * 4) == {256: (64, 4)}
    assert rec_tiles([(256, 512)] * 5) == {256: (128, 5)}
    assert rec_tiles([(1024, 1024)] * 10 + [(256, 256)] * 2) == {1024: (128, 10), 256: (64, 2)}
    assert rec_tiles([(1024, 1024)] * 11) == {1024: (256, 11)}       # next entry with room for 11
    assert rec_tiles([(8192, 8192)]) == {8192: (256, 1)}            # beyond every entry: the last


@pytest.mark.parametrize("entries", [
    [{"max_m": 256, "max_batch": 8, "rec": 64, "syrk": 64, "final": 64},
     {"max_m": 256, "max_batch": 8, "rec": 64, "syrk": 64, "final": 64}],       # repeated key
    [{"max_m": 256, "max_batch": 9, "rec": 64, "syrk": 64, "final": 64},
     {"max_m": 256, "max_batch": 8, "rec": 64, "syrk": 64, "final": 64}],       # decreasing batch
    [{"max_m": 256, "max_batch": 0, "rec": 64, "syrk": 64, "final": 64}],       # non-positive batch
])
def test_tune_table_batch_order_is_checked(lib, tmp_path, entries):
    path = tmp_path / "bad.json"
    path.write_text(json.dumps({"entries": entries}))
    with pytest.raises(dm.DmuonError) as e:
        dm.Plan([(64, 64)], device=False, tune_path=str(path))
    assert e.value.code == dm.EINVAL


def test_tune_rejects_bad_arguments_before_any_device_call(lib):
    rows = (ctypes.c_int64 * 1)(64)
    assert lib.dmuon_tune(rows, rows, 1, 5, 3.4445, -4.775, 2.0315, 1, 0, b"/tmp/x.json", None) == dm.EINVAL
    assert lib.dmuon_tune(rows, rows, 0, 5, 3.4445, -4.775, 2.0315, 1, 3, b"/tmp/x.json", None) == dm.EINVAL
    assert lib.dmuon_tune(rows, rows, 1, 5, 3.4445, -4.775, 2.0315, 1, 3, None, None) == dm.EINVAL


def test_tune_tables_merge_into_one_sorted_table(lib, tmp_path):
    from matrix_orthogonalising_optimizer_amd import autotune as tune
    t1 = {"arch": "gfx950", "entries": [{"max_m": 1024, "max_batch": 100, "rec": 256, "syrk": 256, "final": 256},
                                        {"max_m": 256, "max_batch": 50, "rec": 64, "syrk": 64, "final": 64}],
          "measured": [{"m": 256, "count": 50, "candidates": []}]}
    t2 = {"arch": "gfx950", "entries": [{"max_m": 256, "max_batch": 8, "rec": 128, "syrk": 128, "final": 128}]}
    m = tune.merge([("a", t1), ("b", t2)])
    assert [(e["max_m"], e.get("max_batch")) for e in m["entries"]] == [(256, 8), (256, None), (1024, None)]
    assert m["measured"][0]["workload"] == "a" and m["workloads"] == ["a", "b"]
    path = tmp_path / "t.json"
    path.write_text(json.dumps(m))
    d = dm.Plan([(256, 256)] * 9 + [(512, 1024)], device=False, tune_path=str(path)).describe()
    assert {b["m"]: b["tile"] for b in d["recurrence"]} == {256: 64, 512: 256}
