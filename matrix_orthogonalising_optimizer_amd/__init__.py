"""MI355X-native batched Gram Newton-Schulz and fused Muon step.

Thin ctypes binding over libdmuon.so (C ABI declared in include/dmuon.h).
This module only marshals arguments: tensor data pointers, the current HIP
stream and scalars.  Every step of the computation runs in the HIP kernels of
the library; there is no host or PyTorch fallback, and every entry point
raises if the library has not been built.

Method: DMuon, "Efficient Distributed Muon Training with Near-Adam Overhead"
(gist.science technical summary, section 2.2 for the Gram-space iteration,
section 2.4 for per-shape tile selection, sections 1 and 5 for the Muon step).
"""

from __future__ import annotations

import ctypes
import json
import os

import numpy as np

__all__ = [
    "QUINTIC", "DmuonError", "load_library", "library_path", "ns_batched", "Plan",
    "version", "PREC", "SCALE", "timing_enable", "timing_report", "assign_owners", "profile_costs",
    "ASSIGN", "FORM", "ns_batched_noalloc", "release_workspace", "workspace_info",
    "adamw_step", "tune",
]

QUINTIC = (3.4445, -4.7750, 2.0315)

_HERE = os.path.dirname(os.path.abspath(__file__))
# DMUON_LIBRARY names another build of the library to load instead (for
# example one compiled with different options); default: the in-tree build
_LIB_PATH = os.environ.get("DMUON_LIBRARY") or os.path.join(_HERE, "libdmuon.so")

# enum values of include/dmuon.h
OK, EINVAL, EUNSUPPORTED, EHIP, ENOMEM, EPLAN = 0, -1, -2, -3, -4, -5
BF16, F32 = 0, 1
PREC = {"auto": 0, "f16": 1, "bf16": 2, "f32": 3}
SCALE = {"sqrt_ratio": 0, "none": 1}
ASSIGN = {"auto": 0, "exact": 1, "greedy": 2}
FORM = {"auto": 0, "gram": 1, "standard": 2}
STORAGE = {"auto": 0, "full": 1}
FUSED = {"auto": 0, "off": 1, "one": 2, "split": 3}
_ERR_NAMES = {EINVAL: "EINVAL", EUNSUPPORTED: "EUNSUPPORTED", EHIP: "EHIP", ENOMEM: "ENOMEM", EPLAN: "EPLAN"}


class DmuonError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_ERR_NAMES.get(code, code)}: {msg}")
        self.code = code


class _PlanOpts(ctypes.Structure):
    _fields_ = [
        ("precision", ctypes.c_int),
        ("scale_mode", ctypes.c_int),
        ("no_device", ctypes.c_int),
        ("eps", ctypes.c_float),
        ("max_workspace", ctypes.c_int64),
        ("tune_path", ctypes.c_char_p),
        ("form", ctypes.c_int),
        ("pad_ratio", ctypes.c_float),
        ("storage", ctypes.c_int),
        ("fused", ctypes.c_int),
    ]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load libdmuon.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it with "
            "`python -m matrix_orthogonalising_optimizer_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, f32, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    pp = ctypes.POINTER(ctypes.c_void_p)
    lib.dmuon_ns_batched.argtypes = [pp, i64, i64, i64, i32, f32, f32, f32, vp]
    lib.dmuon_ns_batched_f32.argtypes = [pp, i64, i64, i64, i32, f32, f32, f32, vp]
    lib.dmuon_ns_batched_ex.argtypes = [pp, i64, i64, i64, i32, i32, i32, f32, f32, f32, vp]
    lib.dmuon_ns_batched_noalloc.argtypes = [pp, i64, i64, i64, i32, f32, f32, f32, vp]
    lib.dmuon_release_workspace.argtypes = []
    lib.dmuon_adamw_step.argtypes = [pp, pp, pp, pp, ctypes.POINTER(i64), i64, i32, f32, f32, f32, f32, f32,
                                     i64, vp]
    lib.dmuon_workspace_info.argtypes = [ctypes.POINTER(i64), ctypes.POINTER(i64), ctypes.POINTER(ctypes.c_int32)]
    lib.dmuon_plan_opts_default.argtypes = [ctypes.POINTER(_PlanOpts)]
    lib.dmuon_plan_opts_default.restype = None
    lib.dmuon_plan.argtypes = [ctypes.POINTER(i64), ctypes.POINTER(i64), i64, i32,
                               ctypes.POINTER(_PlanOpts), ctypes.POINTER(vp)]
    lib.dmuon_plan_destroy.argtypes = [vp]
    lib.dmuon_plan_describe.argtypes = [vp, ctypes.c_char_p, ctypes.c_size_t]
    lib.dmuon_plan_describe.restype = i64
    lib.dmuon_step.argtypes = [vp, pp, pp, pp, f32, f32, f32, i32, i32, f32, f32, f32, vp]
    lib.dmuon_plan_ns.argtypes = [vp, pp, i32, f32, f32, f32, vp]
    lib.dmuon_timing_enable.argtypes = [i32]
    lib.dmuon_timing_enable.restype = i32
    lib.dmuon_timing_report.argtypes = [ctypes.c_char_p, ctypes.c_size_t]
    lib.dmuon_timing_report.restype = i64
    i32p, f64p = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_double)
    lib.dmuon_assign_owners.argtypes = [i32p, i64, i32p, ctypes.c_int32, f64p, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, i64, i32p, f64p, i32p]
    lib.dmuon_profile_costs.argtypes = [ctypes.POINTER(i64), ctypes.POINTER(i64), ctypes.c_int32, i32p,
                                        ctypes.c_int32, i32, f32, f32, f32, ctypes.c_int32, ctypes.c_int32,
                                        f64p, vp]
    lib.dmuon_tune.argtypes = [ctypes.POINTER(i64), ctypes.POINTER(i64), i64, i32, f32, f32, f32, ctypes.c_int32,
                               ctypes.c_int32, ctypes.c_char_p, vp]
    lib.dmuon_last_error.restype = ctypes.c_char_p
    lib.dmuon_version.restype = ctypes.c_char_p
    for name in ("dmuon_ns_batched", "dmuon_ns_batched_f32", "dmuon_ns_batched_ex", "dmuon_ns_batched_noalloc",
                 "dmuon_release_workspace", "dmuon_workspace_info", "dmuon_adamw_step", "dmuon_tune",
                 "dmuon_plan", "dmuon_plan_destroy", "dmuon_step", "dmuon_assign_owners",
                 "dmuon_profile_costs"):
        getattr(lib, name).restype = i32
    _lib = lib
    return lib


def _check(rc: int) -> None:
    if rc != OK:
        raise DmuonError(rc, load_library().dmuon_last_error().decode())


def version() -> str:
    return load_library().dmuon_version().decode()


def _ptr_array(ptrs):
    if not ptrs:
        return (ctypes.c_void_p * 1)()
    return (ctypes.c_void_p * len(ptrs))(*ptrs)


def _batch_ptrs(t, what: str):
    """(pointer array, rows, cols, count) of a contiguous (count, rows, cols)
    GPU tensor: matrix i starts i * rows * cols elements in."""
    if not t.is_cuda or t.dim() != 3 or not t.is_contiguous():
        raise ValueError(f"{what}: a batch tensor must be a contiguous 3-D GPU tensor (count, rows, cols)")
    count, rows, cols = (int(x) for x in t.shape)
    if count == 0:
        raise ValueError(f"{what}: empty batch")
    step = rows * cols * t.element_size()
    ptrs = np.arange(count, dtype=np.uint64) * np.uint64(step) + np.uint64(t.data_ptr())
    return (ctypes.c_void_p * count).from_buffer(ptrs), rows, cols, count


def _all_gpu_contiguous(ts) -> bool:
    return all(t.is_cuda and t.is_contiguous() for t in ts)


def _torch():
    import torch  # imported lazily so that the CPU-only parts need no GPU
    return torch


def _stream_handle(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _check_mats(mats, what: str):
    if len(mats) == 0:
        raise ValueError(f"{what}: empty list")
    t0 = mats[0]
    dt, dev = t0.dtype, t0.device
    # one pass per property when all is well; the loop below names the problem
    if (_all_gpu_contiguous(mats) and all(t.dim() == 2 for t in mats) and all(t.dtype is dt for t in mats)
            and all(t.device == dev for t in mats)):
        return
    for t in mats:
        if not t.is_cuda:
            raise ValueError(f"{what}: tensors must live on the GPU")
        if t.dim() != 2 or not t.is_contiguous():
            raise ValueError(f"{what}: tensors must be contiguous 2-D matrices")
        if t.dtype != t0.dtype or t.device != t0.device:
            raise ValueError(f"{what}: mixed dtype or device")


def ns_batched(mats, steps: int = 5, coeffs=QUINTIC, precision: str = "auto", stream=None) -> None:
    """Orthogonalise same-shape matrices in place (``dmuon_ns_batched_ex``).

    ``mats`` is a list of contiguous 2-D GPU tensors of one shape and dtype,
    or one contiguous 3-D tensor (count, rows, cols) holding the batch, whose
    pointers are formed without a Python pass over the matrices."""
    lib = load_library()
    torch = _torch()
    if isinstance(mats, torch.Tensor) and mats.dim() == 3:
        arr, rows, cols, count = _batch_ptrs(mats, "ns_batched")
        a, b, c = coeffs
        _check(lib.dmuon_ns_batched_ex(arr, rows, cols, count, _dtype_code(mats), PREC[precision], int(steps),
                                       a, b, c, _stream_handle(stream)))
        return
    mats = list(mats)
    _check_mats(mats, "ns_batched")
    shape = tuple(mats[0].shape)
    if any(tuple(t.shape) != shape for t in mats):
        raise ValueError("ns_batched: all matrices must share one shape")
    arr = _ptr_array([t.data_ptr() for t in mats])
    a, b, c = coeffs
    _check(lib.dmuon_ns_batched_ex(arr, shape[0], shape[1], len(mats), _dtype_code(mats[0]),
                                   PREC[precision], int(steps), a, b, c, _stream_handle(stream)))


def ns_batched_noalloc(mats, steps: int = 5, coeffs=QUINTIC, stream=None) -> None:
    """``ns_batched`` for bf16 matrices in the library's static device scratch
    (``dmuon_ns_batched_noalloc``): no device allocation on any path."""
    lib = load_library()
    mats = list(mats)
    _check_mats(mats, "ns_batched_noalloc")
    shape = tuple(mats[0].shape)
    if any(tuple(t.shape) != shape for t in mats):
        raise ValueError("ns_batched_noalloc: all matrices must share one shape")
    if _dtype_code(mats[0]) != BF16:
        raise ValueError("ns_batched_noalloc: bf16 matrices only")
    arr = _ptr_array([t.data_ptr() for t in mats])
    a, b, c = coeffs
    _check(lib.dmuon_ns_batched_noalloc(arr, shape[0], shape[1], len(mats), int(steps), a, b, c,
                                        _stream_handle(stream)))


def adamw_step(params, grads, exp_avgs, exp_avg_sqs, *, lr: float, step: int, betas=(0.9, 0.999),
               eps: float = 1e-8, weight_decay: float = 0.0, stream=None) -> None:
    """One fused AdamW step over lists of tensors, in place (``dmuon_adamw_step``).

    Parameters and gradients share one dtype (bfloat16 or float32); the
    moments are float32 tensors of the parameters' sizes.  ``step`` counts
    from 1."""
    lib = load_library()
    params, grads = list(params), list(grads)
    exp_avgs, exp_avg_sqs = list(exp_avgs), list(exp_avg_sqs)
    n = len(params)
    if not (n == len(grads) == len(exp_avgs) == len(exp_avg_sqs)) or n == 0:
        raise ValueError("adamw_step: need one grad and two moments per parameter")
    torch = _torch()
    dt = params[0].dtype
    numel = [t.numel() for t in params]
    ok = (_all_gpu_contiguous(params) and _all_gpu_contiguous(grads) and _all_gpu_contiguous(exp_avgs)
          and _all_gpu_contiguous(exp_avg_sqs) and all(t.dtype is dt for t in params)
          and all(t.dtype is dt for t in grads) and all(t.dtype is torch.float32 for t in exp_avgs)
          and all(t.dtype is torch.float32 for t in exp_avg_sqs)
          and [t.numel() for t in grads] == numel and [t.numel() for t in exp_avgs] == numel
          and [t.numel() for t in exp_avg_sqs] == numel)
    if not ok:
        raise ValueError("adamw_step: contiguous GPU tensors; params and grads of one dtype, float32 moments, "
                         "equal sizes per parameter")
    b1, b2 = betas
    nm = (ctypes.c_int64 * n)(*numel)
    _check(lib.dmuon_adamw_step(_ptr_array([t.data_ptr() for t in params]),
                                _ptr_array([t.data_ptr() for t in grads]),
                                _ptr_array([t.data_ptr() for t in exp_avgs]),
                                _ptr_array([t.data_ptr() for t in exp_avg_sqs]), nm, n, _dtype_code(params[0]),
                                lr, b1, b2, eps, weight_decay, int(step), _stream_handle(stream)))


def release_workspace() -> None:
    """Free the current device's implicit workspace (``dmuon_release_workspace``)."""
    _check(load_library().dmuon_release_workspace())


def workspace_info() -> dict:
    """Live and retired bytes of the implicit workspace (``dmuon_workspace_info``)."""
    live, ret, cnt = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
    _check(load_library().dmuon_workspace_info(ctypes.byref(live), ctypes.byref(ret), ctypes.byref(cnt)))
    return {"live_bytes": live.value, "retired_bytes": ret.value, "retired_count": cnt.value}


def timing_enable(enable: bool = True) -> None:
    """Bracket every library kernel launch with HIP events (dmuon_timing_enable)."""
    _check(load_library().dmuon_timing_enable(1 if enable else 0))


def timing_report() -> dict:
    """Per-kernel launch counts, times and algorithmic work; clears the records."""
    lib = load_library()
    buf = ctypes.create_string_buffer(1 << 20)
    need = lib.dmuon_timing_report(buf, len(buf))
    if need < 0:
        _check(int(need))
    if need >= len(buf):
        raise RuntimeError("timing report truncated")
    return json.loads(buf.value.decode())


def assign_owners(shape_of, batches, times, ranks: int, method: str = "auto", node_limit: int = 0):
    """Owner rank of every matrix (``dmuon_assign_owners``).

    ``shape_of[i]`` is matrix i's shape index; ``times[s][p]`` the cost of a
    batch of ``batches[p]`` matrices of shape s.  Returns
    ``(owners, makespan, optimal)``."""
    lib = load_library()
    shape_of = [int(x) for x in shape_of]
    batches = [int(x) for x in batches]
    flat = [float(t) for row in times for t in row]
    nshapes = len(times)
    if nshapes == 0 or any(len(row) != len(batches) for row in times):
        raise ValueError("assign_owners: times must be nshapes x len(batches)")
    so = (ctypes.c_int32 * max(1, len(shape_of)))(*shape_of)
    bt = (ctypes.c_int32 * max(1, len(batches)))(*batches)
    tm = (ctypes.c_double * max(1, len(flat)))(*flat)
    out = (ctypes.c_int32 * max(1, len(shape_of)))()
    mk, opt = ctypes.c_double(), ctypes.c_int32()
    _check(lib.dmuon_assign_owners(so, len(shape_of), bt, len(batches), tm, nshapes, int(ranks),
                                   ASSIGN[method], int(node_limit), out, ctypes.byref(mk), ctypes.byref(opt)))
    return [int(out[i]) for i in range(len(shape_of))], mk.value, bool(opt.value)


def profile_costs(shapes, batches, steps: int = 5, coeffs=QUINTIC, warmup: int = 1, repeats: int = 3,
                  stream=None):
    """Median milliseconds of ``dmuon_ns_batched`` per (shape, batch size) on the
    current device (``dmuon_profile_costs``); returns ``times[s][p]``."""
    lib = load_library()
    shapes = [(int(r), int(c)) for r, c in shapes]
    batches = [int(x) for x in batches]
    rows = (ctypes.c_int64 * max(1, len(shapes)))(*[r for r, _ in shapes])
    cols = (ctypes.c_int64 * max(1, len(shapes)))(*[c for _, c in shapes])
    bt = (ctypes.c_int32 * max(1, len(batches)))(*batches)
    tm = (ctypes.c_double * max(1, len(shapes) * len(batches)))()
    a, b, c = coeffs
    _check(lib.dmuon_profile_costs(rows, cols, len(shapes), bt, len(batches), int(steps), a, b, c,
                                   int(warmup), int(repeats), tm, _stream_handle(stream)))
    return [[tm[s * len(batches) + p] for p in range(len(batches))] for s in range(len(shapes))]


def tune(shapes, out_path: str, steps: int = 5, coeffs=QUINTIC, warmup: int = 1, repeats: int = 5,
         stream=None) -> dict:
    """Time the tile configurations of every recurrence bucket of ``shapes``
    on the current device and write the tune table to ``out_path``
    (``dmuon_tune``); returns the written table."""
    lib = load_library()
    shapes = [(int(r), int(c)) for r, c in shapes]
    n = len(shapes)
    rows = (ctypes.c_int64 * max(1, n))(*[r for r, _ in shapes])
    cols = (ctypes.c_int64 * max(1, n))(*[c for _, c in shapes])
    a, b, c = coeffs
    _check(lib.dmuon_tune(rows, cols, n, int(steps), a, b, c, int(warmup), int(repeats), str(out_path).encode(),
                          _stream_handle(stream)))
    with open(out_path) as fh:
        return json.load(fh)


class Plan:
    """Shape buckets, tile choices and workspace for repeated Muon steps."""

    def __init__(self, shapes, dtype="bf16", precision: str = "auto", scale_mode: str = "sqrt_ratio",
                 eps: float = 1e-7, device: bool = True, max_workspace: int = 0, tune_path=None,
                 form: str = "auto", pad_ratio: float = 0.0, storage: str = "auto",
                 fused: str = "auto"):
        lib = load_library()
        shapes = [(int(r), int(c)) for r, c in shapes]
        n = len(shapes)
        rows = (ctypes.c_int64 * max(1, n))(*[r for r, _ in shapes])
        cols = (ctypes.c_int64 * max(1, n))(*[c for _, c in shapes])
        opts = _PlanOpts()
        lib.dmuon_plan_opts_default(ctypes.byref(opts))
        opts.precision = PREC[precision]
        opts.scale_mode = SCALE[scale_mode]
        opts.no_device = 0 if device else 1
        opts.eps = eps
        opts.max_workspace = max_workspace
        opts.tune_path = tune_path.encode() if tune_path else None
        opts.form = FORM[form]
        opts.pad_ratio = pad_ratio
        opts.storage = STORAGE[storage]
        opts.fused = FUSED[fused]
        dcode = {"bf16": BF16, "f32": F32}[dtype] if isinstance(dtype, str) else _dtype_code(
            _torch().empty(0, dtype=dtype))
        handle = ctypes.c_void_p()
        _check(lib.dmuon_plan(rows, cols, n, dcode, ctypes.byref(opts), ctypes.byref(handle)))
        self._h = handle
        self.shapes = shapes
        self.dtype = dcode

    def describe(self) -> dict:
        lib = load_library()
        need = lib.dmuon_plan_describe(self._h, None, 0)
        if need < 0:
            _check(int(need))
        buf = ctypes.create_string_buffer(int(need) + 1)
        lib.dmuon_plan_describe(self._h, buf, len(buf))
        return json.loads(buf.value.decode())

    def step(self, params, grads, momenta, *, lr: float, weight_decay: float, mu: float,
             nesterov: bool = True, steps: int = 5, coeffs=QUINTIC, stream=None) -> None:
        """One fused Muon step over the planned matrices (``dmuon_step``).

        ``params``, ``grads`` and ``momenta`` are lists of one contiguous GPU
        tensor per planned matrix, in plan order (parameters and gradients in
        the plan's dtype, momenta fp32), or, when every planned matrix has
        one shape, three contiguous (count, rows, cols) tensors."""
        lib = load_library()
        torch = _torch()
        a, b, c = coeffs
        if isinstance(params, torch.Tensor) and params.dim() == 3:
            ptrs = self._batch_args(params, grads, momenta)
            _check(lib.dmuon_step(self._h, *ptrs, lr, weight_decay, mu, 1 if nesterov else 0, int(steps),
                                  a, b, c, _stream_handle(stream)))
            return
        params, grads, momenta = list(params), list(grads), list(momenta)
        if not (len(params) == len(grads) == len(momenta) == len(self.shapes)):
            raise ValueError("step: need one param, grad and momentum per planned matrix")
        if not self._args_ok(params, grads, momenta):
            self._explain_args(params, grads, momenta)
        _check(lib.dmuon_step(self._h, _ptr_array([t.data_ptr() for t in params]),
                              _ptr_array([t.data_ptr() for t in grads]),
                              _ptr_array([t.data_ptr() for t in momenta]), lr, weight_decay, mu,
                              1 if nesterov else 0, int(steps), a, b, c, _stream_handle(stream)))

    def ns(self, mats, *, steps: int = 5, coeffs=QUINTIC, stream=None) -> None:
        """The Gram Newton-Schulz map of every planned matrix, in place
        (``dmuon_plan_ns``): matrices of one short side share the recurrence's
        launches, whatever their long side.  ``mats`` is a list of one
        contiguous GPU tensor per planned matrix, in plan order and the plan's
        dtype, or one contiguous (count, rows, cols) tensor when every planned
        matrix has one shape."""
        lib = load_library()
        torch = _torch()
        a, b, c = coeffs
        wdt = torch.bfloat16 if self.dtype == BF16 else torch.float32
        if isinstance(mats, torch.Tensor) and mats.dim() == 3:
            if len(set(self.shapes)) != 1:
                raise ValueError("ns: a batch tensor needs a plan whose matrices share one shape")
            want = (len(self.shapes),) + self.shapes[0]
            if tuple(mats.shape) != want or mats.dtype != wdt:
                raise ValueError(f"ns: batch tensor {tuple(mats.shape)} {mats.dtype}, the plan needs {want} {wdt}")
            ptrs = _batch_ptrs(mats, "ns")[0]
        else:
            mats = list(mats)
            if len(mats) != len(self.shapes):
                raise ValueError(f"ns: {len(mats)} matrices for a plan of {len(self.shapes)}")
            for i, (t, shp) in enumerate(zip(mats, self.shapes)):
                if not (isinstance(t, torch.Tensor) and t.is_cuda and t.is_contiguous()):
                    raise ValueError(f"ns: matrix {i} must be a contiguous GPU tensor")
                if tuple(t.shape) != shp or t.dtype != wdt:
                    raise ValueError(f"ns: matrix {i} is {tuple(t.shape)} {t.dtype}, the plan needs {shp} {wdt}")
            ptrs = _ptr_array([t.data_ptr() for t in mats])
        _check(lib.dmuon_plan_ns(self._h, ptrs, int(steps), a, b, c, _stream_handle(stream)))

    def _batch_args(self, params, grads, momenta):
        # three (count, rows, cols) batch tensors for a plan of one shape
        torch = _torch()
        if not all(isinstance(t, torch.Tensor) and t.dim() == 3 for t in (grads, momenta)):
            raise ValueError("step: pass params, grads and momenta all as lists or all as 3-D batch tensors")
        if len(set(self.shapes)) != 1:
            raise ValueError("step: batch tensors need a plan whose matrices share one shape")
        want = (len(self.shapes),) + self.shapes[0]
        wdt = torch.bfloat16 if self.dtype == BF16 else torch.float32
        for name, t, dt in (("params", params, wdt), ("grads", grads, wdt), ("momenta", momenta, torch.float32)):
            if tuple(t.shape) != want:
                raise ValueError(f"step: {name} has shape {tuple(t.shape)}, the plan needs {want}")
            if t.dtype != dt:
                raise ValueError(f"step: {name} has dtype {t.dtype}, the plan needs {dt}")
        return tuple(_batch_ptrs(t, "step")[0] for t in (params, grads, momenta))

    def _args_ok(self, params, grads, momenta) -> bool:
        # a few passes over the lists with no per-matrix Python calls: for a
        # batch of small matrices these checks cost more than the GPU work
        torch = _torch()
        wdt = torch.bfloat16 if self.dtype == BF16 else torch.float32
        f32 = torch.float32
        sh = self.shapes
        return ([t.shape for t in params] == sh and [t.shape for t in grads] == sh
                and [t.shape for t in momenta] == sh
                and all(t.dtype is wdt for t in params) and all(t.dtype is wdt for t in grads)
                and all(t.dtype is f32 for t in momenta)
                and _all_gpu_contiguous(params) and _all_gpu_contiguous(grads) and _all_gpu_contiguous(momenta))

    def _explain_args(self, params, grads, momenta) -> None:
        # shapes of every matrix first, then dtypes, then placement
        triples = list(zip(params, grads, momenta))
        for i, ts in enumerate(triples):
            if any(tuple(t.shape) != self.shapes[i] for t in ts):
                raise ValueError(f"step: matrix {i} does not have the planned shape {self.shapes[i]}")
        for i, (w, g, m) in enumerate(triples):
            if _dtype_code(w) != self.dtype or _dtype_code(g) != self.dtype or _dtype_code(m) != F32:
                raise ValueError(f"step: matrix {i} has the wrong dtype")
        for i, ts in enumerate(triples):
            if not _all_gpu_contiguous(ts):
                raise ValueError(f"step: matrix {i} must be a contiguous GPU tensor")
        raise ValueError("step: invalid arguments")

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            lib = load_library()
            _check(lib.dmuon_plan_destroy(self._h))
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
