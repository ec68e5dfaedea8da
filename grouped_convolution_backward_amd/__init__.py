"""Grouped 1D/2D/3D convolution backward-weight (wgrad), and backward data
(dgrad) of the same convolution, for MI355X (gfx950).

A thin ctypes binding over libwgrad.so, whose C ABI is include/wgrad.h. The
functions keep the ABI's names (``wgrad_plan``, ``wgrad_run``,
``wgrad_workspace_bytes``, ``wgrad_plan_query``, ``wgrad_plan_describe``,
``wgrad_plan_destroy``, ``wgrad_last_error``, ``wgrad_dgrad_plan``,
``wgrad_dgrad_run``, ``wgrad_run_noalloc``); this module only marshals
arguments. Every step of the computation runs in the HIP kernels; there is
no CPU or PyTorch fallback, and loading fails loudly if the library has not
been built (``python -m grouped_convolution_backward_amd.build``).

PyTorch is used for device memory and streams only: tensors are passed as
raw device pointers together with ``torch.cuda.current_stream()``.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwgrad.so")

BF16, FP16, FP32 = 0, 1, 2
DTYPES = {"bf16": BF16, "fp16": FP16, "fp32": FP32}
VARIANT_AUTO, VARIANT_MFMA, VARIANT_DEPTHWISE, VARIANT_ROWSLAB, VARIANT_DGRAD = 0, 1, 2, 3, 4
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP = 0, 1, 2, 3
NOALLOC_SCRATCH_BYTES = 16 << 20   # WGRAD_NOALLOC_SCRATCH_BYTES


class WgradError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"wgrad error {code}: {msg}")
        self.code = code


class wgrad_problem(ctypes.Structure):
    _fields_ = [
        ("ndim", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("G", ctypes.c_int64), ("N", ctypes.c_int64), ("C", ctypes.c_int64), ("K", ctypes.c_int64),
        ("in_len", ctypes.c_int64 * 3), ("filt_len", ctypes.c_int64 * 3),
        ("stride", ctypes.c_int64 * 3), ("dilation", ctypes.c_int64 * 3),
        ("pad_lo", ctypes.c_int64 * 3), ("pad_hi", ctypes.c_int64 * 3),
    ]


class wgrad_overrides(ctypes.Structure):
    _fields_ = [("split_k", ctypes.c_int32), ("group_merge", ctypes.c_int32),
                ("variant", ctypes.c_int32), ("tile", ctypes.c_int32)]


class wgrad_plan_info(ctypes.Structure):
    _fields_ = [
        ("out_len", ctypes.c_int64 * 3), ("gemm_m", ctypes.c_int64), ("gemm_n", ctypes.c_int64),
        ("gemm_k", ctypes.c_int64), ("variant", ctypes.c_int32), ("tile", ctypes.c_int32),
        ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32), ("tile_k", ctypes.c_int32),
        ("split_k", ctypes.c_int32), ("group_merge", ctypes.c_int32), ("vector_width", ctypes.c_int32),
        ("grid_main", ctypes.c_int64), ("grid_reduce", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_int64), ("num_cus", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]


# every symbol include/wgrad.h declares
EXPORTS = ("wgrad_plan", "wgrad_workspace_bytes", "wgrad_run", "wgrad_run_stage", "wgrad_plan_query",
           "wgrad_plan_describe", "wgrad_plan_destroy", "wgrad_last_error", "wgrad_version",
           "wgrad_dgrad_plan", "wgrad_dgrad_run", "wgrad_run_noalloc", "wgrad_probe_transpose_read")

_lib = None


def load_library():
    """Load libwgrad.so; raises if it is missing (no fallback path exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run python -m grouped_convolution_backward_amd.build")
    # torch ships its own HIP runtime with the same soname as /opt/rocm's; load
    # it first so that this library binds to the runtime that owns torch's
    # streams and allocations (one runtime per process)
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    vp = ctypes.c_void_p
    lib.wgrad_plan.argtypes = [ctypes.POINTER(wgrad_problem), ctypes.POINTER(wgrad_overrides),
                               ctypes.c_int, ctypes.POINTER(vp)]
    lib.wgrad_plan.restype = ctypes.c_int
    lib.wgrad_workspace_bytes.argtypes = [vp]
    lib.wgrad_workspace_bytes.restype = ctypes.c_size_t
    lib.wgrad_run.argtypes = [vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.wgrad_run.restype = ctypes.c_int
    lib.wgrad_run_stage.argtypes = [vp, ctypes.c_int, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.wgrad_run_stage.restype = ctypes.c_int
    lib.wgrad_plan_query.argtypes = [vp, ctypes.POINTER(wgrad_plan_info)]
    lib.wgrad_plan_query.restype = ctypes.c_int
    lib.wgrad_plan_describe.argtypes = [vp]
    lib.wgrad_plan_describe.restype = ctypes.c_char_p
    lib.wgrad_plan_destroy.argtypes = [vp]
    lib.wgrad_plan_destroy.restype = None
    lib.wgrad_last_error.argtypes = []
    lib.wgrad_last_error.restype = ctypes.c_char_p
    lib.wgrad_version.argtypes = []
    lib.wgrad_version.restype = ctypes.c_char_p
    lib.wgrad_dgrad_plan.argtypes = [ctypes.POINTER(wgrad_problem), ctypes.POINTER(wgrad_overrides),
                                     ctypes.c_int, ctypes.POINTER(vp)]
    lib.wgrad_dgrad_plan.restype = ctypes.c_int
    lib.wgrad_dgrad_run.argtypes = [vp, vp, vp, vp, vp]
    lib.wgrad_dgrad_run.restype = ctypes.c_int
    lib.wgrad_run_noalloc.argtypes = [vp, vp, vp, vp, vp]
    lib.wgrad_run_noalloc.restype = ctypes.c_int
    lib.wgrad_probe_transpose_read.argtypes = [vp, vp]
    lib.wgrad_probe_transpose_read.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(rc: int):
    if rc != OK:
        raise WgradError(rc, load_library().wgrad_last_error().decode())


def make_problem(p: dict) -> wgrad_problem:
    """Problem dict (keys as in the workloads module) -> C struct."""
    s = wgrad_problem()
    nd = int(p["ndim"])
    s.ndim = nd
    s.in_dtype = DTYPES[p["in_dtype"]]
    s.out_dtype = DTYPES[p.get("out_dtype", p["in_dtype"])]
    s.reserved = 0
    s.G, s.N, s.C, s.K = (int(p[k]) for k in ("G", "N", "C", "K"))
    for name in ("in_len", "filt_len", "stride", "dilation", "pad_lo", "pad_hi"):
        v = tuple(p[name])[:nd]
        arr = getattr(s, name)
        for i in range(3):
            arr[i] = int(v[i]) if i < len(v) else 0
    return s


# ---------------------------------------------------------------- ABI-named wrappers


def wgrad_plan(problem: dict, split_k: int = 0, group_merge: int = 0, variant: int = 0,
               tile: int = 0, hip_device: int | None = None) -> "Plan":
    """Create a plan. hip_device None = torch's current device; -1 = host-only
    (sized for an MI355X, no HIP calls)."""
    return Plan(problem, split_k, group_merge, variant, tile, hip_device)


def wgrad_workspace_bytes(plan: "Plan") -> int:
    return int(load_library().wgrad_workspace_bytes(plan.handle))


def wgrad_plan_query(plan: "Plan") -> dict:
    info = wgrad_plan_info()
    _check(load_library().wgrad_plan_query(plan.handle, ctypes.byref(info)))
    d = {name: getattr(info, name) for name, _ in wgrad_plan_info._fields_ if name != "reserved"}
    d["out_len"] = tuple(info.out_len)
    return d


def wgrad_plan_describe(plan: "Plan") -> str:
    return load_library().wgrad_plan_describe(plan.handle).decode()


def wgrad_plan_destroy(plan: "Plan") -> None:
    plan.close()


def wgrad_last_error() -> str:
    return load_library().wgrad_last_error().decode()


def wgrad_version() -> str:
    return load_library().wgrad_version().decode()


def wgrad_run(plan: "Plan", x, dy, dw, ws=None, stream=None) -> None:
    """Enqueue dW = wgrad(X, dY) on the stream (torch tensors on the GPU)."""
    plan.run(x, dy, dw, ws, stream)


def wgrad_run_stage(plan: "Plan", stage: int, x, dy, dw, ws=None, stream=None) -> None:
    """Enqueue one of wgrad_run's two launches (1 = main kernel, 2 = reduce)."""
    plan.run(x, dy, dw, ws, stream, stage=stage)


def wgrad_run_noalloc(plan: "Plan", x, dy, dw, stream=None) -> None:
    """wgrad_run with the library's per-GPU scratch as the split-K workspace
    (no caller workspace, no device allocation)."""
    plan.run_noalloc(x, dy, dw, stream)


def wgrad_probe_transpose_read(out, stream=None) -> None:
    """Enqueue the transposed-LDS-read lane-map self-test into out, a
    contiguous int16 GPU tensor of 512 elements."""
    import torch
    if not out.is_cuda or out.dtype != torch.int16 or not out.is_contiguous() or out.numel() != 512:
        raise ValueError("out: need a contiguous int16 GPU tensor of 512 elements")
    _check(load_library().wgrad_probe_transpose_read(out.data_ptr(), Plan._stream_ptr(stream)))


def wgrad_dgrad_plan(problem: dict, variant: int = 0, tile: int = 0, split_k: int = 0, group_merge: int = 0,
                     hip_device: int | None = None) -> "DgradPlan":
    """Create a backward-data plan (same problem dict; in_dtype is dY's and
    W's type, out_dtype dX's)."""
    return DgradPlan(problem, split_k, group_merge, variant, tile, hip_device)


def wgrad_dgrad_run(plan: "DgradPlan", dy, w, dx, stream=None) -> None:
    """Enqueue dX = dgrad(dY, W) on the stream (torch tensors on the GPU)."""
    plan.run(dy, w, dx, stream)


class Plan:
    """Owns a wgrad_plan_t. Immutable; run() may be called many times."""

    _create = "wgrad_plan"

    def __init__(self, problem: dict, split_k=0, group_merge=0, variant=0, tile=0, hip_device=None):
        lib = load_library()
        self.problem = dict(problem)
        if hip_device is None:
            import torch
            hip_device = torch.cuda.current_device()
        ov = wgrad_overrides(int(split_k), int(group_merge), int(variant), int(tile))
        h = ctypes.c_void_p()
        _check(getattr(lib, self._create)(ctypes.byref(make_problem(problem)), ctypes.byref(ov), int(hip_device),
                                          ctypes.byref(h)))
        self.handle = h
        self.info = wgrad_plan_query(self)
        self.name = wgrad_plan_describe(self)
        self.workspace_bytes = wgrad_workspace_bytes(self)

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            load_library().wgrad_plan_destroy(self.handle)
            self.handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- shapes
    def x_shape(self):
        p = self.problem
        return (p["N"], *tuple(p["in_len"])[: p["ndim"]], p["C"])

    def dy_shape(self):
        p = self.problem
        ol = self.info["out_len"][: p["ndim"]]
        return (p["N"], *ol, p["K"])

    def dw_shape(self):
        p = self.problem
        return (p["K"], *tuple(p["filt_len"])[: p["ndim"]], p["C"] // p["G"])

    def _check_io(self, x, dy, dw):
        import torch
        p = self.problem
        in_t = torch.bfloat16 if p["in_dtype"] == "bf16" else torch.float16
        out_t = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[p.get("out_dtype", p["in_dtype"])]
        for name, t, shape, dt in (("x", x, self.x_shape(), in_t), ("dy", dy, self.dy_shape(), in_t),
                                   ("dw", dw, self.dw_shape(), out_t)):
            if not t.is_cuda or t.dtype != dt or not t.is_contiguous() or t.numel() != _prod(shape):
                raise ValueError(f"{name}: need a contiguous {dt} GPU tensor with {_prod(shape)} elements "
                                 f"(got {t.dtype}, {tuple(t.shape)}, cuda={t.is_cuda})")

    @staticmethod
    def _stream_ptr(stream):
        import torch
        if stream is None:
            stream = torch.cuda.current_stream()
        sp = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
        return sp or None

    def run(self, x, dy, dw, ws=None, stream=None, stage=0):
        """stage 0 = the whole path (wgrad_run); 1 or 2 = wgrad_run_stage."""
        self._check_io(x, dy, dw)
        ws_ptr, ws_n = None, 0
        if self.workspace_bytes:
            if ws is None or not ws.is_cuda or ws.numel() * ws.element_size() < self.workspace_bytes:
                raise ValueError(f"workspace of {self.workspace_bytes} bytes required")
            ws_ptr, ws_n = ws.data_ptr(), ws.numel() * ws.element_size()
        lib = load_library()
        args = (x.data_ptr() or None, dy.data_ptr() or None, dw.data_ptr(), ws_ptr, ws_n, self._stream_ptr(stream))
        if stage:
            _check(lib.wgrad_run_stage(self.handle, int(stage), *args))
        else:
            _check(lib.wgrad_run(self.handle, *args))

    def run_noalloc(self, x, dy, dw, stream=None):
        """wgrad_run_noalloc: the split-K partials go to the library's
        per-GPU scratch; plans whose workspace exceeds NOALLOC_SCRATCH_BYTES
        are rejected (WgradError, ERR_INVALID_ARG)."""
        self._check_io(x, dy, dw)
        _check(load_library().wgrad_run_noalloc(self.handle, x.data_ptr() or None, dy.data_ptr() or None,
                                                dw.data_ptr(), self._stream_ptr(stream)))

    def new_workspace(self, device=None):
        import torch
        n = max(self.workspace_bytes, 16)
        return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


class DgradPlan(Plan):
    """Owns a backward-data wgrad_plan_t (from wgrad_dgrad_plan)."""

    _create = "wgrad_dgrad_plan"

    def dx_shape(self):
        return self.x_shape()

    def w_shape(self):
        return self.dw_shape()

    def run(self, dy, w, dx, stream=None):
        import torch
        p = self.problem
        in_t = torch.bfloat16 if p["in_dtype"] == "bf16" else torch.float16
        out_t = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[p.get("out_dtype", p["in_dtype"])]
        for name, t, shape, dt in (("dy", dy, self.dy_shape(), in_t), ("w", w, self.w_shape(), in_t),
                                   ("dx", dx, self.dx_shape(), out_t)):
            if not t.is_cuda or t.dtype != dt or not t.is_contiguous() or t.numel() != _prod(shape):
                raise ValueError(f"{name}: need a contiguous {dt} GPU tensor with {_prod(shape)} elements "
                                 f"(got {t.dtype}, {tuple(t.shape)}, cuda={t.is_cuda})")
        if stream is None:
            stream = torch.cuda.current_stream()
        sp = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
        _check(load_library().wgrad_dgrad_run(self.handle, dy.data_ptr() or None, w.data_ptr() or None,
                                              dx.data_ptr() or None, sp or None))


def dgrad(problem: dict, dy, w, **overrides):
    """Convenience: plan, allocate dX with torch, run."""
    import torch
    plan = DgradPlan(problem, **overrides)
    out_t = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[problem.get("out_dtype", problem["in_dtype"])]
    dx = torch.empty(plan.dx_shape(), dtype=out_t, device=dy.device)
    plan.run(dy, w, dx)
    return dx


def _prod(shape):
    n = 1
    for s in shape:
        n *= int(s)
    return n


def wgrad(problem: dict, x, dy, **overrides):
    """Convenience: plan, allocate dW (and the workspace) with torch, run."""
    import torch
    plan = Plan(problem, **overrides)
    out_t = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[problem.get("out_dtype", problem["in_dtype"])]
    dw = torch.empty(plan.dw_shape(), dtype=out_t, device=x.device)
    ws = plan.new_workspace(x.device) if plan.workspace_bytes else None
    plan.run(x, dy, dw, ws)
    return dw
