"""CPU oracle for grouped 1D/2D convolution backward-weight (wgrad).

TEST INFRASTRUCTURE. Only tests/, ``__graft_entry__.smoke()`` and bench.py's
``cpu_baseline`` leg may import this package. It shares no code with the HIP
path in ``grouped_convolution_backward_amd`` and imports nothing from it.

The sums themselves run in ``wgrad_oracle.c`` (fp64, direct loop, one fixed
summation order per element); this module builds and loads that library and
adds the pieces of the acceptance test that sit on the oracle side:

* ``wgrad`` / ``wgrad_sampled``: dW and sum|dY*X| in fp64 (GK[Z]YXC order).
* ``dgrad``: the backward-data sums dX and sum|dY*W| in fp64 (N[D]HWGC order).
* ``round_to``: fp64 -> bf16/fp16 round-to-nearest-even, done directly from
  fp64 (no intermediate fp32, so no double rounding).
* ``bound``: the elementwise acceptance bound tau*sum|dY*X| + 1e-6 with
  tau = 2^-7 (bf16 out), 2^-10 (fp16 out), 1e-5 (fp32 out).

The operation is the one the Composable Kernel page
"grouped_convolution_backward_weight_kernel.hpp" describes through its
NWGC/GKXC/NWGK and NHWGC/GKYXC/NHWGK argument constructors and the per-group
offsets used in ``operator()``; the formula is restated in wgrad_oracle.c.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "wgrad_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DTYPE_CODE = {"bf16": 0, "fp16": 1}
TAU = {"bf16": 2.0 ** -7, "fp16": 2.0 ** -10, "fp32": 1e-5}
ABS_FLOOR = 1e-6


class _Problem(ctypes.Structure):
    _fields_ = [
        ("ndim", ctypes.c_int64),
        ("G", ctypes.c_int64), ("N", ctypes.c_int64),
        ("C", ctypes.c_int64), ("K", ctypes.c_int64),
        ("in_len", ctypes.c_int64 * 3), ("filt_len", ctypes.c_int64 * 3),
        ("stride", ctypes.c_int64 * 3), ("dilation", ctypes.c_int64 * 3),
        ("pad_lo", ctypes.c_int64 * 3), ("pad_hi", ctypes.c_int64 * 3),
        ("in_dtype", ctypes.c_int64),
    ]


def build(force: bool = True) -> str:
    """Compile wgrad_oracle.c with gcc (OpenMP) into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                        _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.POINTER(_Problem)
        u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
        f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
        i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
        lib.oracle_wgrad.argtypes = [P, u16p, u16p, f64p, f64p, ctypes.c_int]
        lib.oracle_wgrad.restype = ctypes.c_int
        lib.oracle_wgrad_sampled.argtypes = [P, u16p, u16p, ctypes.c_int64, i64p,
                                             f64p, f64p, ctypes.c_int]
        lib.oracle_wgrad_sampled.restype = ctypes.c_int
        lib.oracle_out_len.argtypes = [P, ctypes.POINTER(ctypes.c_int64),
                                       ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]
        lib.oracle_out_len.restype = ctypes.c_int
        lib.oracle_dgrad.argtypes = [P, u16p, u16p, f64p, f64p, ctypes.c_int]
        lib.oracle_dgrad.restype = ctypes.c_int
        lib.oracle_widen.argtypes = [u16p, ctypes.c_int64, ctypes.c_int64, f64p]
        lib.oracle_widen.restype = ctypes.c_int
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_last_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _to_struct(prob: dict) -> _Problem:
    nd = int(prob["ndim"])
    p = _Problem()
    p.ndim = nd
    p.G, p.N, p.C, p.K = (int(prob[k]) for k in ("G", "N", "C", "K"))
    for name in ("in_len", "filt_len", "stride", "dilation", "pad_lo", "pad_hi"):
        v = tuple(prob[name])[:nd]
        arr = getattr(p, name)
        for i in range(3):
            arr[i] = int(v[i]) if i < len(v) else 0
    p.in_dtype = DTYPE_CODE[prob["in_dtype"]]
    return p


def out_len(prob: dict) -> tuple:
    """Output spatial lengths, outermost first: (Do, Ho, Wo) for 3D, (Ho, Wo)
    for 2D, (Wo,) for 1D."""
    od, oh, ow = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    if _load().oracle_out_len(ctypes.byref(_to_struct(prob)), ctypes.byref(od), ctypes.byref(oh),
                              ctypes.byref(ow)):
        raise ValueError("invalid problem")
    return (od.value, oh.value, ow.value)[3 - int(prob["ndim"]):]


def dw_shape(prob: dict) -> tuple:
    """GK[Z]YXC shape as (K_total, *filter, C/G)."""
    return (int(prob["K"]), *tuple(prob["filt_len"])[: int(prob["ndim"])],
            int(prob["C"]) // int(prob["G"]))


def _check_sizes(prob, x_bits, dy_bits):
    nd = int(prob["ndim"])
    sp_in = int(np.prod(tuple(prob["in_len"])[:nd]))
    sp_out = int(np.prod(out_len(prob)))
    if x_bits.size != int(prob["N"]) * sp_in * int(prob["C"]):
        raise ValueError("x has the wrong number of elements")
    if dy_bits.size != int(prob["N"]) * sp_out * int(prob["K"]):
        raise ValueError("dy has the wrong number of elements")


def wgrad(prob: dict, x_bits: np.ndarray, dy_bits: np.ndarray, nthreads: int = 0):
    """Full dW and sum|dY*X| in fp64, each shaped (K, [Z,] [Y,] X, C/G)."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16).reshape(-1)
    dy_bits = np.ascontiguousarray(dy_bits, dtype=np.uint16).reshape(-1)
    _check_sizes(prob, x_bits, dy_bits)
    shape = dw_shape(prob)
    dw = np.zeros(int(np.prod(shape)), np.float64)
    ab = np.zeros_like(dw)
    if _load().oracle_wgrad(ctypes.byref(_to_struct(prob)), x_bits, dy_bits, dw, ab, nthreads):
        raise ValueError("oracle rejected the problem")
    return dw.reshape(shape), ab.reshape(shape)


def wgrad_sampled(prob: dict, x_bits: np.ndarray, dy_bits: np.ndarray,
                  flat_idx: np.ndarray, nthreads: int = 0):
    """dW and sum|dY*X| at the given flat GK[Z]YXC indices only."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16).reshape(-1)
    dy_bits = np.ascontiguousarray(dy_bits, dtype=np.uint16).reshape(-1)
    _check_sizes(prob, x_bits, dy_bits)
    idx = np.ascontiguousarray(flat_idx, dtype=np.int64).reshape(-1)
    dw = np.zeros(idx.size, np.float64)
    ab = np.zeros_like(dw)
    if _load().oracle_wgrad_sampled(ctypes.byref(_to_struct(prob)), x_bits, dy_bits,
                                    idx.size, idx, dw, ab, nthreads):
        raise ValueError("oracle rejected the problem or an index")
    return dw, ab


def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """16-bit patterns (bf16 or fp16) to fp64, exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).reshape(-1)
    out = np.zeros(b.size, np.float64)
    _load().oracle_widen(b, b.size, DTYPE_CODE[dtype], out)
    return out.reshape(np.shape(bits))


def max_threads() -> int:
    """Threads a call with nthreads=0 uses (OpenMP's default team size)."""
    return int(_load().oracle_max_threads())


def last_threads() -> int:
    """Threads the last wgrad / wgrad_sampled / dgrad loop actually ran on."""
    return int(_load().oracle_last_threads())


# --- fp64 -> 16-bit rounding (round to nearest, ties to even) -------------

# (significand bits incl. the implicit one, min normal exponent, max finite)
_FMT = {
    "bf16": (8, -126, (2.0 - 2.0 ** -7) * 2.0 ** 127),
    "fp16": (11, -14, 65504.0),
}


def _quantize(v: np.ndarray, fmt: str) -> np.ndarray:
    """Nearest representable value (ties to even) of an fp64 array, in fp64."""
    p, emin, vmax = _FMT[fmt]
    v = np.asarray(v, np.float64)
    out = np.empty_like(v)
    finite = np.isfinite(v)
    out[~finite] = v[~finite]
    a = np.abs(v[finite])
    # exponent of the leading bit; values below the normal range share the
    # subnormal quantum 2^(emin - p + 1)
    _, e = np.frexp(a)                    # a = m * 2^e, m in [0.5, 1)
    lead = np.maximum(e - 1, emin)
    quantum_exp = lead - (p - 1)
    q = np.ldexp(np.rint(np.ldexp(a, -quantum_exp)), quantum_exp)   # rint: ties to even
    # values at or past max + half an ulp round to infinity
    ulp_top = 2.0 ** (np.floor(np.log2(vmax)) - (p - 1))
    q = np.where(a >= vmax + ulp_top / 2, np.inf, q)
    out[finite] = np.copysign(q, v[finite])
    return out


def round_to(v: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 -> out dtype by RNE, returned widened back to fp64 (fp32 out: RNE to binary32)."""
    if dtype == "fp32":
        return np.asarray(v, np.float64).astype(np.float32).astype(np.float64)
    return _quantize(v, dtype)


def round_to_bits(v: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 -> 16-bit patterns of the out dtype, by RNE."""
    q = _quantize(v, dtype)
    if dtype == "fp16":
        return q.astype(np.float16).view(np.uint16)          # exact: q is representable
    return (q.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def bound(absdw: np.ndarray, out_dtype: str) -> np.ndarray:
    """Elementwise acceptance bound tau*sum|dY*X| + 1e-6."""
    return TAU[out_dtype] * np.asarray(absdw, np.float64) + ABS_FLOOR


def violations(gpu64: np.ndarray, dw64: np.ndarray, absdw: np.ndarray, out_dtype: str):
    """Boolean mask of elements outside the bound (NaN counts as outside)."""
    err = np.abs(np.asarray(gpu64, np.float64) - dw64)
    return ~(err <= bound(absdw, out_dtype))


def dgrad(prob: dict, dy_bits: np.ndarray, w_bits: np.ndarray, nthreads: int = 0):
    """Backward data: dX and sum|dY*W| in fp64, each shaped (N, *in_len, C)
    (NDHWGC order). w_bits is the GK[Z]YXC weight, dy_bits the NDHWGK output
    gradient."""
    nd = int(prob["ndim"])
    dy_bits = np.ascontiguousarray(dy_bits, dtype=np.uint16).reshape(-1)
    w_bits = np.ascontiguousarray(w_bits, dtype=np.uint16).reshape(-1)
    if dy_bits.size != int(prob["N"]) * int(np.prod(out_len(prob))) * int(prob["K"]):
        raise ValueError("dy has the wrong number of elements")
    if w_bits.size != int(np.prod(dw_shape(prob))):
        raise ValueError("w has the wrong number of elements")
    shape = (int(prob["N"]), *tuple(prob["in_len"])[:nd], int(prob["C"]))
    dx = np.zeros(int(np.prod(shape)), np.float64)
    ab = np.zeros_like(dx)
    if _load().oracle_dgrad(ctypes.byref(_to_struct(prob)), dy_bits, w_bits, dx, ab, nthreads):
        raise ValueError("oracle rejected the problem")
    return dx.reshape(shape), ab.reshape(shape)
