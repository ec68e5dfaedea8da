"""Seeded synthetic inputs and the workload shapes, shared by both sides.

This module holds no part of the wgrad arithmetic: it only names the problem
shapes and draws the 16-bit input patterns that the HIP path and the CPU
oracle both consume. It imports neither of them.

Generator: a counter-based splitmix64 (Steele, Lea and Flood, "Fast
splittable pseudorandom number generators", OOPSLA 2014). Element i of a
stream with seed s is mix64(s + (i + 1) * 0x9E3779B97F4A7C15). From it:

* ``uniform``: u = (z >> 40) * 2^-24 * 2 - 1, i.e. fp32 uniform on [-1, 1),
  then round-to-nearest-even to the 16-bit input type.
* ``normal``: Box-Muller on two 53-bit uniforms from counters 2i and 2i+1,
  scaled by sigma, in fp64, then to fp32, then RNE to the input type.
* ``int``: integers in {-2, ..., 2} ((z >> 32) mod 5 - 2), exact in bf16 and
  fp16; every product and partial sum of the reduction is then an integer
  well below 2^24, so fp32 accumulation is exact in any order.
* ``ones``: every element 1.0.

The workloads are the five configurations of grouped convolution
backward-weight this repository is measured on (the 2D golden shape
n1h8c16k32r3, a split-K dense shape, a strided non-tile-aligned fp16 shape,
a grouped 2D/1D pair with C/G = K/G = 8 and a 512-group depthwise shape).
"""

from __future__ import annotations

import numpy as np

_GOLD = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def splitmix64(seed: int, count: int, start: int = 0) -> np.ndarray:
    """Elements [start, start+count) of the counter-based splitmix64 stream."""
    with np.errstate(over="ignore"):
        i = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        return _mix64(np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + i * _GOLD)


def _f32_to_bf16_bits(f: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(f, np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return rounded.astype(np.uint16)


def _f32_to_bits(f: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return _f32_to_bf16_bits(f)
    if dtype == "fp16":
        return np.asarray(f, np.float32).astype(np.float16).view(np.uint16)
    raise ValueError(dtype)


def draw(shape, dtype: str, dist: str, seed: int, sigma: float = 0.5) -> np.ndarray:
    """16-bit patterns (uint16) of the given shape, dtype and distribution."""
    n = int(np.prod(shape))
    if dist == "ones":
        one = np.ones(n, np.float32)
        return _f32_to_bits(one, dtype).reshape(shape)
    if dist == "uniform":
        z = splitmix64(seed, n)
        u = (z >> np.uint64(40)).astype(np.float32) * np.float32(2.0 ** -24)
        return _f32_to_bits(u * np.float32(2.0) - np.float32(1.0), dtype).reshape(shape)
    if dist == "normal":
        z = splitmix64(seed, 2 * n)
        u1 = ((z[0::2] >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0 ** -53   # (0, 1]
        u2 = (z[1::2] >> np.uint64(11)).astype(np.float64) * 2.0 ** -53           # [0, 1)
        v = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2) * sigma
        return _f32_to_bits(v.astype(np.float32), dtype).reshape(shape)
    if dist == "int":
        z = splitmix64(seed, n)
        v = ((z >> np.uint64(32)) % np.uint64(5)).astype(np.int64) - 2
        return _f32_to_bits(v.astype(np.float32), dtype).reshape(shape)
    raise ValueError(dist)


def _cfg(name, ndim, G, N, C, K, in_len, filt, stride, pad, dil, out_len,
         in_dtype, out_dtype, dist, seeds, note):
    return {
        "name": name, "ndim": ndim, "G": G, "N": N, "C": C, "K": K,
        "in_len": tuple(in_len), "filt_len": tuple(filt), "stride": tuple(stride),
        "dilation": tuple(dil), "pad_lo": tuple(pad), "pad_hi": tuple(pad),
        "out_len": tuple(out_len), "in_dtype": in_dtype, "out_dtype": out_dtype,
        "dist": dist, "seeds": seeds, "note": note,
    }


# Shapes are stated with totals C and K (C/G and K/G per group). out_len is
# the size the configuration states (or implies, for "same" padding); both
# sides recompute it and check it against this value.
CONFIGS = {
    "c1": _cfg("c1", 2, 1, 1, 16, 32, (8, 8), (3, 3), (1, 1), (1, 1), (1, 1), (8, 8),
               "bf16", "bf16", "uniform", (1001, 1002),
               "golden 2D shape n1h8c16k32r3: G=1 N=1 8x8 C=16 K=32 3x3 s1 p1"),
    "c2": _cfg("c2", 2, 1, 32, 64, 64, (56, 56), (3, 3), (1, 1), (1, 1), (1, 1), (56, 56),
               "bf16", "bf16", "uniform", (2001, 2002),
               "dense split-K regime: G=1 N=32 56x56 C=64 K=64 3x3 s1 p1"),
    "c3": _cfg("c3", 2, 1, 16, 128, 200, (56, 56), (3, 3), (2, 2), (1, 1), (1, 1), (28, 28),
               "fp16", "fp16", "normal", (3001, 3002),
               "strided, M not tile-aligned: G=1 N=16 56x56 C=128 K=200 3x3 s2 p1, fp16"),
    "c4a": _cfg("c4a", 2, 32, 32, 256, 256, (28, 28), (3, 3), (1, 1), (1, 1), (1, 1), (28, 28),
                "bf16", "bf16", "uniform", (4001, 4002),
                "grouped 2D: G=32 C/G=K/G=8 N=32 28x28 3x3 s1 p1"),
    "c4b": _cfg("c4b", 1, 32, 32, 256, 256, (1024,), (5,), (1,), (2,), (1,), (1024,),
                "bf16", "bf16", "uniform", (4101, 4102),
                "grouped 1D NWGC: G=32 C/G=K/G=8 N=32 W=1024 X=5 p2"),
    "c5": _cfg("c5", 2, 512, 16, 512, 512, (56, 56), (3, 3), (1, 1), (1, 1), (1, 1), (56, 56),
               "bf16", "bf16", "uniform", (5001, 5002),
               "depthwise: G=512 C/G=K/G=1 N=16 56x56 3x3 s1 p1"),
}


# Shapes for the rows beyond the five configurations (pointwise and 3D),
# measured and parity-tested the same way.
WIDER = {
    "pw": _cfg("pw", 2, 1, 32, 256, 64, (56, 56), (1, 1), (1, 1), (0, 0), (1, 1), (56, 56),
               "bf16", "bf16", "uniform", (6001, 6002),
               "pointwise: G=1 N=32 56x56 C=256 K=64 1x1 s1 p0"),
    "c3d": _cfg("c3d", 3, 1, 4, 64, 64, (16, 28, 28), (3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1),
                (16, 28, 28), "bf16", "bf16", "uniform", (7001, 7002),
                "3D dense: G=1 N=4 16x28x28 C=64 K=64 3x3x3 s1 p1"),
}


def get(name: str) -> dict:
    """A configuration by name, from CONFIGS or WIDER."""
    return CONFIGS[name] if name in CONFIGS else WIDER[name]


def problem(name_or_cfg, **changes) -> dict:
    """A copy of a configuration with some fields replaced."""
    cfg = dict(get(name_or_cfg)) if isinstance(name_or_cfg, str) else dict(name_or_cfg)
    cfg.update(changes)
    return cfg


def x_shape(cfg) -> tuple:
    return (cfg["N"], *cfg["in_len"][: cfg["ndim"]], cfg["C"])


def dy_shape(cfg) -> tuple:
    return (cfg["N"], *cfg["out_len"][: cfg["ndim"]], cfg["K"])


def inputs(cfg, dist: str | None = None, seed_offset: int = 0):
    """(x_bits, dy_bits) for a configuration. dist overrides the configured one;
    the integer mode uses seeds + 10 unless seed_offset says otherwise."""
    d = dist or cfg["dist"]
    sx, sdy = cfg["seeds"]
    off = seed_offset if (seed_offset or d != "int") else 10
    x = draw(x_shape(cfg), cfg["in_dtype"], d, sx + off)
    dy = draw(dy_shape(cfg), cfg["in_dtype"], d, sdy + off)
    return x, dy
