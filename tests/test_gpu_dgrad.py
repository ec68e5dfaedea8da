"""GPU parity of backward data (dgrad): the HIP kernel through the C ABI
(wgrad_dgrad_plan / wgrad_dgrad_run) against the CPU oracle's dgrad on the
same seeded dY and W.

Bars, as for backward weight:
* integer inputs in {-2..2}: every product and partial sum is an integer far
  below 2^24, so the fp32 accumulation is exact in any order and dX must equal
  RNE_out(oracle) bit for bit;
* random inputs: |gpu - oracle| <= tau*sum|dY*W| + 1e-6 with tau = 2^-7 (bf16
  out), 2^-10 (fp16 out), 1e-5 (fp32 out);
* dX is prefilled with NaN and a guard band after it must stay NaN (every
  element written, nothing past the end); two runs give the same bits.
Every case compares every dX element (the oracle's dgrad finishes the
largest shape here in a few seconds).
"""

import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
gcb = pytest.importorskip("grouped_convolution_backward_amd")

pytestmark = pytest.mark.gpu

OUT_T = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}
GUARD = 4096


def to_dev(bits, dtype):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).reshape(-1).copy())
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).cuda()


def draw(cfg, dist, seeds=None):
    s0, s1 = seeds or cfg.get("seeds", (11, 12))
    dys = (cfg["N"], *oracle.out_len(cfg), cfg["K"])
    return (workloads.draw(dys, cfg["in_dtype"], dist, s0 + 100),
            workloads.draw(oracle.dw_shape(cfg), cfg["in_dtype"], dist, s1 + 100))


def run_dgrad(cfg, dyb, wb, **ov):
    p = gcb.DgradPlan(cfg, **ov)
    out_dtype = cfg.get("out_dtype", cfg["in_dtype"])
    dy = to_dev(dyb, cfg["in_dtype"])
    w = to_dev(wb, cfg["in_dtype"])
    n = int(np.prod(p.dx_shape()))
    buf = torch.full((n + GUARD,), float("nan"), dtype=OUT_T[out_dtype], device="cuda")
    dx = buf[:n]
    print(f"[gpu] dgrad {cfg.get('name', '?')} {p.name}", flush=True)
    p.run(dy, w, dx)
    torch.cuda.synchronize()
    assert np.all(np.isnan(buf[n:].float().cpu().numpy())), "kernel wrote past the end of dX"
    if out_dtype == "fp32":
        bits = dx.cpu().numpy().view(np.uint32)
        vals = bits.view(np.float32).astype(np.float64)
    else:
        bits = dx.view(torch.int16).cpu().numpy().view(np.uint16)
        vals = oracle.widen(bits, out_dtype)
    return vals, bits, p


def check_exact(cfg, bits, dx64):
    out_dtype = cfg.get("out_dtype", cfg["in_dtype"])
    want = dx64.reshape(-1).astype(np.float32).view(np.uint32) if out_dtype == "fp32" \
        else oracle.round_to_bits(dx64.reshape(-1), out_dtype)
    bad = np.nonzero(bits.reshape(-1) != want)[0]
    assert bad.size == 0, f"{bad.size} of {want.size} elements differ, first at {bad[:5]}"


def check_tol(cfg, vals, dx64, ab64):
    out_dtype = cfg.get("out_dtype", cfg["in_dtype"])
    v, d, a = vals.reshape(-1), dx64.reshape(-1), ab64.reshape(-1)
    assert not np.any(np.isnan(v)), "dX has unwritten (NaN) elements"
    bad = np.nonzero(oracle.violations(v, d, a, out_dtype))[0]
    assert bad.size == 0, (f"{bad.size} elements outside tau*sum|dY*W|+1e-6, e.g. gpu={v[bad[:3]]} "
                           f"ref={d[bad[:3]]}")


ALL = {**workloads.CONFIGS, **workloads.WIDER}


@pytest.mark.parametrize("name", list(ALL))
def test_dgrad_configs_exact_integer(name):
    cfg = ALL[name]
    dyb, wb = draw(cfg, "int")
    _, bits, _ = run_dgrad(cfg, dyb, wb)
    dx64, _ = oracle.dgrad(cfg, dyb, wb)
    check_exact(cfg, bits, dx64)


@pytest.mark.parametrize("name", list(ALL))
def test_dgrad_configs_random_within_tolerance(name):
    cfg = ALL[name]
    dyb, wb = draw(cfg, cfg["dist"])
    vals, bits, _ = run_dgrad(cfg, dyb, wb)
    dx64, ab64 = oracle.dgrad(cfg, dyb, wb)
    check_tol(cfg, vals, dx64, ab64)
    # same plan, same inputs: same bits
    _, bits2, _ = run_dgrad(cfg, dyb, wb)
    assert np.array_equal(bits, bits2)


def prob(ndim, G, N, cpg, kpg, in_len, filt, stride, pad_lo, pad_hi, dil, dtype="bf16", out=None, name="edge"):
    return {"name": name, "ndim": ndim, "G": G, "N": N, "C": G * cpg, "K": G * kpg, "in_len": tuple(in_len),
            "filt_len": tuple(filt), "stride": tuple(stride), "dilation": tuple(dil),
            "pad_lo": tuple(pad_lo), "pad_hi": tuple(pad_hi), "in_dtype": dtype, "out_dtype": out or dtype}


# (ndim, G, N, C/G, K/G, in_len, filt, stride, pad_lo, pad_hi, dil, dtype, out)
EDGE = [
    # ragged M (positions not a multiple of 128), K/G not a multiple of 32, C/G = 40
    (2, 1, 3, 40, 72, (13, 11), (3, 3), (1, 1), (1, 1), (1, 1), (1, 1), "bf16", None),
    # strided and dilated, asymmetric pads, fp16 in, fp32 out
    (2, 2, 2, 24, 48, (17, 15), (3, 5), (2, 3), (2, 1), (0, 2), (2, 1), "fp16", "fp32"),
    # odd channel runs: 2-element then 1-element loads
    (2, 3, 2, 6, 10, (9, 8), (3, 3), (1, 2), (1, 1), (1, 0), (1, 1), "bf16", None),
    (2, 2, 1, 3, 5, (7, 9), (2, 3), (1, 1), (0, 1), (1, 1), (1, 2), "bf16", "fp32"),
    # wide channel runs: two 128-wide tiles along C/G
    (2, 1, 2, 200, 64, (10, 12), (3, 3), (1, 1), (1, 1), (1, 1), (1, 1), "bf16", None),
    # grouped, C/G = K/G = 8; depthwise C/G = K/G = 1
    (2, 16, 4, 8, 8, (14, 14), (3, 3), (1, 1), (1, 1), (1, 1), (1, 1), "bf16", None),
    (2, 64, 2, 1, 1, (12, 12), (3, 3), (1, 1), (1, 1), (1, 1), (1, 1), "bf16", None),
    # 1x1 with stride 2: three quarters of dX receive no tap and must be 0
    (2, 1, 2, 64, 32, (12, 10), (1, 1), (2, 2), (0, 0), (0, 0), (1, 1), "bf16", None),
    # kernel larger than the stride gaps, pads larger than the dilated filter reach
    (2, 1, 1, 32, 32, (6, 7), (5, 5), (3, 2), (4, 3), (4, 3), (1, 1), "fp16", None),
    # 1D and 3D
    (1, 4, 3, 16, 24, (37,), (5,), (2,), (2,), (1,), (1,), "bf16", None),
    (3, 2, 2, 16, 32, (5, 6, 7), (3, 3, 3), (1, 2, 1), (1, 1, 1), (1, 0, 1), (1, 1, 2), "bf16", None),
    (3, 1, 1, 8, 8, (3, 4, 5), (2, 1, 3), (2, 1, 1), (0, 0, 1), (1, 0, 1), (1, 1, 1), "fp16", "fp32"),
    # stride and dilation sharing a factor: valid taps every other tap (s 4,
    # d 2) or every tap with unit output steps (s 3, d 3)
    (2, 1, 2, 16, 24, (17, 13), (5, 3), (4, 3), (3, 2), (2, 0), (2, 3), "bf16", None),
    (1, 2, 2, 8, 40, (29,), (4,), (3,), (5,), (4,), (3,), "fp16", None),
]


@pytest.mark.parametrize("i", range(len(EDGE)))
def test_dgrad_edge_shapes(i):
    cfg = prob(*EDGE[i], name=f"edge{i}")
    dyb, wb = draw(cfg, "int", (300 + i, 400 + i))
    _, bits, _ = run_dgrad(cfg, dyb, wb)
    dx64, _ = oracle.dgrad(cfg, dyb, wb)
    check_exact(cfg, bits, dx64)
    dyb, wb = draw(cfg, "uniform", (500 + i, 600 + i))
    vals, _, _ = run_dgrad(cfg, dyb, wb)
    dx64, ab64 = oracle.dgrad(cfg, dyb, wb)
    check_tol(cfg, vals, dx64, ab64)


# Stride phases with grids large enough that the kernel rotates the phase
# order within groups of tiles (2D stride 2 and 3, mixed strides, 3D stride
# 2: 4, 9, 6 and 8 phases). A rotation that were not a permutation would
# leave some phase of some tile unwritten (NaN) and write another twice.
PHASED = [
    (2, 1, 2, 64, 64, (64, 64), (3, 3), (2, 2), (1, 1), (1, 1), (1, 1), "bf16", None),
    (2, 1, 2, 32, 32, (72, 72), (3, 3), (3, 3), (1, 1), (1, 1), (1, 1), "fp16", None),
    (2, 1, 2, 32, 32, (48, 72), (3, 3), (2, 3), (1, 1), (1, 1), (1, 1), "bf16", "fp32"),
    (3, 1, 2, 32, 32, (8, 32, 32), (3, 3, 3), (2, 2, 2), (1, 1, 1), (1, 1, 1), (1, 1, 1), "bf16", None),
    # grouped: four groups, and eight merged two at a time with one-sided pads
    (2, 4, 2, 32, 32, (48, 48), (3, 3), (2, 2), (1, 1), (1, 1), (1, 1), "bf16", None),
    (2, 8, 1, 16, 24, (40, 40), (3, 3), (2, 2), (1, 1), (0, 0), (1, 1), "fp16", "fp32"),
]


@pytest.mark.parametrize("i", range(len(PHASED)))
def test_dgrad_stride_phase_rotation(i):
    cfg = prob(*PHASED[i], name=f"phased{i}")
    dyb, wb = draw(cfg, "int", (700 + i, 800 + i))
    _, bits, p = run_dgrad(cfg, dyb, wb)
    assert p.name.startswith("dgrad_mfma_"), p.name
    phases = int(np.prod(cfg["stride"]))
    # more tile groups than one XCD's CUs take per phase: the order rotates
    assert p.info["grid_main"] // phases > max(1, 32 // phases), p.info["grid_main"]
    dx64, _ = oracle.dgrad(cfg, dyb, wb)
    check_exact(cfg, bits, dx64)


@pytest.mark.parametrize("tile", [1, 2, 3])
def test_dgrad_every_tile(tile):
    cfg = prob(2, 2, 2, 72, 40, (11, 13), (3, 3), (1, 1), (1, 1), (1, 1), (1, 1), name=f"tile{tile}")
    dyb, wb = draw(cfg, "int", (71, 72))
    _, bits, p = run_dgrad(cfg, dyb, wb, tile=tile)
    assert p.info["tile"] == tile
    dx64, _ = oracle.dgrad(cfg, dyb, wb)
    check_exact(cfg, bits, dx64)


# depthwise direct kernel (C/G = K/G = 1); the 3x3 unit-stride shapes take
# the row-walking form (ragged widths, one-row images, chunks of one row)
DW = [
    (2, 64, 3, 1, 1, (9, 10), (3, 3), (1, 1), (1, 1), (1, 1), (1, 1), "bf16", None),
    (2, 128, 1, 1, 1, (1, 7), (3, 3), (1, 1), (1, 1), (1, 1), (1, 1), "fp16", "fp32"),
    (2, 32, 2, 1, 1, (6, 5), (3, 3), (1, 1), (0, 2), (2, 0), (1, 1), "bf16", None),
    (2, 24, 1, 1, 1, (40, 3), (3, 3), (1, 1), (1, 1), (1, 1), (1, 1), "bf16", None),
    (2, 512, 2, 1, 1, (13, 11), (3, 3), (1, 1), (1, 1), (1, 1), (1, 1), "bf16", None),
    (2, 24, 2, 1, 1, (9, 10), (5, 5), (2, 2), (2, 1), (1, 2), (1, 1), "fp16", "fp32"),
    (2, 64, 1, 1, 1, (10, 9), (3, 3), (1, 1), (2, 2), (2, 2), (2, 2), "bf16", None),
    (1, 40, 3, 1, 1, (50,), (7,), (3,), (3,), (3,), (1,), "bf16", None),
    (3, 32, 1, 1, 1, (5, 6, 7), (3, 3, 3), (2, 1, 1), (1, 1, 1), (1, 1, 1), (1, 1, 1), "fp16", None),
    (2, 16, 1, 1, 1, (3, 3), (1, 1), (2, 2), (0, 0), (0, 0), (1, 1), "bf16", None),
    (2, 1024, 1, 1, 1, (6, 5), (3, 3), (1, 1), (1, 1), (1, 1), (1, 1), "bf16", "fp32"),
]


@pytest.mark.parametrize("i", range(len(DW)))
def test_dgrad_depthwise_kernel(i):
    cfg = prob(*DW[i], name=f"dw{i}")
    dyb, wb = draw(cfg, "int", (700 + i, 800 + i))
    _, bits, p = run_dgrad(cfg, dyb, wb)
    assert p.info["tile"] in (4, 5, 7) and p.name.startswith("dgrad_dw")
    # both depthwise forms (row walk where it applies) agree bitwise
    _, bits5, p5 = run_dgrad(cfg, dyb, wb, tile=5)
    assert p5.info["tile"] == 5 and np.array_equal(bits, bits5)
    dx64, _ = oracle.dgrad(cfg, dyb, wb)
    check_exact(cfg, bits, dx64)
    # the MFMA kernel on the same shape gives the same (exact) bits
    _, bits_mfma, p1 = run_dgrad(cfg, dyb, wb, tile=1)
    assert p1.info["tile"] == 1 and np.array_equal(bits, bits_mfma)
    dyb, wb = draw(cfg, "uniform", (900 + i, 1000 + i))
    vals, _, _ = run_dgrad(cfg, dyb, wb)
    dx64, ab64 = oracle.dgrad(cfg, dyb, wb)
    check_tol(cfg, vals, dx64, ab64)


# depthwise tile kernel (2D 3x3, unit stride and dilation, C a multiple of
# 256): ragged tiles both ways, images smaller than a tile, pads 0 to 2,
# several channel blocks, fp16 and fp32 outputs, and more tiles than
# workgroups (a workgroup walks several, taller tiles)
DW_TILE = [
    (2, 256, 2, 1, 1, (17, 30), (3, 3), (1, 1), (1, 1), (1, 1), (1, 1), "bf16", None),
    (2, 512, 1, 1, 1, (9, 31), (3, 3), (1, 1), (0, 2), (2, 0), (1, 1), "fp16", "fp32"),
    (2, 768, 3, 1, 1, (1, 1), (3, 3), (1, 1), (1, 1), (1, 1), (1, 1), "bf16", None),
    (2, 256, 1, 1, 1, (40, 3), (3, 3), (1, 1), (2, 2), (2, 2), (1, 1), "fp16", None),
    (2, 256, 2, 1, 1, (6, 60), (3, 3), (1, 1), (0, 0), (0, 0), (1, 1), "bf16", None),
    (2, 256, 256, 1, 1, (8, 8), (3, 3), (1, 1), (1, 1), (1, 1), (1, 1), "bf16", None),
]


@pytest.mark.parametrize("i", range(len(DW_TILE)))
def test_dgrad_depthwise_tile(i):
    cfg = prob(*DW_TILE[i], name=f"dwt{i}")
    dyb, wb = draw(cfg, "int", (1700 + i, 1800 + i))
    _, bits, p = run_dgrad(cfg, dyb, wb)
    assert p.info["tile"] == 7 and p.name.startswith("dgrad_dwtile")
    dx64, _ = oracle.dgrad(cfg, dyb, wb)
    check_exact(cfg, bits, dx64)
    # the row-walking form gives the same (exact) bits
    _, bits4, p4 = run_dgrad(cfg, dyb, wb, tile=4)
    assert p4.info["tile"] == 4 and np.array_equal(bits, bits4)
    dyb, wb = draw(cfg, "uniform", (1900 + i, 2000 + i))
    vals, _, _ = run_dgrad(cfg, dyb, wb)
    dx64, ab64 = oracle.dgrad(cfg, dyb, wb)
    check_tol(cfg, vals, dx64, ab64)


@pytest.mark.parametrize("gm", [1, 2, 4, 8])
def test_dgrad_group_merge(gm):
    # C/G = 8, K/G = 12 (merged rows and columns of different widths), and a
    # ragged tail of positions; every merge degree gives the exact sums
    cfg = prob(2, 8, 2, 8, 12, (9, 11), (3, 3), (1, 2), (1, 1), (1, 1), (1, 1), name=f"gm{gm}")
    dyb, wb = draw(cfg, "int", (81, 82))
    _, bits, p = run_dgrad(cfg, dyb, wb, group_merge=gm)
    assert p.info["group_merge"] == gm
    dx64, _ = oracle.dgrad(cfg, dyb, wb)
    check_exact(cfg, bits, dx64)
    # depthwise through the merged MFMA kernel
    cfg = prob(2, 16, 1, 1, 1, (7, 6), (3, 3), (1, 1), (1, 1), (1, 1), (1, 1), name=f"dwgm{gm}")
    dyb, wb = draw(cfg, "uniform", (83, 84))
    vals, _, p = run_dgrad(cfg, dyb, wb, group_merge=gm, tile=1)
    dx64, ab64 = oracle.dgrad(cfg, dyb, wb)
    check_tol(cfg, vals, dx64, ab64)


def test_dgrad_empty_batch():
    cfg = prob(2, 1, 0, 16, 16, (8, 8), (3, 3), (1, 1), (1, 1), (1, 1), (1, 1))
    p = gcb.DgradPlan(cfg)
    assert p.info["grid_main"] == 0
    e = torch.empty(0, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(p.w_shape(), dtype=torch.bfloat16, device="cuda")
    p.run(e, w, e)
    torch.cuda.synchronize()


# row-ring form (tile 6): images crossing step boundaries, one-row and
# narrow images, every pad the form takes, 32- and 64-channel dY runs, one
# to three dX channel blocks, merged groups, fp16 in and fp32 out
RING = [
    (2, 1, 3, 64, 64, (13, 56), (3, 3), (1, 1), (1, 1), (1, 1), (1, 1), "bf16", None),
    (2, 1, 2, 96, 32, (9, 30), (3, 3), (1, 1), (1, 1), (1, 1), (1, 1), "bf16", None),
    (2, 16, 3, 8, 8, (7, 28), (3, 3), (1, 1), (1, 1), (1, 1), (1, 1), "bf16", None),
    (2, 4, 2, 16, 16, (6, 40), (3, 3), (1, 1), (0, 2), (2, 0), (1, 1), "bf16", None),
    (2, 1, 2, 64, 32, (5, 17), (3, 3), (1, 1), (2, 0), (0, 2), (1, 1), "bf16", None),
    (2, 1, 2, 32, 64, (4, 64), (3, 3), (1, 1), (1, 1), (1, 1), (1, 1), "fp16", "fp32"),
    (2, 1, 5, 32, 64, (1, 20), (3, 3), (1, 1), (1, 1), (1, 1), (1, 1), "bf16", None),
    (2, 2, 3, 64, 32, (9, 3), (3, 3), (1, 1), (0, 0), (0, 0), (1, 1), "fp16", None),
]


@pytest.mark.parametrize("i", range(len(RING)))
def test_dgrad_ring_form(i):
    cfg = prob(*RING[i], name=f"ring{i}")
    dyb, wb = draw(cfg, "int", (1100 + i, 1200 + i))
    _, bits, p = run_dgrad(cfg, dyb, wb, tile=6)
    assert p.info["tile"] == 6 and p.name.startswith("dgrad_ring_"), p.name
    dx64, _ = oracle.dgrad(cfg, dyb, wb)
    check_exact(cfg, bits, dx64)
    # the flat MFMA kernel gives the same (exact) bits
    _, bits1, _ = run_dgrad(cfg, dyb, wb, tile=1)
    assert np.array_equal(bits, bits1)
    dyb, wb = draw(cfg, "uniform", (1300 + i, 1400 + i))
    vals, bits, _ = run_dgrad(cfg, dyb, wb, tile=6)
    dx64, ab64 = oracle.dgrad(cfg, dyb, wb)
    check_tol(cfg, vals, dx64, ab64)
    _, bits2, _ = run_dgrad(cfg, dyb, wb, tile=6)
    assert np.array_equal(bits, bits2)
