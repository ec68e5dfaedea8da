"""Pins for the CPU oracle: each test checks it against something other than
itself (a closed form, an invariant computed a different way, a library
routine, exact integer arithmetic, or a finite difference of the forward
convolution), chosen so that a dropped term, a wrong sign or index, a
transposed operand or a pad/stride/dilation slip fails at least one.

The operation is grouped convolution backward-weight over NHWGC input,
NHWGK output-gradient and GKYXC weight layouts (Composable Kernel page
"grouped_convolution_backward_weight_kernel.hpp", the 1D and 2D argument
constructors and the per-group offsets in operator()).
"""

import itertools
import os

import numpy as np
import pytest

import oracle
import workloads

# ---------------------------------------------------------------- helpers


def small_problem(ndim, G, N, cpg, kpg, in_len, filt, stride, pad_lo, pad_hi, dil, dtype="bf16"):
    return {
        "ndim": ndim, "G": G, "N": N, "C": G * cpg, "K": G * kpg,
        "in_len": tuple(in_len), "filt_len": tuple(filt), "stride": tuple(stride),
        "dilation": tuple(dil), "pad_lo": tuple(pad_lo), "pad_hi": tuple(pad_hi),
        "in_dtype": dtype, "out_dtype": dtype,
    }


def draw_for(prob, dist, seed):
    ol = oracle.out_len(prob)
    nd = prob["ndim"]
    xs = (prob["N"], *prob["in_len"][:nd], prob["C"])
    ys = (prob["N"], *ol, prob["K"])
    return (workloads.draw(xs, prob["in_dtype"], dist, seed),
            workloads.draw(ys, prob["in_dtype"], dist, seed + 1))


def as_2d(prob, xv, dyv):
    """View 1D problems as 2D with a unit h axis: returns (x, dy, geometry)."""
    nd = prob["ndim"]
    ol = oracle.out_len(prob)
    if nd == 1:
        x = None if xv is None else xv.reshape(prob["N"], 1, prob["in_len"][0], prob["C"])
        dy = None if dyv is None else dyv.reshape(prob["N"], 1, ol[0], prob["K"])
        geo = dict(Hi=1, Wi=prob["in_len"][0], Y=1, X=prob["filt_len"][0], sh=1,
                   sw=prob["stride"][0], dh=1, dw=prob["dilation"][0], ph=0,
                   pw=prob["pad_lo"][0], Ho=1, Wo=ol[0])
    else:
        x = None if xv is None else xv.reshape(prob["N"], *prob["in_len"], prob["C"])
        dy = None if dyv is None else dyv.reshape(prob["N"], *ol, prob["K"])
        geo = dict(Hi=prob["in_len"][0], Wi=prob["in_len"][1], Y=prob["filt_len"][0],
                   X=prob["filt_len"][1], sh=prob["stride"][0], sw=prob["stride"][1],
                   dh=prob["dilation"][0], dw=prob["dilation"][1], ph=prob["pad_lo"][0],
                   pw=prob["pad_lo"][1], Ho=ol[0], Wo=ol[1])
    return x, dy, geo


def valid_range(o_len, i_len, s, p, d, t):
    """Closed form: the output positions o in [lo, hi] with 0 <= o*s - p + t*d < i_len."""
    a = p - t * d                               # need o*s >= a
    lo = max(0, -((-a) // s))                   # ceil(a / s), at least 0
    hi = min(o_len - 1, (i_len - 1 + p - t * d) // s)
    return lo, hi


def count_closed_form(o_len, i_len, s, p, d, t):
    lo, hi = valid_range(o_len, i_len, s, p, d, t)
    return max(0, hi - lo + 1)


def per_tap_matmul(prob, xv, dyv, dtype=np.float64):
    """dW via one matmul per filter tap over the valid (strided) window.
    A different decomposition from the oracle's element-by-element loop."""
    x, dy, geo = as_2d(prob, xv, dyv)
    G = prob["G"]
    cpg, kpg = prob["C"] // G, prob["K"] // G
    out = np.zeros((G, kpg, geo["Y"], geo["X"], cpg), dtype)
    for y, xx in itertools.product(range(geo["Y"]), range(geo["X"])):
        hlo, hhi = valid_range(geo["Ho"], geo["Hi"], geo["sh"], geo["ph"], geo["dh"], y)
        wlo, whi = valid_range(geo["Wo"], geo["Wi"], geo["sw"], geo["pw"], geo["dw"], xx)
        if hhi < hlo or whi < wlo:
            continue
        dsel = dy[:, hlo:hhi + 1, wlo:whi + 1, :]
        h0 = hlo * geo["sh"] - geo["ph"] + y * geo["dh"]
        w0 = wlo * geo["sw"] - geo["pw"] + xx * geo["dw"]
        xsel = x[:, h0:h0 + (hhi - hlo) * geo["sh"] + 1:geo["sh"],
                 w0:w0 + (whi - wlo) * geo["sw"] + 1:geo["sw"], :]
        assert xsel.shape[1:3] == dsel.shape[1:3]
        a = dsel.reshape(-1, G, kpg).astype(dtype)
        b = xsel.reshape(-1, G, cpg).astype(dtype)
        for g in range(G):
            out[g, :, y, xx, :] = a[:, g, :].T @ b[:, g, :]
    shape = oracle.dw_shape(prob)
    return out.reshape(shape)


def conv_fwd(prob, xv, w):
    """Direct fp64 forward grouped convolution (cross-correlation) with the same
    geometry: Y[n,ho,wo,g,k] = sum_{y,x,c} X[n,hi,wi,g,c] * W[g,k,y,x,c]."""
    x, _, geo = as_2d(prob, xv, None)
    G = prob["G"]
    cpg, kpg = prob["C"] // G, prob["K"] // G
    w = np.asarray(w, np.float64).reshape(G, kpg, geo["Y"], geo["X"], cpg)
    out = np.zeros((prob["N"], geo["Ho"], geo["Wo"], G, kpg))
    xg = x.reshape(prob["N"], geo["Hi"], geo["Wi"], G, cpg)
    for ho in range(geo["Ho"]):
        for wo in range(geo["Wo"]):
            for y in range(geo["Y"]):
                hi = ho * geo["sh"] - geo["ph"] + y * geo["dh"]
                if not 0 <= hi < geo["Hi"]:
                    continue
                for xx in range(geo["X"]):
                    wi = wo * geo["sw"] - geo["pw"] + xx * geo["dw"]
                    if not 0 <= wi < geo["Wi"]:
                        continue
                    # (n, g, c) x (g, k, c) -> (n, g, k)
                    out[:, ho, wo] += np.einsum("ngc,gkc->ngk", xg[:, hi, wi], w[:, :, y, xx, :])
    return out


RANDOM_SMALL = [
    # ndim, G, N, cpg, kpg, in_len, filt, stride, pad_lo, pad_hi, dil
    (2, 1, 2, 3, 4, (7, 6), (3, 3), (1, 1), (1, 1), (1, 1), (1, 1)),
    (2, 2, 1, 2, 3, (7, 7), (3, 2), (2, 1), (1, 0), (2, 1), (1, 2)),
    (2, 4, 2, 1, 1, (6, 5), (3, 3), (3, 2), (2, 0), (0, 2), (2, 1)),
    (2, 1, 1, 5, 2, (5, 7), (1, 1), (1, 1), (0, 0), (0, 0), (1, 1)),
    (2, 2, 2, 2, 2, (4, 4), (5, 5), (1, 1), (2, 2), (2, 2), (1, 1)),
    (1, 2, 2, 3, 2, (9,), (5,), (1,), (2,), (2,), (1,)),
    (1, 4, 1, 1, 1, (11,), (3,), (2,), (0,), (1,), (3,)),
    (1, 1, 2, 4, 3, (8,), (2,), (3,), (1,), (0,), (2,)),
]


def _ids(cases):
    return [f"case{i}" for i in range(len(cases))]


# ---------------------------------------------------------------- widening and rounding


def test_widen_fp16_exhaustive_matches_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.widen(bits, "fp16")
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_widen_bf16_exhaustive_matches_torch():
    torch = pytest.importorskip("torch")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.widen(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_round_bf16_matches_torch_on_fp32_values():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    v = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-40, 38, 20000),
        rng.integers(-300000, 300000, 20000).astype(np.float64),
        [0.0, -0.0, 1e-45, 3e38, 3.4e38, -3.39e38],
    ]).astype(np.float32).astype(np.float64)      # values exact in fp32: one rounding only
    ours = oracle.round_to_bits(v, "bf16")
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_round_fp16_matches_numpy():
    rng = np.random.default_rng(8)
    v = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 5, 20000),
        [65504.0, 65519.999, 65520.0, 2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0001, 0.0],
    ])
    ours = oracle.round_to_bits(v, "fp16")
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)   # numpy rounds fp64 -> fp16 directly
    assert np.array_equal(ours, ref)


def test_round_bf16_ties_and_no_double_rounding():
    # all-ones values that land on bf16 ties (2D 3x3 pad-1 shapes): ties go to even
    ties = {98560.0: 98304.0, 49280.0: 49152.0, 32704.0: 32768.0, 96800.0: 96768.0}
    for v, want in ties.items():
        assert oracle.round_to(np.array([v]), "bf16")[0] == want
    # just above a tie must round up, which a detour through fp32 would lose
    v = np.array([98560.0 + 2.0 ** -20])
    assert oracle.round_to(v, "bf16")[0] == 98816.0
    assert np.float64(np.float32(v[0])) == 98560.0


# ---------------------------------------------------------------- output size


@pytest.mark.parametrize("case", RANDOM_SMALL, ids=_ids(RANDOM_SMALL))
def test_out_len_matches_torch(case):
    torch = pytest.importorskip("torch")
    prob = small_problem(*case)
    nd = prob["ndim"]
    x = torch.zeros(1, prob["C"], *prob["in_len"][:nd], dtype=torch.float64)
    pads = []
    for i in reversed(range(nd)):
        pads += [prob["pad_lo"][i], prob["pad_hi"][i]]
    xp = torch.nn.functional.pad(x, pads)
    w = torch.zeros(prob["K"], prob["C"] // prob["G"], *prob["filt_len"][:nd], dtype=torch.float64)
    conv = torch.nn.functional.conv2d if nd == 2 else torch.nn.functional.conv1d
    y = conv(xp, w, stride=prob["stride"][:nd], dilation=prob["dilation"][:nd], groups=prob["G"])
    assert tuple(y.shape[2:]) == oracle.out_len(prob)


def test_configs_out_len():
    for name, cfg in workloads.CONFIGS.items():
        assert oracle.out_len(cfg) == cfg["out_len"][: cfg["ndim"]], name


# ---------------------------------------------------------------- closed form, all ones


def _ones_expected(prob, flat_idx):
    """N * cnt_h(y) * cnt_w(x), with the counts from the closed-form interval."""
    nd = prob["ndim"]
    ol = oracle.out_len(prob)
    cpg = prob["C"] // prob["G"]
    if nd == 1:
        X = prob["filt_len"][0]
        xx = (flat_idx // cpg) % X
        cw = np.array([count_closed_form(ol[0], prob["in_len"][0], prob["stride"][0],
                                         prob["pad_lo"][0], prob["dilation"][0], t) for t in range(X)])
        return prob["N"] * cw[xx].astype(np.float64)
    Y, X = prob["filt_len"]
    xx = (flat_idx // cpg) % X
    yy = (flat_idx // (cpg * X)) % Y
    ch = np.array([count_closed_form(ol[0], prob["in_len"][0], prob["stride"][0],
                                     prob["pad_lo"][0], prob["dilation"][0], t) for t in range(Y)])
    cw = np.array([count_closed_form(ol[1], prob["in_len"][1], prob["stride"][1],
                                     prob["pad_lo"][1], prob["dilation"][1], t) for t in range(X)])
    return prob["N"] * (ch[yy] * cw[xx]).astype(np.float64)


@pytest.mark.parametrize("name", list(workloads.CONFIGS))
def test_all_ones_closed_form_full_size_sampled(name):
    cfg = workloads.CONFIGS[name]
    x, dy = workloads.inputs(cfg, "ones")
    total = int(np.prod(oracle.dw_shape(cfg)))
    rng = np.random.default_rng(11)
    # every filter tap of the first and last output channel, plus random ones
    per_k = total // cfg["K"]
    idx = np.unique(np.concatenate([np.arange(per_k), total - per_k + np.arange(per_k),
                                    rng.integers(0, total, 64)]))
    dw, ab = oracle.wgrad_sampled(cfg, x, dy, idx)
    want = _ones_expected(cfg, idx)
    assert np.array_equal(dw, want)
    assert np.array_equal(ab, want)


def test_all_ones_c1_tap_values():
    # 8x8, 3x3, pad 1, stride 1: per-tap counts (7, 8, 7) on each axis
    cfg = workloads.CONFIGS["c1"]
    x, dy = workloads.inputs(cfg, "ones")
    dw, _ = oracle.wgrad(cfg, x, dy)
    want = np.array([[49, 56, 49], [56, 64, 56], [49, 56, 49]], np.float64)
    for k in range(cfg["K"]):
        for c in range(cfg["C"]):
            assert np.array_equal(dw[k, :, :, c], want)


@pytest.mark.parametrize("case", RANDOM_SMALL, ids=_ids(RANDOM_SMALL))
def test_all_ones_closed_form_small(case):
    prob = small_problem(*case)
    x, dy = draw_for(prob, "ones", 0)
    dw, _ = oracle.wgrad(prob, x, dy)
    idx = np.arange(dw.size)
    assert np.array_equal(dw.reshape(-1), _ones_expected(prob, idx))


# ---------------------------------------------------------------- dY == 1 and X == 1 invariants


@pytest.mark.parametrize("case", RANDOM_SMALL, ids=_ids(RANDOM_SMALL))
def test_dy_ones_is_window_sum_of_x(case):
    prob = small_problem(*case)
    xb, _ = draw_for(prob, "uniform", 31)
    _, dyb = draw_for(prob, "ones", 0)
    dw, _ = oracle.wgrad(prob, xb, dyb)
    x, _, geo = as_2d(prob, oracle.widen(xb, "bf16"), None)
    G, cpg, kpg = prob["G"], prob["C"] // prob["G"], prob["K"] // prob["G"]
    dw = dw.reshape(G, kpg, geo["Y"], geo["X"], cpg)
    for y, xx in itertools.product(range(geo["Y"]), range(geo["X"])):
        hlo, hhi = valid_range(geo["Ho"], geo["Hi"], geo["sh"], geo["ph"], geo["dh"], y)
        wlo, whi = valid_range(geo["Wo"], geo["Wi"], geo["sw"], geo["pw"], geo["dw"], xx)
        if hhi < hlo or whi < wlo:
            assert np.all(dw[:, :, y, xx, :] == 0)
            continue
        h0 = hlo * geo["sh"] - geo["ph"] + y * geo["dh"]
        w0 = wlo * geo["sw"] - geo["pw"] + xx * geo["dw"]
        win = x[:, h0:h0 + (hhi - hlo) * geo["sh"] + 1:geo["sh"],
                w0:w0 + (whi - wlo) * geo["sw"] + 1:geo["sw"], :]
        s = win.sum(axis=(0, 1, 2)).reshape(G, cpg)
        for k in range(kpg):
            np.testing.assert_allclose(dw[:, k, y, xx, :], s, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("case", RANDOM_SMALL, ids=_ids(RANDOM_SMALL))
def test_x_ones_is_rectangle_sum_of_dy(case):
    prob = small_problem(*case)
    xb, _ = draw_for(prob, "ones", 0)
    _, dyb = draw_for(prob, "uniform", 41)
    dw, _ = oracle.wgrad(prob, xb, dyb)
    _, dy, geo = as_2d(prob, None, oracle.widen(dyb, "bf16"))
    # 2D prefix sums over (ho, wo), summed over n
    P = np.zeros((geo["Ho"] + 1, geo["Wo"] + 1, prob["K"]))
    P[1:, 1:] = dy.sum(axis=0).cumsum(0).cumsum(1)
    G, cpg, kpg = prob["G"], prob["C"] // prob["G"], prob["K"] // prob["G"]
    dw = dw.reshape(G, kpg, geo["Y"], geo["X"], cpg)
    for y, xx in itertools.product(range(geo["Y"]), range(geo["X"])):
        hlo, hhi = valid_range(geo["Ho"], geo["Hi"], geo["sh"], geo["ph"], geo["dh"], y)
        wlo, whi = valid_range(geo["Wo"], geo["Wi"], geo["sw"], geo["pw"], geo["dw"], xx)
        if hhi < hlo or whi < wlo:
            s = np.zeros(prob["K"])
        else:
            s = P[hhi + 1, whi + 1] - P[hlo, whi + 1] - P[hhi + 1, wlo] + P[hlo, wlo]
        for c in range(cpg):
            np.testing.assert_allclose(dw[:, :, y, xx, c], s.reshape(G, kpg), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("name", ["c2", "c3", "c4b", "c5"])
def test_dy_ones_full_size_sampled(name):
    cfg = workloads.CONFIGS[name]
    xb, _ = workloads.inputs(cfg)
    _, dyb = workloads.inputs(cfg, "ones")
    total = int(np.prod(oracle.dw_shape(cfg)))
    idx = np.random.default_rng(3).integers(0, total, 24)
    dw, _ = oracle.wgrad_sampled(cfg, xb, dyb, idx)
    x, _, geo = as_2d(cfg, oracle.widen(xb, cfg["in_dtype"]), None)
    G, cpg, kpg = cfg["G"], cfg["C"] // cfg["G"], cfg["K"] // cfg["G"]
    for i, e in enumerate(idx):
        c = e % cpg
        t = e // cpg
        xx = t % geo["X"]
        t //= geo["X"]
        y = t % geo["Y"]
        kt = t // geo["Y"]
        g = kt // kpg
        hlo, hhi = valid_range(geo["Ho"], geo["Hi"], geo["sh"], geo["ph"], geo["dh"], y)
        wlo, whi = valid_range(geo["Wo"], geo["Wi"], geo["sw"], geo["pw"], geo["dw"], xx)
        h0 = hlo * geo["sh"] - geo["ph"] + y * geo["dh"]
        w0 = wlo * geo["sw"] - geo["pw"] + xx * geo["dw"]
        win = x[:, h0:h0 + (hhi - hlo) * geo["sh"] + 1:geo["sh"],
                w0:w0 + (whi - wlo) * geo["sw"] + 1:geo["sw"], g * cpg + c]
        assert abs(dw[i] - win.sum()) <= 1e-9 * max(1.0, np.abs(win).sum())


# ---------------------------------------------------------------- exact integers vs per-tap matmul


@pytest.mark.parametrize("case", RANDOM_SMALL, ids=_ids(RANDOM_SMALL))
def test_integer_inputs_match_per_tap_int_matmul(case):
    prob = small_problem(*case)
    xb, dyb = draw_for(prob, "int", 51)
    dw, ab = oracle.wgrad(prob, xb, dyb)
    xi = oracle.widen(xb, "bf16").astype(np.int64)
    dyi = oracle.widen(dyb, "bf16").astype(np.int64)
    ref = per_tap_matmul(prob, xi, dyi, dtype=np.int64)
    assert np.array_equal(dw, ref.astype(np.float64))
    # the absolute sums are the same computation on |X|, |dY|
    ref_abs = per_tap_matmul(prob, np.abs(xi), np.abs(dyi), dtype=np.int64)
    assert np.array_equal(ab, ref_abs.astype(np.float64))


@pytest.mark.parametrize("name", ["c1", "c4a", "c4b"])
def test_integer_inputs_configs_full(name):
    cfg = workloads.CONFIGS[name]
    xb, dyb = workloads.inputs(cfg, "int")
    dw, _ = oracle.wgrad(cfg, xb, dyb)
    xi = oracle.widen(xb, cfg["in_dtype"]).astype(np.int64)
    dyi = oracle.widen(dyb, cfg["in_dtype"]).astype(np.int64)
    ref = per_tap_matmul(cfg, xi, dyi, dtype=np.int64)
    assert np.array_equal(dw, ref.astype(np.float64))


# ---------------------------------------------------------------- finite difference of the forward conv


@pytest.mark.parametrize("case", RANDOM_SMALL[:6], ids=_ids(RANDOM_SMALL[:6]))
def test_finite_difference_of_linear_loss(case):
    """L(W) = sum dY * conv_fwd(X, W) is linear in W, so dW_j = L(e_j) - L(0) exactly."""
    prob = small_problem(*case)
    xb, dyb = draw_for(prob, "uniform", 61)
    dw, _ = oracle.wgrad(prob, xb, dyb)
    xv = oracle.widen(xb, "bf16")
    dyv = oracle.widen(dyb, "bf16").reshape(-1)
    shape = oracle.dw_shape(prob)
    n = int(np.prod(shape))
    fd = np.zeros(n)
    for j in range(n):
        e = np.zeros(n)
        e[j] = 1.0
        fd[j] = np.dot(dyv, conv_fwd(prob, xv, e).reshape(-1))
    np.testing.assert_allclose(dw.reshape(-1), fd, rtol=1e-12, atol=1e-12)


def test_finite_difference_golden_shape_c1():
    cfg = workloads.CONFIGS["c1"]
    xb, dyb = workloads.inputs(cfg)
    dw, _ = oracle.wgrad(cfg, xb, dyb)
    xv = oracle.widen(xb, "bf16")
    dyv = oracle.widen(dyb, "bf16").reshape(-1)
    n = dw.size
    rng = np.random.default_rng(5)
    for j in rng.choice(n, 40, replace=False):
        e = np.zeros(n)
        e[j] = 1.0
        fdj = np.dot(dyv, conv_fwd(cfg, xv, e).reshape(-1))
        assert abs(dw.reshape(-1)[j] - fdj) <= 1e-12 * max(1.0, abs(fdj))


@pytest.mark.parametrize("name", ["c2", "c3", "c4a", "c4b"])
def test_random_linear_functional_full_size(name):
    """<dW, V> = sum dY * conv_fwd(X, V) for a random V, at full size, on the
    per-tap-matmul form (the oracle's full dW at these sizes is checked on the
    GPU parity path; here the functional pins the per-tap form used there)."""
    cfg = workloads.CONFIGS[name]
    if name in ("c2", "c3"):
        cfg = workloads.problem(name, N=2)          # keep the CPU suite fast
    xb, dyb = (workloads.draw((cfg["N"], *cfg["in_len"][:cfg["ndim"]], cfg["C"]), cfg["in_dtype"], "uniform", 71),
               workloads.draw((cfg["N"], *oracle.out_len(cfg), cfg["K"]), cfg["in_dtype"], "uniform", 72))
    dw, _ = oracle.wgrad(cfg, xb, dyb)
    xv = oracle.widen(xb, cfg["in_dtype"])
    dyv = oracle.widen(dyb, cfg["in_dtype"])
    v = np.random.default_rng(9).standard_normal(dw.size)
    lhs = float(np.dot(dw.reshape(-1), v))
    torch = pytest.importorskip("torch")
    # forward conv in fp64 through torch (a library routine) on NCHW views
    nd = cfg["ndim"]
    G, cpg, kpg = cfg["G"], cfg["C"] // cfg["G"], cfg["K"] // cfg["G"]
    xt = torch.from_numpy(xv.reshape(cfg["N"], *cfg["in_len"][:nd], cfg["C"])).movedim(-1, 1)
    wt = torch.from_numpy(v.reshape(cfg["K"], *cfg["filt_len"][:nd], cpg)).movedim(-1, 1)
    pads = []
    for i in reversed(range(nd)):
        pads += [cfg["pad_lo"][i], cfg["pad_hi"][i]]
    xt = torch.nn.functional.pad(xt, pads)
    conv = torch.nn.functional.conv2d if nd == 2 else torch.nn.functional.conv1d
    yt = conv(xt, wt, stride=cfg["stride"][:nd], dilation=cfg["dilation"][:nd], groups=G)
    dyt = torch.from_numpy(dyv.reshape(cfg["N"], *oracle.out_len(cfg), cfg["K"])).movedim(-1, 1)
    rhs = float((yt * dyt).sum())
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(rhs))


# ---------------------------------------------------------------- textbook special case and library cross-check


def test_1x1_stride1_pad0_is_per_group_gemm():
    prob = small_problem(2, 3, 2, 5, 4, (6, 7), (1, 1), (1, 1), (0, 0), (0, 0), (1, 1), "fp16")
    xb, dyb = draw_for(prob, "normal", 81)
    dw, _ = oracle.wgrad(prob, xb, dyb)
    x = oracle.widen(xb, "fp16").reshape(-1, 3, 5)
    dy = oracle.widen(dyb, "fp16").reshape(-1, 3, 4)
    for g in range(3):
        ref = dy[:, g, :].T @ x[:, g, :]
        np.testing.assert_allclose(dw.reshape(3, 4, 5)[g], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("case", RANDOM_SMALL, ids=_ids(RANDOM_SMALL))
def test_matches_torch_weight_grad_fp64(case):
    torch = pytest.importorskip("torch")
    prob = small_problem(*case)
    xb, dyb = draw_for(prob, "uniform", 91)
    dw, _ = oracle.wgrad(prob, xb, dyb)
    nd = prob["ndim"]
    x, dy, _ = as_2d(prob, oracle.widen(xb, "bf16"), oracle.widen(dyb, "bf16"))
    xt = torch.from_numpy(x).movedim(-1, 1)
    dyt = torch.from_numpy(dy).movedim(-1, 1)
    if nd == 1:
        xt = xt[:, :, 0, :]
        dyt = dyt[:, :, 0, :]
    pads = []
    for i in reversed(range(nd)):
        pads += [prob["pad_lo"][i], prob["pad_hi"][i]]
    xp = torch.nn.functional.pad(xt, pads)
    cpg = prob["C"] // prob["G"]
    wshape = (prob["K"], cpg, *prob["filt_len"][:nd])
    fn = torch.nn.grad.conv2d_weight if nd == 2 else torch.nn.grad.conv1d_weight
    ref = fn(xp, wshape, dyt, stride=prob["stride"][:nd], dilation=prob["dilation"][:nd],
             groups=prob["G"]).movedim(1, -1).numpy()
    np.testing.assert_allclose(dw, ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- absolute sums, empty sums, determinism


def test_abs_output_is_wgrad_of_absolute_inputs():
    prob = small_problem(2, 2, 2, 3, 2, (6, 6), (3, 3), (1, 1), (1, 1), (1, 1), (1, 1))
    xb, dyb = draw_for(prob, "uniform", 101)
    dw, ab = oracle.wgrad(prob, xb, dyb)
    absx = xb & np.uint16(0x7FFF)         # clear the sign bit: |value| for bf16
    absdy = dyb & np.uint16(0x7FFF)
    dw_abs, _ = oracle.wgrad(prob, absx, absdy)
    np.testing.assert_allclose(ab, dw_abs, rtol=1e-13)
    assert np.all(ab >= np.abs(dw))


def test_empty_batch_and_empty_taps_are_zero():
    prob = small_problem(2, 1, 0, 2, 2, (5, 5), (3, 3), (1, 1), (1, 1), (1, 1), (1, 1))
    dw, ab = oracle.wgrad(prob, np.zeros(0, np.uint16), np.zeros(0, np.uint16))
    assert np.all(dw == 0) and np.all(ab == 0)
    # dilation 4, a 3-tap filter on a 3-wide input and right pad 6: one output,
    # and taps 1 and 2 only ever see padding, so their dW is exactly 0
    prob = small_problem(1, 1, 1, 1, 1, (3,), (3,), (1,), (0,), (6,), (4,))
    xb, dyb = draw_for(prob, "uniform", 5)
    dw, _ = oracle.wgrad(prob, xb, dyb)
    ol = oracle.out_len(prob)[0]
    assert ol == 1
    assert [count_closed_form(ol, 3, 1, 0, 4, t) for t in range(3)] == [1, 0, 0]
    assert dw[0, 1, 0] == 0.0 and dw[0, 2, 0] == 0.0 and dw[0, 0, 0] != 0.0


def test_invalid_problems_rejected():
    bad = small_problem(2, 1, 1, 2, 2, (2, 2), (5, 5), (1, 1), (0, 0), (0, 0), (1, 1))
    with pytest.raises(ValueError):
        oracle.out_len(bad)


def test_multithreaded_is_bitwise_deterministic():
    """One thread and every core give the same bits (each element is one
    ascending sum whatever thread computes it), and a one-thread call does not
    leave later calls on one thread."""
    cfg = workloads.CONFIGS["c4b"]
    xb, dyb = workloads.inputs(cfg)
    a, _ = oracle.wgrad(cfg, xb, dyb, nthreads=1)
    assert oracle.last_threads() == 1
    b, _ = oracle.wgrad(cfg, xb, dyb, nthreads=0)
    assert oracle.last_threads() == oracle.max_threads()
    if (os.cpu_count() or 1) > 1:
        assert oracle.max_threads() > 1, "a one-thread call lowered the default team size"
    assert np.array_equal(a, b)
    i = np.arange(0, a.size, 7, dtype=np.int64)
    c, _ = oracle.wgrad_sampled(cfg, xb, dyb, i, nthreads=3)
    assert oracle.last_threads() == 3
    assert np.array_equal(c, a.reshape(-1)[i])


def test_violations_comparator():
    """The acceptance comparator itself: an error exactly at the bound passes,
    a few ulps above it fails, on either side of the reference; NaN and
    infinities on the GPU side always fail; a NaN reference cannot pass."""
    for out_dtype in ("bf16", "fp16", "fp32"):
        ref = np.array([0.0, 3.0, -7.5, 1024.0, -0.25])
        ab = np.array([0.0, 5.0, 12.0, 2048.0, 0.5])
        b = oracle.bound(ab, out_dtype)
        # an error exactly equal to the bound passes (reference 0: the
        # error is the GPU value itself, with no rounding in between)
        z = np.zeros_like(ref)
        assert not oracle.violations(b, z, ab, out_dtype).any()
        assert not oracle.violations(-b, z, ab, out_dtype).any()
        assert not oracle.violations(ref.copy(), ref, ab, out_dtype).any()
        # three ulps past the bound fails
        over = np.nextafter(np.nextafter(np.nextafter(b, np.inf), np.inf), np.inf)
        assert oracle.violations(over, z, ab, out_dtype).all()
        assert oracle.violations(-over, z, ab, out_dtype).all()
        # nonzero reference: the farthest fp64 value whose error is still
        # within the bound passes, and the value three ulps beyond it fails
        for sgn in (1.0, -1.0):
            edge = ref + sgn * b
            while np.any(np.abs(edge - ref) > b):
                edge = np.where(np.abs(edge - ref) > b, np.nextafter(edge, ref), edge)
            assert not oracle.violations(edge, ref, ab, out_dtype).any()
            far = edge
            for _ in range(3):
                far = np.nextafter(far, sgn * np.inf)
            far = np.where(np.abs(far - ref) > b, far, ref + sgn * 2 * b)
            assert oracle.violations(far, ref, ab, out_dtype).all()
        # non-finite GPU values
        for bad in (np.nan, np.inf, -np.inf):
            v = oracle.violations(np.full(ref.shape, bad), ref, ab, out_dtype)
            assert v.all(), (out_dtype, bad)
        # one bad element among good ones is flagged alone
        g = ref.copy()
        g[2] = np.nan
        assert list(np.nonzero(oracle.violations(g, ref, ab, out_dtype))[0]) == [2]
        # a NaN reference never passes
        assert oracle.violations(ref, np.full(ref.shape, np.nan), ab, out_dtype).all()
    # the bound scales with sum|dY*X|, not with |dW|: a cancelling sum
    # (ref 0, sum of magnitudes 256) tolerates 2 in bf16 and flags 2.01
    assert not oracle.violations(np.array([2.0]), np.array([0.0]), np.array([256.0]), "bf16").any()
    assert oracle.violations(np.array([2.01]), np.array([0.0]), np.array([256.0]), "bf16").all()


def test_bound_formula():
    ab = np.array([0.0, 1.0, 128.0])
    assert np.allclose(oracle.bound(ab, "bf16"), [1e-6, 2 ** -7 + 1e-6, 1.0 + 1e-6])
    assert np.allclose(oracle.bound(ab, "fp16"), [1e-6, 2 ** -10 + 1e-6, 0.125 + 1e-6])
    assert np.allclose(oracle.bound(ab, "fp32"), [1e-6, 1e-5 + 1e-6, 1.28e-3 + 1e-6])


def test_golden_shape_fixture_matches_c1_and_its_all_ones_values():
    """The pages name one golden wgrad shape; c1 is that shape, and with
    all-ones inputs every tap counts its valid positions (corner 49, edge 56,
    centre 64)."""
    import json
    import re
    with open(os.path.join(os.path.dirname(__file__), "golden", "golden_shape.json")) as f:
        gold = json.load(f)
    m = re.fullmatch(r"n(\d+)h(\d+)c(\d+)k(\d+)r(\d+)", gold["name"])
    n, h, c, k, r = map(int, m.groups())
    cfg = workloads.CONFIGS["c1"]
    assert (cfg["N"], cfg["in_len"][0], cfg["in_len"][1], cfg["C"], cfg["K"]) == (n, h, h, c, k)
    assert tuple(cfg["filt_len"]) == (r, r) and cfg["G"] == 1
    xb, dyb = workloads.inputs(cfg, "ones")
    dw, _ = oracle.wgrad(cfg, xb, dyb)
    per_tap = dw.reshape(k, r, r, c)
    expect = np.array([[49, 56, 49], [56, 64, 56], [49, 56, 49]], dtype=np.float64)
    assert np.array_equal(per_tap, np.broadcast_to(expect[None, :, :, None], per_tap.shape))
