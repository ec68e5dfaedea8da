"""Pins for the CPU oracle's backward-data (dgrad) sums: dX of the same
grouped convolution, checked against torch autograd in fp64, against finite
differences of a forward convolution written here (exact: the loss is linear
in X), against a pointwise GEMM, and against the zero pattern strided
pointwise filters leave.
"""

import itertools

import numpy as np
import pytest

import oracle
import workloads


def prob(ndim, G, N, cpg, kpg, in_len, filt, stride, pad_lo, pad_hi, dil, dtype="bf16"):
    return {"ndim": ndim, "G": G, "N": N, "C": G * cpg, "K": G * kpg, "in_len": tuple(in_len),
            "filt_len": tuple(filt), "stride": tuple(stride), "dilation": tuple(dil),
            "pad_lo": tuple(pad_lo), "pad_hi": tuple(pad_hi), "in_dtype": dtype, "out_dtype": dtype}


def draw(p, dist, seed):
    dys = (p["N"], *oracle.out_len(p), p["K"])
    return (workloads.draw(dys, p["in_dtype"], dist, seed),
            workloads.draw(oracle.dw_shape(p), p["in_dtype"], dist, seed + 1))


def fwd(p, xv, wv):
    """Direct fp64 forward grouped convolution (cross-correlation) in any of
    1, 2, 3 spatial dims, channels last."""
    nd = p["ndim"]
    G, N = p["G"], p["N"]
    cpg, kpg = p["C"] // G, p["K"] // G
    il, fl = p["in_len"], p["filt_len"]
    ol = oracle.out_len(p)
    x = xv.reshape(N, *il, G, cpg)
    w = np.asarray(wv, np.float64).reshape(G, kpg, *fl, cpg)
    out = np.zeros((N, *ol, G, kpg))
    for o in itertools.product(*(range(n) for n in ol)):
        for t in itertools.product(*(range(f) for f in fl)):
            i = tuple(o[a] * p["stride"][a] - p["pad_lo"][a] + t[a] * p["dilation"][a] for a in range(nd))
            if all(0 <= i[a] < il[a] for a in range(nd)):
                out[(slice(None), *o)] += np.einsum("ngc,gkc->ngk", x[(slice(None), *i)], w[(slice(None), slice(None), *t)])
    return out


CASES = [
    (2, 1, 2, 3, 4, (7, 6), (3, 3), (1, 1), (1, 1), (1, 1), (1, 1)),
    (2, 2, 1, 2, 3, (7, 8), (3, 2), (2, 1), (1, 0), (2, 1), (1, 2)),
    (2, 4, 2, 1, 1, (6, 7), (3, 3), (3, 2), (2, 0), (0, 2), (2, 1)),
    (1, 2, 2, 3, 2, (9,), (5,), (2,), (2,), (1,), (1,)),
    (3, 2, 1, 2, 2, (4, 5, 4), (2, 3, 2), (2, 1, 2), (1, 1, 0), (0, 1, 1), (1, 1, 2)),
]


def _torch_dgrad(p, dyv, wv):
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    nd = p["ndim"]
    N, C, K, G = p["N"], p["C"], p["K"], p["G"]
    x = torch.zeros(N, C, *p["in_len"], dtype=torch.float64, requires_grad=True)
    pads = []
    for a in reversed(range(nd)):
        pads += [p["pad_lo"][a], p["pad_hi"][a]]
    xp = F.pad(x, pads)
    w = torch.from_numpy(wv.reshape(K, *p["filt_len"], C // G)).permute(0, nd + 1, *range(1, nd + 1)).contiguous()
    conv = {1: F.conv1d, 2: F.conv2d, 3: F.conv3d}[nd]
    y = conv(xp, w, stride=p["stride"], dilation=p["dilation"], groups=G)
    g = torch.from_numpy(dyv.reshape(N, *oracle.out_len(p), K)).permute(0, nd + 1, *range(1, nd + 1))
    (y * g).sum().backward()
    return x.grad.permute(0, *range(2, nd + 2), 1).numpy()


@pytest.mark.parametrize("case", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_dgrad_matches_torch_autograd_fp64(case):
    p = prob(*case)
    dyb, wb = draw(p, "uniform", 11)
    dx, _ = oracle.dgrad(p, dyb, wb)
    ref = _torch_dgrad(p, oracle.widen(dyb, "bf16"), oracle.widen(wb, "bf16"))
    np.testing.assert_allclose(dx, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("case", CASES[:4], ids=[f"case{i}" for i in range(4)])
def test_dgrad_finite_difference_of_forward(case):
    # L(X) = sum dY * conv_fwd(X, W) is linear in X, so dX_j = L(e_j) exactly
    p = prob(*case)
    dyb, wb = draw(p, "uniform", 21)
    dx, _ = oracle.dgrad(p, dyb, wb)
    dyv = oracle.widen(dyb, "bf16").reshape(-1)
    wv = oracle.widen(wb, "bf16")
    n = dx.size
    rng = np.random.default_rng(4)
    for j in rng.choice(n, min(n, 40), replace=False):
        e = np.zeros(n)
        e[j] = 1.0
        fd = float(np.dot(dyv, fwd(p, e, wv).reshape(-1)))
        assert abs(dx.reshape(-1)[j] - fd) <= 1e-12 * max(1.0, abs(fd))


def test_dgrad_integer_inputs_are_exact():
    # integer dY and W: the fp64 sums are exact integers, equal to an int64
    # evaluation of the adjoint identity <dX, e_j> on every element
    p = prob(2, 2, 1, 2, 3, (5, 6), (3, 3), (2, 1), (1, 1), (1, 0), (1, 1))
    dyb, wb = draw(p, "int", 31)
    dx, _ = oracle.dgrad(p, dyb, wb)
    assert np.array_equal(dx, np.rint(dx))
    dyv = oracle.widen(dyb, "bf16").reshape(-1)
    wv = oracle.widen(wb, "bf16")
    for j in range(dx.size):
        e = np.zeros(dx.size)
        e[j] = 1.0
        assert dx.reshape(-1)[j] == np.dot(dyv, fwd(p, e, wv).reshape(-1))


def test_dgrad_pointwise_is_a_gemm_and_strided_gaps_are_zero():
    p = prob(2, 1, 2, 5, 3, (4, 6), (1, 1), (1, 1), (0, 0), (0, 0), (1, 1))
    dyb, wb = draw(p, "uniform", 41)
    dx, _ = oracle.dgrad(p, dyb, wb)
    dy = oracle.widen(dyb, "bf16").reshape(-1, 3)
    w = oracle.widen(wb, "bf16").reshape(3, 5)
    np.testing.assert_allclose(dx.reshape(-1, 5), dy @ w, rtol=1e-12, atol=1e-12)
    # 1x1 with stride 2: only even (h, w) positions receive a gradient
    p2 = prob(2, 1, 1, 4, 4, (6, 6), (1, 1), (2, 2), (0, 0), (0, 0), (1, 1))
    dyb, wb = draw(p2, "uniform", 51)
    dx, ab = oracle.dgrad(p2, dyb, wb)
    mask = np.zeros((6, 6), bool)
    mask[::2, ::2] = True
    assert np.all(dx[0][~mask] == 0) and np.all(ab[0][~mask] == 0) and np.all(ab[0][mask] > 0)


def test_dgrad_abs_sum_definition():
    p = prob(*CASES[1])
    dyb, wb = draw(p, "uniform", 61)
    dx, ab = oracle.dgrad(p, dyb, wb)
    # |sum| <= sum|.|, with equality when every product has one sign
    assert np.all(np.abs(dx) <= ab + 1e-15)
    dyo, wo = draw(p, "ones", 0)
    dx1, ab1 = oracle.dgrad(p, dyo, wo)
    assert np.array_equal(dx1, ab1)
