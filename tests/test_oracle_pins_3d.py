"""Pins for the CPU oracle's 3D form (NDHWGC input, NDHWGK output gradient,
GKZYXC weight: the Composable Kernel page
"grouped_convolution_backward_weight_kernel.hpp", its 3D argument
constructor). Each test checks the oracle against something other than
itself: a library routine, a closed form, exact integer arithmetic, a finite
difference of a forward convolution written here, or the 2D oracle on a
depth-1 problem.
"""

import itertools

import numpy as np
import pytest

import oracle
import workloads


def prob3(G, N, cpg, kpg, in_len, filt, stride=(1, 1, 1), pad_lo=(0, 0, 0), pad_hi=(0, 0, 0),
          dil=(1, 1, 1), dtype="bf16"):
    return {"ndim": 3, "G": G, "N": N, "C": G * cpg, "K": G * kpg, "in_len": tuple(in_len),
            "filt_len": tuple(filt), "stride": tuple(stride), "dilation": tuple(dil),
            "pad_lo": tuple(pad_lo), "pad_hi": tuple(pad_hi), "in_dtype": dtype, "out_dtype": dtype}


def draw(prob, dist, seed):
    xs = (prob["N"], *prob["in_len"], prob["C"])
    ys = (prob["N"], *oracle.out_len(prob), prob["K"])
    return (workloads.draw(xs, prob["in_dtype"], dist, seed),
            workloads.draw(ys, prob["in_dtype"], dist, seed + 1))


def fwd3(prob, xv, w):
    """Direct fp64 forward grouped 3D cross-correlation with the problem's
    geometry: Y[n,do,ho,wo,g,k] = sum_{z,y,x,c} X[n,di,hi,wi,g,c] W[g,k,z,y,x,c]."""
    G, N = prob["G"], prob["N"]
    cpg, kpg = prob["C"] // G, prob["K"] // G
    Di, Hi, Wi = prob["in_len"]
    Z, Y, X = prob["filt_len"]
    sd, sh, sw = prob["stride"]
    dd, dh, dw = prob["dilation"]
    pd, ph, pw = prob["pad_lo"]
    Do, Ho, Wo = oracle.out_len(prob)
    x = xv.reshape(N, Di, Hi, Wi, G, cpg)
    w = np.asarray(w, np.float64).reshape(G, kpg, Z, Y, X, cpg)
    out = np.zeros((N, Do, Ho, Wo, G, kpg))
    for od, ho, wo in itertools.product(range(Do), range(Ho), range(Wo)):
        for z, y, xx in itertools.product(range(Z), range(Y), range(X)):
            di, hi, wi = od * sd - pd + z * dd, ho * sh - ph + y * dh, wo * sw - pw + xx * dw
            if 0 <= di < Di and 0 <= hi < Hi and 0 <= wi < Wi:
                out[:, od, ho, wo] += np.einsum("ngc,gkc->ngk", x[:, di, hi, wi], w[:, :, z, y, xx, :])
    return out


SMALL3 = [
    # G, N, cpg, kpg, in_len, filt, stride, pad_lo, pad_hi, dil
    (1, 1, 3, 2, (4, 5, 4), (3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1), (1, 1, 1)),
    (2, 2, 2, 3, (5, 4, 6), (2, 3, 2), (2, 1, 2), (1, 0, 1), (0, 2, 0), (1, 2, 1)),
    (4, 1, 1, 1, (6, 5, 5), (3, 1, 3), (1, 2, 1), (2, 0, 1), (1, 0, 2), (2, 1, 1)),
    (1, 2, 2, 2, (3, 3, 3), (1, 1, 1), (1, 1, 1), (0, 0, 0), (0, 0, 0), (1, 1, 1)),
]


@pytest.mark.parametrize("case", SMALL3, ids=[f"case{i}" for i in range(len(SMALL3))])
def test_3d_matches_torch_conv3d_weight_fp64(case):
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    G, N, cpg, kpg, il, fl, st, pl, ph_, dl = case
    prob = prob3(G, N, cpg, kpg, il, fl, st, pl, ph_, dl)
    xb, dyb = draw(prob, "uniform", 31)
    dw, _ = oracle.wgrad(prob, xb, dyb)
    xv = oracle.widen(xb, "bf16").reshape(N, *il, G * cpg)
    dyv = oracle.widen(dyb, "bf16").reshape(N, *oracle.out_len(prob), G * kpg)
    xt = torch.from_numpy(xv).permute(0, 4, 1, 2, 3).contiguous()
    # asymmetric pads: pad the input explicitly (F.pad takes the last axis first)
    xt = F.pad(xt, (pl[2], ph_[2], pl[1], ph_[1], pl[0], ph_[0]))
    gt = torch.from_numpy(dyv).permute(0, 4, 1, 2, 3).contiguous()
    ref = torch.nn.grad.conv3d_weight(xt, (G * kpg, cpg, *fl), gt, stride=st, padding=0, dilation=dl,
                                      groups=G)
    ref = ref.permute(0, 2, 3, 4, 1).numpy()          # (K, Z, Y, X, C/G)
    np.testing.assert_allclose(dw, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("case", SMALL3[:3], ids=[f"case{i}" for i in range(3)])
def test_3d_finite_difference_of_forward(case):
    # L(W) = sum dY * conv_fwd(X, W) is linear in W, so dW_j = L(e_j) exactly
    G, N, cpg, kpg, il, fl, st, pl, ph_, dl = case
    prob = prob3(G, N, cpg, kpg, il, fl, st, pl, ph_, dl)
    xb, dyb = draw(prob, "uniform", 41)
    dw, _ = oracle.wgrad(prob, xb, dyb)
    xv = oracle.widen(xb, "bf16")
    dyv = oracle.widen(dyb, "bf16").reshape(-1)
    n = dw.size
    rng = np.random.default_rng(3)
    for j in rng.choice(n, min(n, 30), replace=False):
        e = np.zeros(n)
        e[j] = 1.0
        fd = float(np.dot(dyv, fwd3(prob, xv, e).reshape(-1)))
        assert abs(dw.reshape(-1)[j] - fd) <= 1e-12 * max(1.0, abs(fd))


def _count(o_len, i_len, s, p, d, t):
    return sum(1 for o in range(o_len) if 0 <= o * s - p + t * d < i_len)


def test_3d_all_ones_closed_form():
    # X = dY = 1: every element counts its valid (do, ho, wo) positions, a
    # product of three per-axis counts times N
    prob = prob3(2, 3, 2, 2, (5, 6, 7), (3, 2, 3), (2, 1, 2), (1, 0, 1), (1, 1, 0), (1, 2, 1))
    xb, dyb = draw(prob, "ones", 0)
    dw, _ = oracle.wgrad(prob, xb, dyb)
    outl = oracle.out_len(prob)
    for z, y, x in itertools.product(*(range(f) for f in prob["filt_len"])):
        expect = prob["N"]
        for a, t in enumerate((z, y, x)):
            expect *= _count(outl[a], prob["in_len"][a], prob["stride"][a], prob["pad_lo"][a],
                             prob["dilation"][a], t)
        assert np.all(dw[:, z, y, x, :] == expect), (z, y, x)


def test_3d_integer_inputs_equal_int64_per_tap_matmul():
    prob = prob3(2, 2, 3, 2, (4, 5, 5), (2, 3, 3), (1, 2, 1), (1, 1, 1), (0, 1, 1), (2, 1, 1))
    xb, dyb = draw(prob, "int", 51)
    dw, _ = oracle.wgrad(prob, xb, dyb)
    G, N = prob["G"], prob["N"]
    cpg, kpg = prob["C"] // G, prob["K"] // G
    x = np.rint(oracle.widen(xb, "bf16")).astype(np.int64).reshape(N, *prob["in_len"], G, cpg)
    dy = np.rint(oracle.widen(dyb, "bf16")).astype(np.int64).reshape(N, *oracle.out_len(prob), G, kpg)
    outl = oracle.out_len(prob)
    ref = np.zeros((G, kpg, *prob["filt_len"], cpg), np.int64)
    for tap in itertools.product(*(range(f) for f in prob["filt_len"])):
        # the input index of every output position along each axis, -1 when outside
        idx = []
        for a in range(3):
            o = np.arange(outl[a])
            i = o * prob["stride"][a] - prob["pad_lo"][a] + tap[a] * prob["dilation"][a]
            idx.append(np.where((i >= 0) & (i < prob["in_len"][a]), i, -1))
        od, oh, ow = np.meshgrid(*[np.arange(n) for n in outl], indexing="ij")
        di, hi, wi = idx[0][od], idx[1][oh], idx[2][ow]
        ok = (di >= 0) & (hi >= 0) & (wi >= 0)
        a_ = dy[:, od[ok], oh[ok], ow[ok]].reshape(-1, G, kpg)
        b_ = x[:, di[ok], hi[ok], wi[ok]].reshape(-1, G, cpg)
        for g in range(G):
            ref[g, :, tap[0], tap[1], tap[2], :] = a_[:, g, :].T @ b_[:, g, :]
    assert np.array_equal(dw, ref.reshape(dw.shape).astype(np.float64))


def test_3d_depth_one_equals_2d_oracle():
    # one input plane and a depth-1 filter: the 3D sums are the 2D sums
    p2 = {"ndim": 2, "G": 2, "N": 2, "C": 6, "K": 4, "in_len": (7, 6), "filt_len": (3, 2),
          "stride": (2, 1), "dilation": (1, 2), "pad_lo": (1, 1), "pad_hi": (2, 0),
          "in_dtype": "fp16", "out_dtype": "fp16"}
    p3 = dict(p2, ndim=3, in_len=(1, 7, 6), filt_len=(1, 3, 2), stride=(3, 2, 1),
              dilation=(2, 1, 2), pad_lo=(0, 1, 1), pad_hi=(0, 2, 0))
    xs = (2, 7, 6, 6)
    ys = (2, *oracle.out_len(p2), 4)
    xb = workloads.draw(xs, "fp16", "normal", 61)
    dyb = workloads.draw(ys, "fp16", "normal", 62)
    assert oracle.out_len(p3) == (1, *oracle.out_len(p2))
    d2, a2 = oracle.wgrad(p2, xb, dyb)
    d3, a3 = oracle.wgrad(p3, xb, dyb)
    assert np.array_equal(d3.reshape(d2.shape), d2) and np.array_equal(a3.reshape(a2.shape), a2)


def test_3d_pointwise_is_a_gemm():
    prob = prob3(1, 2, 5, 3, (3, 4, 2), (1, 1, 1))
    xb, dyb = draw(prob, "uniform", 71)
    dw, _ = oracle.wgrad(prob, xb, dyb)
    x = oracle.widen(xb, "bf16").reshape(-1, 5)
    dy = oracle.widen(dyb, "bf16").reshape(-1, 3)
    np.testing.assert_allclose(dw.reshape(3, 5), dy.T @ x, rtol=1e-12, atol=1e-12)


def test_3d_out_len_matches_torch():
    torch = pytest.importorskip("torch")
    for case in SMALL3:
        G, N, cpg, kpg, il, fl, st, pl, ph_, dl = case
        prob = prob3(G, N, cpg, kpg, il, fl, st, pl, ph_, dl)
        x = torch.zeros(1, 1, *(i + a + b for i, a, b in zip(il, pl, ph_)), dtype=torch.float64)
        w = torch.zeros(1, 1, *fl, dtype=torch.float64)
        y = torch.nn.functional.conv3d(x, w, stride=st, dilation=dl)
        assert tuple(y.shape[2:]) == oracle.out_len(prob)


def test_3d_sampled_matches_full():
    prob = prob3(2, 1, 2, 2, (4, 4, 5), (2, 2, 3), (1, 1, 1), (1, 0, 1), (0, 1, 1), (1, 1, 1))
    xb, dyb = draw(prob, "uniform", 81)
    dw, ab = oracle.wgrad(prob, xb, dyb)
    idx = np.array([0, 5, 17, dw.size - 1, dw.size // 2], np.int64)
    ds, as_ = oracle.wgrad_sampled(prob, xb, dyb, idx)
    assert np.array_equal(ds, dw.reshape(-1)[idx]) and np.array_equal(as_, ab.reshape(-1)[idx])


def test_3d_invalid_problems_rejected():
    with pytest.raises(ValueError):
        oracle.out_len(prob3(1, 1, 1, 1, (2, 4, 4), (3, 1, 1)))       # depth filter too long
    with pytest.raises(ValueError):
        oracle.out_len(prob3(1, 1, 1, 1, (4, 4, 4), (1, 1, 1), stride=(0, 1, 1)))
