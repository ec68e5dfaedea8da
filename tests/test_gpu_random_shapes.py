"""Seeded random problems through every kernel form that takes them, both
directions, every element against the oracle.

Sixty problems are drawn once from a fixed seed: 1D, 2D and 3D, grouped,
depthwise and dense, with strides, dilations, one-sided pads, channel runs
of 1 to 64, bf16 or fp16 inputs and fp32 or 16-bit outputs, and small
enough that the oracle takes milliseconds. Each one runs under the
automatic plan and under every variant (and a random split-K override) the
planner accepts for it, and dgrad runs under its automatic plan. Inputs
are integers in {-2..2}: every product and partial sum is an integer far
below 2^24, so fp32 accumulation is exact in any order and every output
must equal RNE_out of the oracle bit for bit.
"""

import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
gcb = pytest.importorskip("grouped_convolution_backward_amd")

pytestmark = pytest.mark.gpu

OUT_T = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}
GUARD = 1024


def _draw_cases(n=40, seed=20261202):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        nd = int(rng.integers(1, 4))
        G = int(rng.choice([1, 1, 2, 4, 8, 32]))
        cpg = int(rng.choice([1, 8, 16, 32, 64]))
        kpg = int(rng.choice([1, 8, 16, 32, 64, 96]))
        if G * cpg > 512 or G * kpg > 512:
            continue
        if cpg == 1 or kpg == 1:
            cpg = kpg = 1          # depthwise, or nothing
            G = int(rng.choice([8, 16, 64, 256]))
        hi = {1: 96, 2: 20, 3: 7}[nd]
        in_len = tuple(int(x) for x in rng.integers(1, hi + 1, nd))
        # mostly the filters and unit steps the specialised kernels take,
        # sometimes strides and dilations that send a problem elsewhere
        filt = tuple(int(rng.choice([1, 3, 3, 5] if nd == 1 else [1, 2, 3, 3, 3])) for _ in range(nd))
        stride = tuple(int(rng.choice([1, 1, 1, 2])) for _ in range(nd))
        dil = tuple(int(rng.choice([1, 1, 1, 1, 2])) for _ in range(nd))
        pad_lo = tuple(int(x) for x in rng.integers(0, 3, nd))
        pad_hi = tuple(int(x) for x in rng.integers(0, 3, nd))
        dt = str(rng.choice(["bf16", "fp16"]))
        out = str(rng.choice([dt, dt, "fp32"]))
        cfg = dict(ndim=nd, G=G, N=int(rng.integers(1, 4)), C=G * cpg, K=G * kpg, in_len=in_len, filt_len=filt,
                   stride=stride, dilation=dil, pad_lo=pad_lo, pad_hi=pad_hi, in_dtype=dt, out_dtype=out)
        try:
            ol = oracle.out_len(cfg)
        except Exception:
            continue
        if min(ol[:nd]) < 1:
            continue
        try:
            gcb.Plan(cfg, hip_device=-1)
        except gcb.WgradError:
            continue
        cfg["out_len"] = ol
        cfg["name"] = f"rand{len(cases)}"
        cases.append((cfg, int(rng.choice([0, 0, 2, 3, 7]))))
    return cases


try:
    CASES = _draw_cases(60)
except RuntimeError:          # no library: the tests below cannot run anyway
    CASES = []


def _to_dev(bits, dtype):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).reshape(-1).copy())
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).cuda()


def _bits(t, out_dtype):
    if out_dtype == "fp32":
        return t.cpu().numpy().view(np.uint32).reshape(-1)
    return t.view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)


def _want(v64, out_dtype):
    v = v64.reshape(-1)
    return v.astype(np.float32).view(np.uint32) if out_dtype == "fp32" else oracle.round_to_bits(v, out_dtype)


@pytest.mark.parametrize("i", range(len(CASES)))
def test_random_problem_wgrad(i):
    cfg, split = CASES[i]
    xb = workloads.draw(workloads.x_shape(cfg), cfg["in_dtype"], "int", 900 + i)
    dyb = workloads.draw(workloads.dy_shape(cfg), cfg["in_dtype"], "int", 950 + i)
    dw64, _ = oracle.wgrad(cfg, xb, dyb)
    want = _want(dw64, cfg["out_dtype"])
    x, dy = _to_dev(xb, cfg["in_dtype"]), _to_dev(dyb, cfg["in_dtype"])
    tried = 0
    for ov in ({}, {"variant": gcb.VARIANT_MFMA}, {"variant": gcb.VARIANT_ROWSLAB},
               {"variant": gcb.VARIANT_DEPTHWISE}, {"split_k": split} if split else None):
        if ov is None:
            continue
        try:
            p = gcb.Plan(cfg, **ov)
        except gcb.WgradError:
            continue
        n = int(np.prod(p.dw_shape()))
        buf = torch.full((n + GUARD,), float("nan"), dtype=OUT_T[cfg["out_dtype"]], device="cuda")
        ws = p.new_workspace() if p.workspace_bytes else None
        print(f"[gpu] {cfg['name']} {ov} {p.name}", flush=True)
        p.run(x, dy, buf[:n], ws)
        torch.cuda.synchronize()
        assert np.all(np.isnan(buf[n:].float().cpu().numpy())), f"{p.name}: wrote past the end of dW"
        got = _bits(buf[:n], cfg["out_dtype"])
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, f"{cfg} {ov} {p.name}: {bad.size} of {n} elements differ, first at {bad[:5]}"
        tried += 1
    assert tried >= 1


@pytest.mark.parametrize("i", range(len(CASES)))
def test_random_problem_dgrad(i):
    cfg, _ = CASES[i]
    try:
        p = gcb.DgradPlan(cfg)
    except gcb.WgradError:
        pytest.skip("no dgrad plan for this problem")
    dyb = workloads.draw(workloads.dy_shape(cfg), cfg["in_dtype"], "int", 1900 + i)
    wb = workloads.draw(oracle.dw_shape(cfg), cfg["in_dtype"], "int", 1950 + i)
    dx64, _ = oracle.dgrad(cfg, dyb, wb)
    n = int(np.prod(p.dx_shape()))
    buf = torch.full((n + GUARD,), float("nan"), dtype=OUT_T[cfg["out_dtype"]], device="cuda")
    print(f"[gpu] dgrad {cfg['name']} {p.name}", flush=True)
    p.run(_to_dev(dyb, cfg["in_dtype"]), _to_dev(wb, cfg["in_dtype"]), buf[:n])
    torch.cuda.synchronize()
    assert np.all(np.isnan(buf[n:].float().cpu().numpy())), f"{p.name}: wrote past the end of dX"
    got = _bits(buf[:n], cfg["out_dtype"])
    bad = np.nonzero(got != _want(dx64, cfg["out_dtype"]))[0]
    assert bad.size == 0, f"{cfg} {p.name}: {bad.size} of {n} elements differ, first at {bad[:5]}"
