"""One plan shared by two streams and by several host threads, each run with
its own workspace and output, through the C ABI: the boundary promises that a
plan is immutable and may be used from several threads and streams at once
when every run has its workspace to itself.

Inputs are the shared generator's integers in {-2..2}, so every partial sum
is an exact integer in fp32 and each result must equal RNE_out of the oracle
bit for bit, whatever else runs beside it. Streams are created at the
default priority.
"""

import threading

import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
gcb = pytest.importorskip("grouped_convolution_backward_amd")

pytestmark = pytest.mark.gpu

OUT_T = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


def _dev(bits, dtype):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).reshape(-1).copy())
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).cuda()


def _bits(t):
    return t.view(torch.int32 if t.dtype == torch.float32 else torch.int16).cpu().numpy().reshape(-1)


def _want(cfg, xb, dyb):
    dw64, _ = oracle.wgrad(cfg, xb, dyb)
    out = cfg.get("out_dtype", cfg["in_dtype"])
    v = dw64.reshape(-1)
    if out == "fp32":
        return v.astype(np.float32).view(np.int32)
    return oracle.round_to_bits(v, out).view(np.int16)


def _inputs(cfg, seed):
    xb = workloads.draw(workloads.x_shape(cfg), cfg["in_dtype"], "int", seed)
    dyb = workloads.draw(workloads.dy_shape(cfg), cfg["in_dtype"], "int", seed + 1)
    return xb, dyb


@pytest.mark.parametrize("base,n", [("c2", 4), ("c5", 2), ("c4a", 4)])
def test_one_plan_two_streams(base, n):
    """Two input sets on two streams, runs interleaved, separate workspaces."""
    cfg = workloads.problem(base, N=n)
    p = gcb.Plan(cfg)
    assert p.info["split_k"] > 1, p.name          # both runs need a workspace
    sets = []
    for k, seed in enumerate((3100, 3200)):
        xb, dyb = _inputs(cfg, seed)
        dw = torch.full(p.dw_shape(), float("nan"), dtype=OUT_T[cfg["out_dtype"]], device="cuda")
        sets.append((_dev(xb, cfg["in_dtype"]), _dev(dyb, cfg["in_dtype"]), dw, p.new_workspace(),
                     torch.cuda.Stream(), _want(cfg, xb, dyb)))
    torch.cuda.synchronize()
    print(f"[gpu] two streams {p.name}", flush=True)
    for _ in range(6):
        for x, dy, dw, ws, s, _w in sets:
            p.run(x, dy, dw, ws, stream=s)
    torch.cuda.synchronize()
    for k, (x, dy, dw, ws, s, want) in enumerate(sets):
        got = _bits(dw)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, f"stream {k}: {bad.size} of {got.size} dW elements differ, first at {bad[:5]}"


def test_one_plan_many_host_threads():
    """Four host threads, each with its own stream, workspace and output,
    call wgrad_run on one plan at the same time."""
    cfg = workloads.problem("c2", N=4)
    p = gcb.Plan(cfg)
    xb, dyb = _inputs(cfg, 3300)
    want = _want(cfg, xb, dyb)
    x, dy = _dev(xb, cfg["in_dtype"]), _dev(dyb, cfg["in_dtype"])
    torch.cuda.synchronize()
    results, errors = [None] * 4, []
    start = threading.Barrier(4)

    def worker(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                ws = p.new_workspace()
                dw = torch.full(p.dw_shape(), float("nan"), dtype=OUT_T[cfg["out_dtype"]], device="cuda")
            s.synchronize()
            start.wait(timeout=60)
            for _ in range(8):
                p.run(x, dy, dw, ws, stream=s)
            s.synchronize()
            results[i] = _bits(dw)
        except Exception as e:                     # reported below, in the test's own thread
            errors.append(e)

    print(f"[gpu] four host threads {p.name}", flush=True)
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a host thread did not finish"
    assert not errors, errors
    for i, got in enumerate(results):
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, f"thread {i}: {bad.size} of {got.size} dW elements differ, first at {bad[:5]}"
