"""The whole path captured into a HIP graph (as the bench replays it) gives
the eager result on every replay.

Each case captures one run (wgrad: main kernel and reduce; dgrad: its one
kernel) on a side stream, then replays the graph three times. Between the
replays the program does its own eager work: the output is refilled with NaN,
the same plan runs eagerly into another buffer, and the device is
synchronised. Every replay must reproduce the eager result bit for bit (a
plan is deterministic), and the eager runs in between must too. Inputs are
uniform reals, so the comparison covers real rounding and not only exact
integer sums. Nothing on this path records a memset into the graph.
"""

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
    return t.view(torch.int32 if t.dtype == torch.float32 else torch.int16).cpu().numpy().reshape(-1).copy()


CASES = [("wgrad", "c2", 4), ("wgrad", "c3", 2), ("wgrad", "c4a", 4), ("wgrad", "c4b", 4), ("wgrad", "c5", 2),
         ("dgrad", "c2", 2), ("dgrad", "c3", 2), ("dgrad", "c4a", 4), ("dgrad", "c5", 2)]


@pytest.mark.parametrize("kind,base,n", CASES)
def test_graph_replays_match_eager(kind, base, n):
    cfg = workloads.problem(base, N=n)
    dt = cfg["in_dtype"]
    out_t = OUT_T[cfg["out_dtype"]]
    if kind == "wgrad":
        p = gcb.Plan(cfg)
        a = _dev(workloads.draw(workloads.x_shape(cfg), dt, "uniform", 5100), dt)
        b = _dev(workloads.draw(workloads.dy_shape(cfg), dt, "uniform", 5101), dt)
        shape = p.dw_shape()
        ws = p.new_workspace() if p.workspace_bytes else None

        def run(out, stream=None):
            p.run(a, b, out, ws, stream=stream)
    else:
        p = gcb.DgradPlan(cfg)
        a = _dev(workloads.draw(workloads.dy_shape(cfg), dt, "uniform", 5200), dt)
        b = _dev(workloads.draw(oracle.dw_shape(cfg), dt, "uniform", 5201), dt)
        shape = p.dx_shape()

        def run(out, stream=None):
            p.run(a, b, out, stream=stream)

    print(f"[gpu] graph {kind} {base} N={n} {p.name}", flush=True)
    eager = torch.full(shape, float("nan"), dtype=out_t, device="cuda")
    run(eager)
    torch.cuda.synchronize()
    want = _bits(eager)
    assert not bool(torch.isnan(eager).any()), "eager run left elements unwritten"

    out = torch.full(shape, float("nan"), dtype=out_t, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(out, stream=side)                      # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        run(out, stream=side)
    torch.cuda.synchronize()

    other = torch.empty(shape, dtype=out_t, device="cuda")
    for r in range(3):
        out.fill_(float("nan"))                    # eager work between the replays
        other.fill_(float("nan"))
        run(other)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(other), want), f"eager run {r} differs"
        g.replay()
        torch.cuda.synchronize()
        got = _bits(out)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, f"replay {r}: {bad.size} of {got.size} elements differ from the eager run, first at {bad[:5]}"
