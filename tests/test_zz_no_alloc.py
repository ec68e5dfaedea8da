"""wgrad_run_noalloc (the split-K partials in the library's per-GPU scratch
instead of a caller workspace) against wgrad_run, through the C ABI: the same
plan on the same inputs must give the same bits, on two calls in a row, the
second with a smaller input; plans whose workspace exceeds the scratch are
rejected before anything is enqueued."""

import numpy as np
import pytest

import workloads

torch = pytest.importorskip("torch")
gcb = pytest.importorskip("grouped_convolution_backward_amd")

pytestmark = pytest.mark.gpu

OUT_T = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


def _dev(bits, dtype):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).reshape(-1).copy())
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).cuda()


def _both(cfg, dist):
    """(bits from wgrad_run, bits from wgrad_run_noalloc, plan)."""
    p = gcb.Plan(cfg)
    assert 0 < p.workspace_bytes <= gcb.NOALLOC_SCRATCH_BYTES or p.workspace_bytes == 0
    xb, dyb = workloads.inputs(cfg, dist)
    x, dy = _dev(xb, cfg["in_dtype"]), _dev(dyb, cfg["in_dtype"])
    out_t = OUT_T[cfg.get("out_dtype", cfg["in_dtype"])]
    ref = torch.full(p.dw_shape(), float("nan"), dtype=out_t, device="cuda")
    ws = torch.full((max(p.workspace_bytes, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    print(f"[gpu] noalloc {cfg.get('name', '?')} {dist} {p.name}", flush=True)
    p.run(x, dy, ref, ws if p.workspace_bytes else None)
    got = torch.full(p.dw_shape(), float("nan"), dtype=out_t, device="cuda")
    p.run_noalloc(x, dy, got)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(ref).any()) and not bool(torch.isnan(got).any()), "dW elements left unwritten"
    as_int = torch.int32 if out_t == torch.float32 else torch.int16
    return ref.view(as_int).cpu().numpy(), got.view(as_int).cpu().numpy(), p


def test_noalloc_matches_wgrad_run_large_then_smaller():
    # the dense split-K workload at full size (12 MB of partials), then the
    # strided fp16 workload at N = 2 (a smaller split-K workspace), then a
    # plan without split-K
    cases = [(workloads.CONFIGS["c2"], "int"), (workloads.CONFIGS["c2"], "uniform"),
             (workloads.problem("c3", N=2), "uniform"), (workloads.CONFIGS["c1"], "uniform")]
    sizes = []
    for cfg, dist in cases:
        ref, got, p = _both(cfg, dist)
        assert np.array_equal(ref, got), f"{p.name}: {int((ref != got).sum())} elements differ"
        sizes.append(p.workspace_bytes)
    assert sizes[0] > sizes[2] > 0 and sizes[3] == 0


def test_noalloc_rejects_workspace_beyond_scratch():
    cfg = workloads.CONFIGS["c2"]
    p = gcb.Plan(cfg, split_k=200)
    assert p.workspace_bytes > gcb.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(int(np.prod(p.x_shape())), dtype=torch.bfloat16, device="cuda")
    dy = torch.zeros(int(np.prod(p.dy_shape())), dtype=torch.bfloat16, device="cuda")
    dw = torch.full(p.dw_shape(), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gcb.WgradError) as ei:
        p.run_noalloc(x, dy, dw)
    assert ei.value.code == gcb.ERR_INVALID_ARG and "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert bool((dw == 7.0).all()), "a rejected call wrote dW"
