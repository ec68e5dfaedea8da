"""GPU parity of the filter-row ring form of the row-slab variant (tile 2)
against the CPU oracle, through the C ABI.

The ring form stages each input row once per workgroup and keeps it for the
output rows that share it, so the cases below aim at its bookkeeping: splits
that cross image boundaries (the window restarts), h-strides 1..3 (3 - sh
rows carried over), both w-strides, one-sided pads, ragged M blocks, merged
groups with channel runs of 4 and 8, rows of every instance width, direct
output (no split) and fp32 output. Integer inputs must match the oracle bit
for bit; the configured distributions must meet the tolerance. The ring and
the one-row-per-workgroup form must agree bitwise on integer inputs.
"""

import numpy as np
import pytest

import oracle
import workloads
from test_gpu_parity import check_exact, check_tol, oracle_ref, run_gpu

torch = pytest.importorskip("torch")
gcb = pytest.importorskip("grouped_convolution_backward_amd")

pytestmark = pytest.mark.gpu

RING = dict(variant=3, tile=2)

RING_CASES = [
    ("c4a", dict(N=3)),                                               # Gm = 4; splits cross image starts
    ("c2", dict(N=2)),                                                # dense, two 32-channel blocks, 56-wide rows
    ("c3", dict(N=2)),                                                # stride 2 both axes, fp16, M = 200 (ragged)
    ("c2", dict(N=2, C=64, K=40, in_len=(20, 30), stride=(3, 1))),    # h-stride 3: no row carried over
    ("c2", dict(N=1, in_len=(17, 30), stride=(2, 1))),                # h-stride 2, w-stride 1
    ("c2", dict(N=2, K=64, in_len=(9, 61), stride=(1, 2))),           # w-stride 2 only
    ("c2", dict(N=1, C=32, K=32, in_len=(7, 62))),                    # 62-wide rows, M block 32
    ("c2", dict(N=2, C=96, K=72, pad_lo=(0, 2), pad_hi=(2, 0))),      # one-sided pads, 3 C blocks, ragged M
    (dict(ndim=2, G=64, N=2, C=256, K=128, in_len=(10, 14), filt_len=(3, 3), stride=(1, 1), dilation=(1, 1),
          pad_lo=(1, 1), pad_hi=(1, 1), in_dtype="bf16", out_dtype="fp32", dist="uniform"), {}),   # C/G = 4, Gm = 8
    (dict(ndim=2, G=8, N=3, C=256, K=64, in_len=(5, 11), filt_len=(3, 3), stride=(1, 1), dilation=(1, 1),
          pad_lo=(0, 0), pad_hi=(0, 0), in_dtype="fp16", out_dtype="fp16", dist="normal"), {}),    # no pads, Ho = 3
]


def _cfg(i):
    base, changes = RING_CASES[i]
    cfg = workloads.problem(base, **changes) if isinstance(base, str) else dict(base, **changes)
    cfg["out_len"] = oracle.out_len(cfg)
    cfg["name"] = f"ring{i}"
    return cfg


@pytest.mark.parametrize("i", range(len(RING_CASES)))
def test_ring_form(i):
    cfg = _cfg(i)
    for dist in ("int", None):
        xb = workloads.draw(workloads.x_shape(cfg), cfg["in_dtype"], dist or cfg["dist"], 900 + i)
        dyb = workloads.draw(workloads.dy_shape(cfg), cfg["in_dtype"], dist or cfg["dist"], 950 + i)
        vals, bits, p = run_gpu(cfg, xb, dyb, **RING)
        assert p.name.startswith("wgrad_ring_"), p.name
        dw64, ab64 = oracle_ref(cfg, xb, dyb)
        if dist == "int":
            check_exact(cfg, bits.reshape(-1), dw64)
        else:
            check_tol(cfg, vals.reshape(-1), dw64, ab64)


@pytest.mark.parametrize("split_k", [1, 2, 5, 13, 1000])
def test_ring_split_sweep_bitwise_integer(split_k):
    cfg = workloads.problem("c4a", N=2)
    cfg["name"] = f"ring_split{split_k}"
    xb, dyb = workloads.inputs(cfg, "int")
    _, bits, p = run_gpu(cfg, xb, dyb, split_k=split_k, **RING)
    assert 1 <= p.info["split_k"] <= min(split_k, cfg["N"] * p.info["out_len"][0])
    dw64, _ = oracle_ref(cfg, xb, dyb)
    check_exact(cfg, bits.reshape(-1), dw64)


@pytest.mark.parametrize("i", [0, 1, 2, 7])
def test_ring_and_row_forms_agree_bitwise(i):
    cfg = _cfg(i)
    xb = workloads.draw(workloads.x_shape(cfg), cfg["in_dtype"], "int", 1900 + i)
    dyb = workloads.draw(workloads.dy_shape(cfg), cfg["in_dtype"], "int", 1950 + i)
    _, ring_bits, p2 = run_gpu(cfg, xb, dyb, **RING)
    _, row_bits, p1 = run_gpu(cfg, xb, dyb, variant=3, tile=1)
    assert p2.name.startswith("wgrad_ring_") and p1.name.startswith("wgrad_rowslab_")
    assert np.array_equal(ring_bits, row_bits)


def test_ring_empty_batch_gives_zeros():
    cfg = workloads.problem("c4a", N=0)
    p = gcb.Plan(cfg, **RING)
    assert p.name.startswith("wgrad_ring_")
    x = torch.empty(0, dtype=torch.bfloat16, device="cuda")
    dy = torch.empty(0, dtype=torch.bfloat16, device="cuda")
    dw = torch.full(p.dw_shape(), float("nan"), dtype=torch.bfloat16, device="cuda")
    p.run(x, dy, dw)
    torch.cuda.synchronize()
    assert torch.all(dw == 0)
