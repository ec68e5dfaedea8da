"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Bars:
* exact-integer inputs (integers in {-2..2}): every product and partial sum is
  an integer < 2^24, so fp32 accumulation is exact in any order and the GPU
  must return RNE_out(oracle) bit for bit;
* the configured random inputs: |gpu - oracle| <= tau*sum|dY*X| + 1e-6 with
  tau = 2^-7 (bf16 out), 2^-10 (fp16 out), 1e-5 (fp32 out);
* coverage: dW is prefilled with NaN and a guard band after it must be left
  untouched; determinism: two runs give the same bits.
Every test compares every dW element, at full size too: the oracle's
full dW of the largest dense workload takes a few seconds on the host's cores.
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


def run_gpu(cfg, xb, dyb, **ov):
    """Run through the C ABI; returns (dw as fp64 numpy, raw bits, plan)."""
    p = gcb.Plan(cfg, **ov)
    out_dtype = cfg.get("out_dtype", cfg["in_dtype"])
    x = to_dev(xb, cfg["in_dtype"])
    dy = to_dev(dyb, cfg["in_dtype"])
    n = int(np.prod(p.dw_shape()))
    # dW with a guard band; the whole buffer starts as NaN
    buf = torch.full((n + GUARD,), float("nan"), dtype=OUT_T[out_dtype], device="cuda")
    dw = buf[:n]
    ws = None
    if p.workspace_bytes:
        ws = torch.full((p.workspace_bytes // 4 + GUARD,), float("nan"), dtype=torch.float32, device="cuda")
    print(f"[gpu] {cfg.get('name', '?')} {p.name}", flush=True)
    p.run(x, dy, dw, ws)
    torch.cuda.synchronize()
    guard = buf[n:].float().cpu().numpy()
    assert np.all(np.isnan(guard)), "kernel wrote past the end of dW"
    # every element was written (the inputs here are finite, so a NaN left in
    # dW is one the kernels never stored)
    unwritten = int(torch.isnan(dw).sum().item())
    assert unwritten == 0, f"{unwritten} dW elements were never written"
    if ws is not None:
        wguard = ws[p.workspace_bytes // 4:].cpu().numpy()
        assert np.all(np.isnan(wguard)), "kernel wrote past the end of the workspace"
    if out_dtype == "fp32":
        vals = dw.cpu().numpy().astype(np.float64)
        bits = dw.cpu().numpy().view(np.uint32)
    else:
        bits = dw.view(torch.int16).cpu().numpy().view(np.uint16)
        vals = oracle.widen(bits, out_dtype)
    return vals.reshape(p.dw_shape()), bits.reshape(p.dw_shape()), p


def oracle_ref(cfg, xb, dyb):
    dw, ab = oracle.wgrad(cfg, xb, dyb)
    return dw.reshape(-1), ab.reshape(-1)


def check_exact(cfg, gpu_bits_flat, dw64):
    out_dtype = cfg.get("out_dtype", cfg["in_dtype"])
    sel = gpu_bits_flat
    if out_dtype == "fp32":
        want = dw64.astype(np.float32).view(np.uint32)
    else:
        want = oracle.round_to_bits(dw64, out_dtype)
    bad = np.nonzero(sel != want)[0]
    assert bad.size == 0, f"{bad.size} elements differ, first at {bad[:5]}"


def check_tol(cfg, gpu_vals_flat, dw64, ab64):
    out_dtype = cfg.get("out_dtype", cfg["in_dtype"])
    sel = gpu_vals_flat
    bad = np.nonzero(oracle.violations(sel, dw64, ab64, out_dtype))[0]
    assert bad.size == 0, (f"{bad.size} elements outside tau*sum|dY*X|+1e-6, e.g. gpu={sel[bad[:3]]} "
                           f"ref={dw64[bad[:3]]}")


@pytest.mark.parametrize("name", list(workloads.CONFIGS))
def test_configs_exact_integer(name):
    cfg = workloads.CONFIGS[name]
    xb, dyb = workloads.inputs(cfg, "int")
    vals, bits, p = run_gpu(cfg, xb, dyb)
    dw64, _ = oracle_ref(cfg, xb, dyb)
    check_exact(cfg, bits.reshape(-1), dw64)


@pytest.mark.parametrize("name", list(workloads.CONFIGS))
def test_configs_random_within_tolerance(name):
    cfg = workloads.CONFIGS[name]
    xb, dyb = workloads.inputs(cfg)
    vals, bits, p = run_gpu(cfg, xb, dyb)
    dw64, ab64 = oracle_ref(cfg, xb, dyb)
    check_tol(cfg, vals.reshape(-1), dw64, ab64)


@pytest.mark.parametrize("name", ["c2", "c3"])
def test_dense_reduced_batch_full_compare(name):
    # the dense shapes at N=2: every element, several tiles and ragged M (c3)
    cfg = workloads.problem(name, N=2)
    for dist in ("int", None):
        xb, dyb = workloads.inputs(cfg, dist)
        vals, bits, _ = run_gpu(cfg, xb, dyb)
        dw64, ab64 = oracle_ref(cfg, xb, dyb)
        if dist == "int":
            check_exact(cfg, bits.reshape(-1), dw64)
        else:
            check_tol(cfg, vals.reshape(-1), dw64, ab64)


@pytest.mark.parametrize("name", list(workloads.CONFIGS))
def test_configs_all_ones(name):
    cfg = workloads.CONFIGS[name]
    xb, dyb = workloads.inputs(cfg, "ones")
    vals, bits, _ = run_gpu(cfg, xb, dyb)
    dw64, _ = oracle_ref(cfg, xb, dyb)
    check_exact(cfg, bits.reshape(-1), dw64)


@pytest.mark.parametrize("split_k", [1, 2, 3, 5, 16])
def test_split_k_sweep_bitwise_integer(split_k):
    cfg = workloads.problem("c3", N=2)
    xb, dyb = workloads.inputs(cfg, "int")
    _, bits, p = run_gpu(cfg, xb, dyb, split_k=split_k)
    assert p.info["split_k"] == min(split_k, p.info["split_k"])
    dw64, _ = oracle_ref(cfg, xb, dyb)
    check_exact(cfg, bits.reshape(-1), dw64)


@pytest.mark.parametrize("tile", [1, 2, 3, 4, 5])
def test_every_tile_shape(tile):
    cfg = workloads.problem("c3", N=1, out_dtype="fp32")
    xb, dyb = workloads.inputs(cfg)
    vals, _, p = run_gpu(cfg, xb, dyb, tile=tile, variant=gcb.VARIANT_MFMA)
    assert p.info["tile"] == tile
    dw64, ab64 = oracle_ref(cfg, xb, dyb)
    check_tol(cfg, vals.reshape(-1), dw64, ab64)


@pytest.mark.parametrize("gm", [1, 2, 4, 8])
@pytest.mark.parametrize("split_k", [1, 4])
def test_depthwise_group_merge_mfma(gm, split_k):
    # the MFMA path with Gm merged groups: off-diagonal pairs must be masked
    cfg = workloads.problem("c5", N=1, in_len=(20, 20), out_len=(20, 20))
    xb, dyb = workloads.inputs(cfg, "int")
    _, bits, p = run_gpu(cfg, xb, dyb, variant=gcb.VARIANT_MFMA, group_merge=gm, split_k=split_k)
    assert p.info["group_merge"] == gm
    dw64, _ = oracle_ref(cfg, xb, dyb)
    check_exact(cfg, bits.reshape(-1), dw64)


def test_merge_with_single_merged_group():
    # G == Gm: the merged problem has one group block
    cfg = workloads.problem("c4a", G=4, C=32, K=32, N=2)
    xb, dyb = workloads.inputs(cfg, "int")
    _, bits, p = run_gpu(cfg, xb, dyb, group_merge=4)
    dw64, _ = oracle_ref(cfg, xb, dyb)
    check_exact(cfg, bits.reshape(-1), dw64)


@pytest.mark.parametrize("split_k", [1, 4, 8])
def test_depthwise_kernel_split_sweep(split_k):
    cfg = workloads.problem("c5", N=2, in_len=(17, 23), out_len=(17, 23))
    xb, dyb = workloads.inputs(cfg, "int")
    _, bits, p = run_gpu(cfg, xb, dyb, variant=gcb.VARIANT_DEPTHWISE, split_k=split_k)
    dw64, _ = oracle_ref(cfg, xb, dyb)
    check_exact(cfg, bits.reshape(-1), dw64)


SHAPES = [
    # odd channel counts (scalar loads), strides, dilations, asymmetric pads, 1D
    dict(ndim=2, G=1, N=2, C=3, K=5, in_len=(9, 11), filt_len=(3, 3), stride=(1, 1), dilation=(1, 1),
         pad_lo=(1, 1), pad_hi=(1, 1), in_dtype="bf16", out_dtype="bf16"),
    dict(ndim=2, G=2, N=3, C=12, K=20, in_len=(13, 10), filt_len=(3, 2), stride=(2, 1), dilation=(1, 2),
         pad_lo=(1, 0), pad_hi=(2, 1), in_dtype="fp16", out_dtype="fp16"),
    dict(ndim=2, G=4, N=2, C=64, K=32, in_len=(15, 15), filt_len=(5, 5), stride=(3, 2), dilation=(2, 1),
         pad_lo=(2, 0), pad_hi=(0, 2), in_dtype="bf16", out_dtype="fp32"),
    dict(ndim=2, G=1, N=2, C=40, K=24, in_len=(7, 7), filt_len=(1, 1), stride=(1, 1), dilation=(1, 1),
         pad_lo=(0, 0), pad_hi=(0, 0), in_dtype="fp16", out_dtype="fp32"),
    dict(ndim=1, G=8, N=3, C=64, K=48, in_len=(100,), filt_len=(7,), stride=(2,), dilation=(3,),
         pad_lo=(4,), pad_hi=(1,), in_dtype="bf16", out_dtype="bf16"),
    dict(ndim=1, G=16, N=2, C=16, K=16, in_len=(77,), filt_len=(5,), stride=(1,), dilation=(1,),
         pad_lo=(2,), pad_hi=(2,), in_dtype="fp16", out_dtype="fp16"),
    dict(ndim=1, G=64, N=2, C=64, K=64, in_len=(50,), filt_len=(3,), stride=(1,), dilation=(1,),
         pad_lo=(1,), pad_hi=(1,), in_dtype="bf16", out_dtype="bf16"),
    dict(ndim=2, G=3, N=1, C=6, K=9, in_len=(6, 5), filt_len=(3, 3), stride=(1, 1), dilation=(1, 1),
         pad_lo=(0, 0), pad_hi=(0, 0), in_dtype="bf16", out_dtype="bf16"),
]


@pytest.mark.parametrize("i", range(len(SHAPES)))
def test_edge_shapes(i):
    cfg = dict(SHAPES[i], name=f"edge{i}")
    ol = oracle.out_len(cfg)
    cfg["out_len"] = ol
    for dist, seed in (("int", 900 + i), ("uniform", 950 + i)):
        xb = workloads.draw(workloads.x_shape(cfg), cfg["in_dtype"], dist, seed)
        dyb = workloads.draw(workloads.dy_shape(cfg), cfg["in_dtype"], dist, seed + 1)
        vals, bits, p = run_gpu(cfg, xb, dyb)
        dw64, ab64 = oracle_ref(cfg, xb, dyb)
        if dist == "int":
            check_exact(cfg, bits.reshape(-1), dw64)
        else:
            check_tol(cfg, vals.reshape(-1), dw64, ab64)


def test_empty_batch_gives_zeros():
    cfg = workloads.problem("c2", N=0)
    p = gcb.Plan(cfg)
    x = torch.empty(0, dtype=torch.bfloat16, device="cuda")
    dy = torch.empty(0, dtype=torch.bfloat16, device="cuda")
    dw = torch.full(p.dw_shape(), float("nan"), dtype=torch.bfloat16, device="cuda")
    p.run(x, dy, dw)
    torch.cuda.synchronize()
    assert torch.all(dw == 0)


def test_deterministic_bits_across_runs():
    cfg = workloads.CONFIGS["c2"]
    xb, dyb = workloads.inputs(cfg)
    _, b1, p = run_gpu(cfg, xb, dyb)
    _, b2, _ = run_gpu(cfg, xb, dyb)
    assert p.info["split_k"] > 1
    assert np.array_equal(b1, b2)


def test_misaligned_pointer_is_an_error_not_corruption():
    cfg = workloads.CONFIGS["c1"]
    p = gcb.Plan(cfg)
    x = torch.zeros(p.x_shape(), dtype=torch.bfloat16, device="cuda").reshape(-1)
    big = torch.zeros(x.numel() + 8, dtype=torch.bfloat16, device="cuda")
    dy = torch.zeros(p.dy_shape(), dtype=torch.bfloat16, device="cuda").reshape(-1)
    dw = torch.zeros(p.dw_shape(), dtype=torch.bfloat16, device="cuda")
    rc = gcb.load_library().wgrad_run(p.handle, big.data_ptr() + 2, dy.data_ptr(), dw.data_ptr(), None, 0, None)
    assert rc == gcb.ERR_INVALID_ARG
    assert "aligned" in gcb.wgrad_last_error()


ROWSLAB_CASES = [
    # (base config, changes): slab tails, ragged M blocks, several splits
    ("c2", dict(N=2)),
    ("c2", dict(N=1, in_len=(13, 56), out_len=(13, 56))),       # odd number of output rows
    ("c3", dict(N=2)),                                           # stride 2, M = 200 (ragged block)
    ("c3", dict(N=1, K=96, in_len=(20, 30), out_len=(10, 15))),  # fp16, narrow rows
    ("c4a", dict(N=3)),                                          # merged groups, Gm = 4
    ("c4b", dict(N=2, in_len=(300,), out_len=(300,))),           # 1D, row segments with a tail
    ("c4b", dict(N=3, in_len=(65,), pad_lo=(0,), pad_hi=(4,))),  # width 5: 64-position segment + 1-position tail
    ("c4b", dict(N=2, in_len=(64,), in_dtype="fp16", out_dtype="fp32")),   # one whole segment per row, S = 1
    ("c2", dict(N=1, C=128, K=64, in_len=(10, 200), out_len=(10, 200))),   # wide rows: segments
    ("c2", dict(N=2, pad_lo=(0, 0), pad_hi=(2, 2))),             # asymmetric pad
    # stride 2 with more M blocks: ragged (136 = 2*64 + 8), whole (256), grouped (G = 2, 192 rows each)
    ("c3", dict(N=1, K=136, in_len=(20, 30), out_len=(10, 15))),
    ("c3", dict(N=2, C=64, K=256, in_dtype="bf16", out_dtype="fp32", dist="uniform")),
    ("c3", dict(N=1, G=2, C=128, K=384, in_len=(30, 30), out_len=(15, 15))),
]


@pytest.mark.parametrize("i", range(len(ROWSLAB_CASES)))
def test_rowslab_variant(i):
    base, changes = ROWSLAB_CASES[i]
    cfg = workloads.problem(base, **changes)
    cfg["out_len"] = oracle.out_len(cfg)
    cfg["name"] = f"rowslab{i}"
    for dist in ("int", None):
        xb = workloads.draw(workloads.x_shape(cfg), cfg["in_dtype"], dist or cfg["dist"], 700 + i)
        dyb = workloads.draw(workloads.dy_shape(cfg), cfg["in_dtype"], dist or cfg["dist"], 750 + i)
        vals, bits, p = run_gpu(cfg, xb, dyb, variant=gcb.VARIANT_ROWSLAB)
        assert p.info["variant"] == gcb.VARIANT_ROWSLAB
        dw64, ab64 = oracle_ref(cfg, xb, dyb)
        if dist == "int":
            check_exact(cfg, bits.reshape(-1), dw64)
        else:
            check_tol(cfg, vals.reshape(-1), dw64, ab64)


@pytest.mark.parametrize("split_k", [1, 2, 7])
def test_rowslab_split_sweep(split_k):
    cfg = workloads.problem("c2", N=2)
    xb, dyb = workloads.inputs(cfg, "int")
    _, bits, p = run_gpu(cfg, xb, dyb, variant=gcb.VARIANT_ROWSLAB, split_k=split_k)
    dw64, _ = oracle_ref(cfg, xb, dyb)
    check_exact(cfg, bits.reshape(-1), dw64)


@pytest.mark.parametrize("split_k", [1, 2, 3])
def test_rowslab_interleaved_slabs_uneven(split_k):
    """Slabs dealt to the splits in turn (strided shape): 11 output rows make
    11 slabs, which split counts 2 and 3 share unevenly (6 + 5, 4 + 4 + 3),
    so the four slab streams of a workgroup end on different counts."""
    cfg = workloads.problem("c3", N=1, in_len=(22, 56), out_len=(11, 28))
    cfg["name"] = f"rowslab_interleave_s{split_k}"
    xb, dyb = workloads.inputs(cfg, "int")
    _, bits, p = run_gpu(cfg, xb, dyb, variant=gcb.VARIANT_ROWSLAB, split_k=split_k)
    dw64, _ = oracle_ref(cfg, xb, dyb)
    check_exact(cfg, bits.reshape(-1), dw64)


DEPTHWISE_CASES = [
    # windowed depthwise kernel: tails, padding, strides along h, filter heights, fp16
    dict(ndim=2, G=64, N=2, C=64, K=64, in_len=(9, 13), filt_len=(3, 3), stride=(1, 1), dilation=(1, 1),
         pad_lo=(1, 1), pad_hi=(1, 1), in_dtype="bf16", out_dtype="bf16"),
    dict(ndim=2, G=40, N=1, C=40, K=40, in_len=(11, 7), filt_len=(3, 3), stride=(2, 1), dilation=(2, 1),
         pad_lo=(2, 0), pad_hi=(0, 2), in_dtype="fp16", out_dtype="fp16"),
    dict(ndim=2, G=128, N=2, C=128, K=128, in_len=(12, 10), filt_len=(5, 3), stride=(1, 1), dilation=(1, 1),
         pad_lo=(2, 1), pad_hi=(2, 1), in_dtype="bf16", out_dtype="fp32"),
    dict(ndim=2, G=16, N=3, C=16, K=16, in_len=(6, 30), filt_len=(1, 3), stride=(1, 1), dilation=(1, 1),
         pad_lo=(0, 1), pad_hi=(0, 0), in_dtype="bf16", out_dtype="bf16"),
    dict(ndim=1, G=256, N=2, C=256, K=256, in_len=(37,), filt_len=(3,), stride=(1,), dilation=(1,),
         pad_lo=(1,), pad_hi=(1,), in_dtype="fp16", out_dtype="fp16"),
]


@pytest.mark.parametrize("i", range(len(DEPTHWISE_CASES)))
def test_depthwise_windowed(i):
    cfg = dict(DEPTHWISE_CASES[i], name=f"dw{i}")
    cfg["out_len"] = oracle.out_len(cfg)
    for dist, seed in (("int", 600 + i), ("uniform", 650 + i)):
        xb = workloads.draw(workloads.x_shape(cfg), cfg["in_dtype"], dist, seed)
        dyb = workloads.draw(workloads.dy_shape(cfg), cfg["in_dtype"], dist, seed + 1)
        vals, bits, p = run_gpu(cfg, xb, dyb, variant=gcb.VARIANT_DEPTHWISE)
        assert "dwwin" in p.name or "dwstrip" in p.name or "dwtile" in p.name
        dw64, ab64 = oracle_ref(cfg, xb, dyb)
        if dist == "int":
            check_exact(cfg, bits.reshape(-1), dw64)
        else:
            check_tol(cfg, vals.reshape(-1), dw64, ab64)


# strip depthwise kernel (3x3, unit stride and dilation): narrow channel
# blocks (several workers per wave), outputs 1 or 2 rows high (every step
# starts a strip), width tails, one-sided pads, fp16 and fp32 outputs
STRIP_CASES = [
    dict(ndim=2, G=24, N=3, C=24, K=24, in_len=(5, 7), pad_lo=(2, 0), pad_hi=(0, 2),
         in_dtype="bf16", out_dtype="bf16"),
    dict(ndim=2, G=512, N=1, C=512, K=512, in_len=(1, 10), pad_lo=(1, 1), pad_hi=(1, 1),
         in_dtype="bf16", out_dtype="bf16"),
    dict(ndim=2, G=256, N=5, C=256, K=256, in_len=(2, 5), pad_lo=(1, 1), pad_hi=(1, 1),
         in_dtype="fp16", out_dtype="fp16"),
    dict(ndim=2, G=96, N=2, C=96, K=96, in_len=(17, 6), pad_lo=(0, 0), pad_hi=(0, 0),
         in_dtype="fp16", out_dtype="fp32"),
    dict(ndim=2, G=1024, N=2, C=1024, K=1024, in_len=(9, 9), pad_lo=(1, 2), pad_hi=(1, 0),
         in_dtype="bf16", out_dtype="bf16"),
]


@pytest.mark.parametrize("i", range(len(STRIP_CASES)))
def test_depthwise_strip(i):
    cfg = dict(STRIP_CASES[i], name=f"strip{i}", filt_len=(3, 3), stride=(1, 1), dilation=(1, 1))
    cfg["out_len"] = oracle.out_len(cfg)
    for dist, seed in (("int", 700 + i), ("uniform", 750 + i)):
        xb = workloads.draw(workloads.x_shape(cfg), cfg["in_dtype"], dist, seed)
        dyb = workloads.draw(workloads.dy_shape(cfg), cfg["in_dtype"], dist, seed + 1)
        vals, bits, p = run_gpu(cfg, xb, dyb, variant=gcb.VARIANT_DEPTHWISE, tile=3)
        assert "dwstrip" in p.name
        dw64, ab64 = oracle_ref(cfg, xb, dyb)
        if dist == "int":
            check_exact(cfg, bits.reshape(-1), dw64)
        else:
            check_tol(cfg, vals.reshape(-1), dw64, ab64)


@pytest.mark.parametrize("split_k", [1, 2, 7, 64, 1000])
def test_depthwise_strip_split_sweep(split_k):
    # 1000 splits leave most workers without a step
    cfg = workloads.problem("c5", N=1, in_len=(13, 10), out_len=(13, 10))
    xb, dyb = workloads.inputs(cfg, "int")
    _, bits, p = run_gpu(cfg, xb, dyb, variant=gcb.VARIANT_DEPTHWISE, tile=3, split_k=split_k)
    assert "dwstrip" in p.name
    dw64, _ = oracle_ref(cfg, xb, dyb)
    check_exact(cfg, bits.reshape(-1), dw64)


@pytest.mark.parametrize("split_k", [12, 16, 40])
def test_depthwise_strip_xcd_item_order(split_k):
    # 2 x 7 strips of 30 rows: with 2 channel blocks, 16 and 40 splits give
    # every XCD whole splits (items taken XCD by XCD, item counts that 8 does
    # not divide); 12 splits do not (24 workgroups, 3 per XCD), the items go
    # round-robin over all workers
    cfg = workloads.problem("c5", N=2, in_len=(30, 26), out_len=(30, 26))
    cfg["name"] = f"strip_xcd{split_k}"
    xb, dyb = workloads.inputs(cfg, "int")
    _, bits, p = run_gpu(cfg, xb, dyb, variant=gcb.VARIANT_DEPTHWISE, tile=3, split_k=split_k)
    assert "dwstrip" in p.name and p.info["split_k"] == split_k
    dw64, _ = oracle_ref(cfg, xb, dyb)
    check_exact(cfg, bits.reshape(-1), dw64)


# tile depthwise kernel (3x3, unit stride and dilation, C a multiple of 256):
# 512- and 256-channel workgroups, several channel blocks, ragged tiles in
# both directions (Wo not a multiple of the tile width, Ho of the tile
# height), images narrower or shorter than a tile, pads 0, 1 and 2 on either
# side, fp16 and fp32 outputs
TILE_CASES = [
    dict(G=512, N=2, C=512, K=512, in_len=(17, 30), pad_lo=(1, 1), pad_hi=(1, 1), in_dtype="bf16", out_dtype="bf16"),
    dict(G=256, N=3, C=256, K=256, in_len=(9, 31), pad_lo=(1, 1), pad_hi=(1, 1), in_dtype="fp16", out_dtype="fp16"),
    dict(G=768, N=1, C=768, K=768, in_len=(12, 29), pad_lo=(0, 2), pad_hi=(2, 0), in_dtype="bf16", out_dtype="fp32"),
    dict(G=1024, N=2, C=1024, K=1024, in_len=(5, 15), pad_lo=(1, 0), pad_hi=(0, 1), in_dtype="fp16", out_dtype="fp32"),
    dict(G=512, N=5, C=512, K=512, in_len=(1, 1), pad_lo=(1, 1), pad_hi=(1, 1), in_dtype="bf16", out_dtype="bf16"),
    dict(G=512, N=1, C=512, K=512, in_len=(3, 60), pad_lo=(0, 0), pad_hi=(0, 0), in_dtype="bf16", out_dtype="bf16"),
    dict(G=256, N=2, C=256, K=256, in_len=(40, 3), pad_lo=(2, 2), pad_hi=(2, 2), in_dtype="bf16", out_dtype="bf16"),
]


@pytest.mark.parametrize("i", range(len(TILE_CASES)))
def test_depthwise_tile(i):
    cfg = dict(TILE_CASES[i], name=f"dwtile{i}", ndim=2, filt_len=(3, 3), stride=(1, 1), dilation=(1, 1))
    cfg["out_len"] = oracle.out_len(cfg)
    for dist, seed in (("int", 800 + i), ("uniform", 850 + i)):
        xb = workloads.draw(workloads.x_shape(cfg), cfg["in_dtype"], dist, seed)
        dyb = workloads.draw(workloads.dy_shape(cfg), cfg["in_dtype"], dist, seed + 1)
        vals, bits, p = run_gpu(cfg, xb, dyb)
        assert "dwtile" in p.name
        dw64, ab64 = oracle_ref(cfg, xb, dyb)
        if dist == "int":
            check_exact(cfg, bits.reshape(-1), dw64)
        else:
            check_tol(cfg, vals.reshape(-1), dw64, ab64)


@pytest.mark.parametrize("split_k", [1, 2, 3, 7, 64, 1000])
def test_depthwise_tile_split_sweep(split_k):
    # 2 images of 30 x 29 outputs: tiles of up to 14 x 14 (3 per row, the
    # last one column wide); a workgroup takes several tiles when the split
    # is below the tile count, and the split is cut to the tile count above it
    cfg = workloads.problem("c5", N=2, in_len=(30, 29), out_len=(30, 29))
    cfg["name"] = f"dwtile_split{split_k}"
    xb, dyb = workloads.inputs(cfg, "int")
    _, bits, p = run_gpu(cfg, xb, dyb, variant=gcb.VARIANT_DEPTHWISE, tile=4, split_k=split_k)
    assert "dwtile" in p.name and p.info["split_k"] <= split_k
    dw64, _ = oracle_ref(cfg, xb, dyb)
    check_exact(cfg, bits.reshape(-1), dw64)


@pytest.mark.parametrize("form", [1, 2, 3, 4])
def test_depthwise_forms_agree_bitwise(form):
    # the four depthwise kernel forms on one shape, integer inputs: each is
    # exact, so they agree bit for bit
    cfg = workloads.problem("c5", N=2, in_len=(11, 14), out_len=(11, 14))
    xb, dyb = workloads.inputs(cfg, "int")
    _, bits, p = run_gpu(cfg, xb, dyb, variant=gcb.VARIANT_DEPTHWISE, tile=form)
    assert p.info["tile"] == form
    dw64, _ = oracle_ref(cfg, xb, dyb)
    check_exact(cfg, bits.reshape(-1), dw64)


# 3D (NDHWGC / NDHWGK / GKZYXC): dense, strided fp16, merged groups,
# depthwise (merged MFMA), depth dilation with one-sided pads and fp32
# output, and a depth-1 filter with depth stride 3
THREE_D_CASES = [
    dict(G=1, N=2, C=64, K=64, in_len=(5, 9, 10), filt_len=(3, 3, 3), stride=(1, 1, 1), dilation=(1, 1, 1),
         pad_lo=(1, 1, 1), pad_hi=(1, 1, 1), in_dtype="bf16", out_dtype="bf16"),
    dict(G=1, N=1, C=64, K=96, in_len=(7, 11, 12), filt_len=(3, 3, 3), stride=(2, 2, 2), dilation=(1, 1, 1),
         pad_lo=(1, 1, 1), pad_hi=(1, 1, 1), in_dtype="fp16", out_dtype="fp16"),
    dict(G=4, N=2, C=32, K=32, in_len=(4, 8, 8), filt_len=(3, 3, 3), stride=(1, 1, 1), dilation=(1, 1, 1),
         pad_lo=(1, 1, 1), pad_hi=(1, 1, 1), in_dtype="bf16", out_dtype="bf16"),
    dict(G=64, N=2, C=64, K=64, in_len=(4, 7, 7), filt_len=(3, 3, 3), stride=(1, 1, 1), dilation=(1, 1, 1),
         pad_lo=(1, 1, 1), pad_hi=(1, 1, 1), in_dtype="bf16", out_dtype="bf16"),
    dict(G=2, N=1, C=64, K=64, in_len=(6, 6, 9), filt_len=(2, 3, 3), stride=(1, 1, 1), dilation=(2, 1, 1),
         pad_lo=(1, 0, 1), pad_hi=(0, 1, 1), in_dtype="bf16", out_dtype="fp32"),
    dict(G=1, N=1, C=64, K=64, in_len=(7, 8, 8), filt_len=(1, 3, 3), stride=(3, 1, 1), dilation=(1, 1, 1),
         pad_lo=(0, 1, 1), pad_hi=(0, 1, 1), in_dtype="bf16", out_dtype="bf16"),
]


@pytest.mark.parametrize("i", range(len(THREE_D_CASES)))
@pytest.mark.parametrize("variant", ["auto", "mfma", "rowslab"])
def test_3d(i, variant):
    cfg = dict(THREE_D_CASES[i], ndim=3, name=f"3d{i}")
    cfg["out_len"] = oracle.out_len(cfg)
    ov = {}
    if variant == "mfma":
        ov["variant"] = gcb.VARIANT_MFMA
    elif variant == "rowslab":
        ov["variant"] = gcb.VARIANT_ROWSLAB
        try:
            gcb.Plan(cfg, **ov)
        except gcb.WgradError as e:
            assert e.code == gcb.ERR_UNSUPPORTED
            pytest.skip("row-slab kernel does not take this shape")
    for dist, seed in (("int", 800 + i), ("uniform", 850 + i)):
        xb = workloads.draw(workloads.x_shape(cfg), cfg["in_dtype"], dist, seed)
        dyb = workloads.draw(workloads.dy_shape(cfg), cfg["in_dtype"], dist, seed + 1)
        vals, bits, p = run_gpu(cfg, xb, dyb, **ov)
        assert p.dw_shape() == oracle.dw_shape(cfg)
        dw64, ab64 = oracle_ref(cfg, xb, dyb)
        if dist == "int":
            check_exact(cfg, bits.reshape(-1), dw64)
        else:
            check_tol(cfg, vals.reshape(-1), dw64, ab64)


@pytest.mark.parametrize("split_k", [1, 2, 3, 4])
def test_3d_slab_groups_with_short_tail(split_k):
    """3D filters deal the row slabs to the splits four at a time: 5 x 7
    output rows make 35 slabs, nine groups with a short last one, shared
    evenly and unevenly between the splits."""
    cfg = dict(ndim=3, G=1, N=1, C=64, K=64, in_len=(5, 7, 28), filt_len=(3, 3, 3), stride=(1, 1, 1),
               dilation=(1, 1, 1), pad_lo=(1, 1, 1), pad_hi=(1, 1, 1), in_dtype="bf16", out_dtype="bf16",
               name=f"3d_groups_s{split_k}")
    cfg["out_len"] = oracle.out_len(cfg)
    xb = workloads.draw(workloads.x_shape(cfg), "bf16", "int", 870 + split_k)
    dyb = workloads.draw(workloads.dy_shape(cfg), "bf16", "int", 880 + split_k)
    _, bits, p = run_gpu(cfg, xb, dyb, variant=gcb.VARIANT_ROWSLAB, split_k=split_k)
    assert "_sg4_" in p.name, p.name
    dw64, _ = oracle_ref(cfg, xb, dyb)
    check_exact(cfg, bits.reshape(-1), dw64)


# the widened rows at full size (pointwise and 3D dense), every element
@pytest.mark.parametrize("name", list(workloads.WIDER))
@pytest.mark.parametrize("dist", ["int", "uniform", "ones"])
def test_wider_full_size(name, dist):
    cfg = workloads.WIDER[name]
    assert tuple(oracle.out_len(cfg)) == tuple(cfg["out_len"])
    xb, dyb = workloads.inputs(cfg, dist)
    vals, bits, p = run_gpu(cfg, xb, dyb)
    dw64, ab64 = oracle_ref(cfg, xb, dyb)
    if dist == "uniform":
        check_tol(cfg, vals.reshape(-1), dw64, ab64)
    else:
        check_exact(cfg, bits.reshape(-1), dw64)


# pointwise (1x1) shapes on every element: both row-slab channel blocks,
# stride 2, merged groups, fp16 with fp32 output, and the flat MFMA kernel
POINTWISE_CASES = [
    ("pw", dict(N=2), {}),
    ("pw", dict(N=2, stride=(2, 2), out_len=(28, 28)), {}),
    ("pw", dict(N=1, C=96, K=64, in_len=(20, 30), out_len=(20, 30)), {}),
    ("pw", dict(N=2, G=8, C=256, K=128, in_len=(14, 14), out_len=(14, 14)), {}),
    ("pw", dict(N=1, in_len=(17, 23), out_len=(17, 23), in_dtype="fp16", out_dtype="fp32"), {}),
    ("pw", dict(N=1, in_len=(17, 23), out_len=(17, 23)), dict(variant=gcb.VARIANT_MFMA)),
]


@pytest.mark.parametrize("i", range(len(POINTWISE_CASES)))
def test_pointwise(i):
    base, changes, ov = POINTWISE_CASES[i]
    cfg = workloads.problem(base, **changes)
    cfg["name"] = f"pw{i}"
    assert tuple(oracle.out_len(cfg)) == tuple(cfg["out_len"])
    for dist in ("int", "uniform"):
        xb, dyb = workloads.inputs(cfg, dist)
        vals, bits, p = run_gpu(cfg, xb, dyb, **ov)
        dw64, ab64 = oracle_ref(cfg, xb, dyb)
        if dist == "int":
            check_exact(cfg, bits.reshape(-1), dw64)
        else:
            check_tol(cfg, vals.reshape(-1), dw64, ab64)
