"""Maximum sizes: the kernels at the largest inputs their plans accept, and
the fallback just past that limit, checked exactly against the oracle.

The row-slab, ring, strip, tile and row-ring kernels address X and dY through
32-bit buffer offsets, so their plans take inputs below 2 GiB only; larger
inputs go to the flat kernels. These tests put X and dY within a few
hundred KB of 2 GiB (and one case just past it), where a wrapped or
truncated offset would show.

Inputs: P images drawn by the shared seeded generator, tiled N/P times
along the batch on the GPU. Both operations are linear in the batch, so the
exact result is known from the oracle on the P images alone:

* wgrad: dW(N images) = (N/P) * dW(P images). The inputs are 0 or 1 (the
  generator's integers in {-2..2} mapped to 1 where nonzero), so every
  product is 0 or 1 and every partial sum the GPU forms, in any order, is an
  integer no larger than the final one, which is below 2^24 (checked): fp32
  accumulation is exact and the output must equal RNE_out of the exact value
  bit for bit.
* dgrad: dX of image n depends on dY of image n only, so dX(N) is dX(P)
  tiled N/P times, bit for bit (integers in {-2..2}: each dX element is a
  sum of at most 2304 in absolute value, exact in fp32).

A wrapped 32-bit byte offset moves a read by 2^31 or 2^32 bytes, which is
not a whole number of images here (401408 bytes per 56x56x64 bf16 image,
3211264 per 56x56x512 one), so it lands on other pixels and breaks the
equality even though the images repeat.
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
GIB2 = 1 << 31


def tiled(bits, dtype, reps):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).reshape(-1).copy()).cuda()
    t = t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)
    return t.repeat(reps)


def image_bytes(cfg, channels):
    return int(np.prod(cfg["in_len"][:cfg["ndim"]])) * channels * 2


def zero_one(bits, dtype):
    """1 where the generator's integer is nonzero, else 0 (16-bit patterns)."""
    one = np.uint16(0x3F80 if dtype == "bf16" else 0x3C00)
    return np.where(oracle.widen(bits, dtype) != 0, one, np.uint16(0)).astype(np.uint16).reshape(bits.shape)


def wgrad_case(base, N, P, out_dtype, want_prefix, **ov):
    cfg = dict(base, N=N, out_dtype=out_dtype)
    small = dict(cfg, N=P)
    s0, s1 = base["seeds"]
    dt = cfg["in_dtype"]
    xb = zero_one(workloads.draw((P, *cfg["in_len"][:cfg["ndim"]], cfg["C"]), dt, "int", s0 + 10), dt)
    dyb = zero_one(workloads.draw((P, *oracle.out_len(cfg), cfg["K"]), dt, "int", s1 + 10), dt)
    dw_p, _ = oracle.wgrad(small, xb, dyb)
    exact = dw_p.reshape(-1) * (N // P)
    # non-negative terms: every partial sum is at most the final one
    assert float(np.max(exact)) < 2 ** 24, "inputs too large for an exact fp32 check"
    assert float(np.max(exact)) > 0

    p = gcb.Plan(cfg, **ov)
    assert p.name.startswith(want_prefix), p.name
    x = tiled(xb, cfg["in_dtype"], N // P)
    dy = tiled(dyb, cfg["in_dtype"], N // P)
    n = int(np.prod(p.dw_shape()))
    buf = torch.full((n + GUARD,), float("nan"), dtype=OUT_T[out_dtype], device="cuda")
    dw = buf[:n]
    ws = p.new_workspace() if p.workspace_bytes else None
    print(f"[gpu] max size N={N} X={x.numel() * 2} B {p.name}", flush=True)
    p.run(x, dy, dw, ws)
    torch.cuda.synchronize()
    assert np.all(np.isnan(buf[n:].float().cpu().numpy())), "kernel wrote past the end of dW"
    if out_dtype == "fp32":
        got = dw.cpu().numpy().view(np.uint32)
        want = exact.astype(np.float32).view(np.uint32)
    else:
        got = dw.view(torch.int16).cpu().numpy().view(np.uint16)
        want = oracle.round_to_bits(exact, out_dtype)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} of {n} dW elements differ, first at {bad[:5]}"
    return x.numel() * 2, dy.numel() * 2


@pytest.mark.parametrize("out_dtype", ["fp32", "bf16"])
def test_row_slab_just_below_2_gib(out_dtype):
    base = workloads.CONFIGS["c2"]
    P = 7
    N = (GIB2 - 1) // image_bytes(base, base["C"]) // P * P     # 5348 images
    xbytes, dybytes = wgrad_case(base, N, P, out_dtype, "wgrad_rowslab_")
    assert GIB2 - 8 * image_bytes(base, base["C"]) < xbytes < GIB2 and dybytes < GIB2
    torch.cuda.empty_cache()


def test_just_past_2_gib_takes_the_flat_kernel():
    base = workloads.CONFIGS["c2"]
    P = 7
    N = GIB2 // image_bytes(base, base["C"]) // P * P + P           # 5355 images
    xbytes, _ = wgrad_case(base, N, P, "fp32", "wgrad_mfma_")
    assert xbytes > GIB2
    torch.cuda.empty_cache()


@pytest.mark.parametrize("form,prefix", [(3, "wgrad_dwstrip_"), (4, "wgrad_dwtile_")])
def test_depthwise_just_below_2_gib(form, prefix):
    base = workloads.CONFIGS["c5"]
    P = 16
    N = (GIB2 - 1) // image_bytes(base, base["C"]) // P * P        # 656 images
    xbytes, _ = wgrad_case(base, N, P, "fp32", prefix, variant=gcb.VARIANT_DEPTHWISE, tile=form)
    assert GIB2 - 17 * image_bytes(base, base["C"]) < xbytes < GIB2
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,P", [("c2", 7), ("c5", 16)])
def test_dgrad_just_below_2_gib(name, P):
    base = workloads.CONFIGS[name]
    cfg = dict(base)
    N = (GIB2 - 1) // image_bytes(base, base["K"]) // P * P
    cfg["N"] = N
    small = dict(cfg, N=P)
    s0, s1 = base["seeds"]
    dyb = workloads.draw((P, *oracle.out_len(cfg), cfg["K"]), cfg["in_dtype"], "int", s0 + 110)
    wb = workloads.draw(oracle.dw_shape(cfg), cfg["in_dtype"], "int", s1 + 110)
    dx_p, _ = oracle.dgrad(small, dyb, wb)
    want = torch.from_numpy(oracle.round_to_bits(dx_p.reshape(-1), cfg["out_dtype"]).view(np.int16)).cuda()

    p = gcb.DgradPlan(cfg)
    dy = tiled(dyb, cfg["in_dtype"], N // P)
    assert dy.numel() * 2 < GIB2
    w = tiled(wb, cfg["in_dtype"], 1)
    n = int(np.prod(p.dx_shape()))
    buf = torch.full((n + GUARD,), float("nan"), dtype=OUT_T[cfg["out_dtype"]], device="cuda")
    dx = buf[:n]
    print(f"[gpu] dgrad max size N={N} dY={dy.numel() * 2} B {p.name}", flush=True)
    p.run(dy, w, dx)
    torch.cuda.synchronize()
    assert np.all(np.isnan(buf[n:].float().cpu().numpy())), "kernel wrote past the end of dX"
    got = dx.view(torch.int16).view(N // P, -1)
    mism = int((got != want.view(1, -1)).sum().item())
    assert mism == 0, f"{mism} of {n} dX elements differ from the tiled oracle result"
    del buf, dx, dy, got
    torch.cuda.empty_cache()
