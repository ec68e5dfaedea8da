"""Host-side tests of the C ABI (no GPU): the library loads and exports every
symbol the header declares, plans validate and size problems correctly, and
the split-K / merge choices respect their invariants. Plans are made with
hip_device = -1 (sized for an MI355X without touching the HIP runtime)."""

import os
import re
import subprocess

import pytest

import grouped_convolution_backward_amd as gcb
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wgrad.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wgrad_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = gcb.load_library()
    declared = _declared_functions()
    assert set(declared) == set(gcb.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", gcb.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\b(wgrad_[a-z_]+)\b", out))
    for name in declared:
        assert name in exported, name
        assert hasattr(lib, name)
    assert re.match(r"^\d+\.\d+\.\d+$", gcb.wgrad_version())


def plan(cfg, **kw):
    return gcb.Plan(cfg, hip_device=-1, **kw)


@pytest.mark.parametrize("name", list(workloads.CONFIGS))
def test_plan_sizes_for_configs(name):
    cfg = workloads.CONFIGS[name]
    p = plan(cfg)
    info = p.info
    nd = cfg["ndim"]
    assert info["out_len"][:nd] == cfg["out_len"][:nd]
    G = cfg["G"]
    assert info["gemm_m"] == cfg["K"] // G
    taps = 1
    for f in cfg["filt_len"][:nd]:
        taps *= f
    assert info["gemm_n"] == cfg["C"] // G * taps
    R = cfg["N"]
    for o in cfg["out_len"][:nd]:
        R *= o
    assert info["gemm_k"] == R
    S = info["split_k"]
    ndw = cfg["K"] * taps * (cfg["C"] // G)
    assert info["workspace_bytes"] == (S * ndw * 4 if S > 1 else 0)
    assert p.workspace_bytes == info["workspace_bytes"]
    assert info["num_cus"] == 256
    assert ("spk%d" % S) in p.name


def test_depthwise_config_uses_depthwise_kernel_and_dense_uses_mfma():
    p5 = plan(workloads.CONFIGS["c5"])
    assert p5.info["variant"] == gcb.VARIANT_DEPTHWISE
    assert p5.info["tile"] == 4 and "dwtile" in p5.name      # 3x3, unit stride, C % 256 == 0: tile form
    # the tiny golden shape has too few output rows for row slabs
    assert plan(workloads.CONFIGS["c1"]).info["variant"] == gcb.VARIANT_MFMA
    for n in ("c2", "c3", "c4a", "c4b"):
        assert plan(workloads.CONFIGS[n]).info["variant"] == gcb.VARIANT_ROWSLAB


def test_grid_and_xcd_snap():
    # the main grid is tiles * groups/Gm * S and, whenever S > 1 and the clamp
    # allows it, a multiple of the 8 XCDs
    for name, cfg in workloads.CONFIGS.items():
        info = plan(cfg).info
        if info["variant"] != gcb.VARIANT_MFMA:
            continue
        Gm = info["group_merge"]
        Mm = Gm * info["gemm_m"]
        Nm = Gm * info["gemm_n"]
        tiles = -(-Mm // info["tile_m"]) * -(-Nm // info["tile_n"])
        assert info["grid_main"] == tiles * (cfg["G"] // Gm) * info["split_k"], name
        if info["split_k"] > 1:
            assert info["grid_main"] % 8 == 0, name


def test_split_k_clamped_to_k_tiles_before_snap():
    # a shallow reduction: R = 2*3*3 = 18 positions -> one K tile of 32, so S
    # must be 1 whatever the occupancy target asks for
    cfg = workloads.problem("c1", N=2, in_len=(3, 3))
    info = plan(cfg).info
    assert info["split_k"] == 1
    # R = 4*8*8 = 256 -> 8 K tiles: S <= 8
    info = plan(workloads.problem("c1", N=4)).info
    assert 1 <= info["split_k"] <= 8


def test_split_k_override_and_effective_slices():
    cfg = workloads.CONFIGS["c1"]            # R = 64, tile K = 32
    assert plan(cfg, split_k=2).info["split_k"] == 2
    # more slices than K tiles collapse to the number of non-empty slices
    assert plan(cfg, split_k=7).info["split_k"] == 2
    info = plan(workloads.CONFIGS["c2"], split_k=5).info
    assert info["split_k"] == 5
    assert info["workspace_bytes"] == 5 * 64 * 9 * 64 * 4


def test_group_merge_choices_are_admissible():
    # auto Gm is a power of two dividing G, at most 8, and only merges when the
    # per-group M leaves the 16-row MFMA edge unfilled
    for name, cfg in workloads.CONFIGS.items():
        info = plan(cfg, variant=gcb.VARIANT_MFMA).info
        Gm = info["group_merge"]
        assert Gm & (Gm - 1) == 0 and cfg["G"] % Gm == 0 and Gm <= 8, name
        if info["gemm_m"] >= 16:
            assert Gm == 1
    assert plan(workloads.CONFIGS["c4a"], variant=gcb.VARIANT_MFMA).info["group_merge"] == 2
    # the row-slab kernel fills its 32-row M block with groups instead
    assert plan(workloads.CONFIGS["c4a"]).info["group_merge"] == 4
    assert plan(workloads.CONFIGS["c5"], variant=gcb.VARIANT_MFMA).info["group_merge"] == 8
    for gm in (1, 2, 4, 8):
        info = plan(workloads.CONFIGS["c5"], variant=gcb.VARIANT_MFMA, group_merge=gm).info
        assert info["group_merge"] == gm
        assert info["vector_width"] == gm
        # workspace is sized from the unmerged dW, whatever Gm is
        S = info["split_k"]
        assert info["workspace_bytes"] == (S * 512 * 9 * 4 if S > 1 else 0)


def _expect(code, cfg, **kw):
    with pytest.raises(gcb.WgradError) as ei:
        plan(cfg, **kw)
    assert ei.value.code == code
    assert gcb.wgrad_last_error() != ""
    return str(ei.value)


def test_invalid_problems_are_rejected_with_reasons():
    c1 = workloads.CONFIGS["c1"]
    assert "multiples of G" in _expect(gcb.ERR_INVALID_ARG, workloads.problem("c1", G=3))
    _expect(gcb.ERR_INVALID_ARG, workloads.problem("c1", in_dtype="fp32"))
    _expect(gcb.ERR_INVALID_ARG, workloads.problem("c1", out_dtype="fp16"))
    _expect(gcb.ERR_INVALID_ARG, workloads.problem("c1", ndim=3, in_len=(8, 8, 8)))
    assert "empty output" in _expect(gcb.ERR_INVALID_ARG, workloads.problem("c1", in_len=(1, 1), pad_lo=(0, 0), pad_hi=(0, 0)))
    _expect(gcb.ERR_INVALID_ARG, workloads.problem("c1", stride=(0, 1)))
    _expect(gcb.ERR_INVALID_ARG, workloads.problem("c1", dilation=(1, 0)))
    _expect(gcb.ERR_INVALID_ARG, workloads.problem("c1", pad_lo=(-1, 1)))
    _expect(gcb.ERR_INVALID_ARG, workloads.problem("c1", N=-1))
    assert "31 bits" in _expect(gcb.ERR_INVALID_ARG, workloads.problem("c2", N=20000))
    # overrides the kernels cannot honour
    _expect(gcb.ERR_UNSUPPORTED, workloads.CONFIGS["c5"], variant=gcb.VARIANT_MFMA, group_merge=3)
    _expect(gcb.ERR_UNSUPPORTED, workloads.CONFIGS["c4a"], group_merge=64)
    _expect(gcb.ERR_UNSUPPORTED, c1, variant=gcb.VARIANT_DEPTHWISE)
    _expect(gcb.ERR_UNSUPPORTED, c1, tile=99)


def test_empty_batch_plans_one_slice():
    info = plan(workloads.problem("c2", N=0)).info
    assert info["gemm_k"] == 0 and info["split_k"] == 1 and info["workspace_bytes"] == 0


def test_fp32_output_mode_plans():
    p = plan(workloads.problem("c3", out_dtype="fp32"))
    assert p.info["variant"] in (gcb.VARIANT_MFMA, gcb.VARIANT_ROWSLAB)


def test_depthwise_kernel_forms():
    # tile selects the depthwise kernel form: 1 generic, 2 windowed, 3 strip, 4 tile
    c5 = workloads.CONFIGS["c5"]
    for form, tag in ((1, "wgrad_dw_"), (2, "wgrad_dwwin_"), (3, "wgrad_dwstrip_"), (4, "wgrad_dwtile_")):
        p = plan(c5, variant=gcb.VARIANT_DEPTHWISE, tile=form)
        assert p.info["tile"] == form and p.name.startswith(tag), (form, p.name)
    # the strip and tile forms need unit stride and dilation in both axes
    strided = workloads.problem("c5", stride=(2, 1))
    assert plan(strided).info["tile"] == 2
    _expect(gcb.ERR_UNSUPPORTED, strided, variant=gcb.VARIANT_DEPTHWISE, tile=3)
    _expect(gcb.ERR_UNSUPPORTED, strided, variant=gcb.VARIANT_DEPTHWISE, tile=4)
    _expect(gcb.ERR_UNSUPPORTED, c5, variant=gcb.VARIANT_DEPTHWISE, tile=5)
    # strip form: one 8-wave workgroup per CU, a split per workgroup of a
    # 256-channel block (two blocks for C = 512)
    p = plan(c5, variant=gcb.VARIANT_DEPTHWISE, tile=3)
    assert p.info["grid_main"] == 256 and p.info["split_k"] == 128


def test_depthwise_tile_form_plans():
    # c5: 256-channel workgroups (two blocks), 14 x 28 output tiles (56 / 14 =
    # 4 rows of tiles, 56 / 28 = 2 columns), 16 x 8 tiles = 128 workgroups per
    # block, one tile each, one slice per workgroup
    p = plan(workloads.CONFIGS["c5"])
    assert p.info["grid_main"] == 256 and p.info["split_k"] == 128
    assert p.name == "wgrad_dwtile_bf16_3x3_t14x28_spk128_gm256"
    assert p.workspace_bytes == 128 * 512 * 9 * 4
    # three blocks for C = 768
    p = plan(dict(workloads.CONFIGS["c5"], G=768, C=768, K=768))
    assert p.info["tile"] == 4 and "x28_" in p.name and p.name.endswith("gm256")
    assert p.info["grid_main"] == 3 * p.info["split_k"] and p.info["split_k"] <= 256 // 3
    # channels not a multiple of 256: the strip form
    assert plan(dict(workloads.CONFIGS["c5"], G=96, C=96, K=96)).info["tile"] == 3
    # split_k: workgroups per channel block, at most one per tile; S = 1 writes dW
    p = plan(workloads.CONFIGS["c5"], split_k=1)
    assert p.info["split_k"] == 1 and p.workspace_bytes == 0 and p.info["grid_main"] == 2
    small = workloads.problem("c5", N=1, in_len=(3, 3), out_len=(3, 3))
    p = plan(small, split_k=50)
    assert p.info["split_k"] == 3 and "_t1x28_" in p.name    # three 1-row tiles, one per workgroup
    # more tiles than workgroups: rows per tile grow before tiles are shared
    big = workloads.problem("c5", N=64)
    p = plan(big)
    assert p.info["split_k"] == 128 and p.info["grid_main"] == 256


def test_magic_division_exhaustive(tmp_path):
    """The (n, ho, wo) decode divides by Wo and Ho with a multiply-high; check
    the header's constants against real division for every dividend the
    configurations use (and beyond), in a host program built from the same header."""
    src = tmp_path / "magic.cpp"
    src.write_text(r'''
#include <cstdio>
#include <cstdint>
#include "grouped_convolution_backward_amd/csrc/wgrad_internal.hpp"
int main() {
    const uint32_t divs[] = {1, 2, 3, 5, 7, 8, 28, 56, 1024, 1000, 4095, 65537, 3000017u};
    long bad = 0;
    for (uint32_t d : divs) {
        wgrad::MagicU32 m = wgrad::make_magic(d);
        for (uint32_t n = 0; n < (1u << 22); ++n)
            if (wgrad::magic_div_host(n, m) != n / d) ++bad;
        for (uint32_t n = 0x7fffffffu; n > 0x7fffffffu - (1u << 20); --n)
            if (wgrad::magic_div_host(n, m) != n / d) ++bad;
    }
    for (uint32_t d = 1; d < 5000; ++d) {
        wgrad::MagicU32 m = wgrad::make_magic(d);
        for (uint32_t n = 0; n < 200000; n += 7)
            if (wgrad::magic_div_host(n, m) != n / d) ++bad;
    }
    printf("%ld\n", bad);
    return bad != 0;
}
''')
    exe = tmp_path / "magic"
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", ROOT, "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.strip() == "0"


def test_run_rejects_null_plan_and_pointers_without_gpu():
    lib = gcb.load_library()
    assert lib.wgrad_run(None, None, None, None, None, 0, None) == gcb.ERR_INVALID_ARG
    p = plan(workloads.CONFIGS["c1"])
    # NULL dw is rejected before anything touches the device
    assert lib.wgrad_run(p.handle, 16, 16, None, None, 0, None) == gcb.ERR_INVALID_ARG
    assert "dw" in gcb.wgrad_last_error()
    # misaligned pointers are rejected, not truncated
    assert lib.wgrad_run(p.handle, 18, 16, 16, None, 0, None) == gcb.ERR_INVALID_ARG
    assert "aligned" in gcb.wgrad_last_error()
    # a plan that needs a workspace refuses a missing or short one
    p2 = plan(workloads.CONFIGS["c2"])
    assert p2.workspace_bytes > 0
    assert lib.wgrad_run(p2.handle, 16, 16, 16, None, 0, None) == gcb.ERR_INVALID_ARG
    assert lib.wgrad_run(p2.handle, 16, 16, 16, 16, p2.workspace_bytes - 1, None) == gcb.ERR_INVALID_ARG
    assert "smaller" in gcb.wgrad_last_error()


def test_abi_struct_layouts_match_the_header(tmp_path):
    """The ctypes mirrors of wgrad_problem, wgrad_overrides and
    wgrad_plan_info have the sizes and field offsets a C compiler gives the
    header's structs."""
    import ctypes
    fields = {
        "wgrad_problem": gcb.wgrad_problem,
        "wgrad_overrides": gcb.wgrad_overrides,
        "wgrad_plan_info": gcb.wgrad_plan_info,
    }
    lines = ["#include <cstdio>", "#include <cstddef>", '#include "wgrad.h"', "int main() {"]
    for sname, cls in fields.items():
        lines.append(f'    printf("{sname} size %zu\\n", sizeof({sname}));')
        for fname, _ in cls._fields_:
            lines.append(f'    printf("{sname} {fname} %zu\\n", offsetof({sname}, {fname}));')
    lines += ["    return 0;", "}"]
    src = tmp_path / "layout.cpp"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["g++", "-std=c++17", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    got = {}
    for line in out:
        if line:
            parts = line.split()
            got[tuple(parts[:-1])] = int(parts[-1])
    for sname, cls in fields.items():
        assert got[(sname, "size")] == ctypes.sizeof(cls), sname
        for fname, _ in cls._fields_:
            assert got[(sname, fname)] == getattr(cls, fname).offset, (sname, fname)


def prob3(G, N, C, K, in_len, filt, stride=(1, 1, 1), pad=(0, 0, 0), dil=(1, 1, 1), dtype="bf16"):
    return {"ndim": 3, "G": G, "N": N, "C": C, "K": K, "in_len": in_len, "filt_len": filt,
            "stride": stride, "dilation": dil, "pad_lo": pad, "pad_hi": pad,
            "in_dtype": dtype, "out_dtype": dtype}


def test_3d_plans_sizes_and_kernels():
    import oracle
    cfg = prob3(1, 2, 64, 64, (6, 10, 12), (3, 3, 3), pad=(1, 1, 1))
    p = plan(cfg)
    ol = oracle.out_len(cfg)
    assert p.info["out_len"] == ol
    assert p.info["gemm_k"] == 2 * ol[0] * ol[1] * ol[2]
    assert p.info["gemm_n"] == 64 * 27 and p.info["gemm_m"] == 64
    assert p.info["variant"] == gcb.VARIANT_ROWSLAB
    # one row-slab tile per filter row (z, y): the grid is a multiple of 9
    assert p.info["grid_main"] % 9 == 0
    S = p.info["split_k"]
    assert p.workspace_bytes == (S * 64 * 27 * 64 * 4 if S > 1 else 0)
    assert p.dw_shape() == (64, 3, 3, 3, 64)
    # the flat MFMA kernel takes any 3D shape
    p = plan(cfg, variant=gcb.VARIANT_MFMA)
    assert p.info["variant"] == gcb.VARIANT_MFMA
    # depthwise 3D has no channel-vector kernel: it plans the MFMA kernel
    # with merged groups, and asking for the depthwise form is unsupported
    dw = prob3(32, 1, 32, 32, (4, 6, 6), (3, 3, 3), pad=(1, 1, 1))
    p = plan(dw)
    assert p.info["variant"] in (gcb.VARIANT_MFMA, gcb.VARIANT_ROWSLAB) and p.info["group_merge"] > 1
    _expect(gcb.ERR_UNSUPPORTED, dw, variant=gcb.VARIANT_DEPTHWISE)


def test_3d_invalid_problems_rejected():
    _expect(gcb.ERR_INVALID_ARG, prob3(1, 1, 8, 8, (2, 4, 4), (3, 1, 1)))          # empty depth output
    _expect(gcb.ERR_INVALID_ARG, prob3(1, 1, 8, 8, (4, 4, 4), (1, 1, 1), stride=(0, 1, 1)))
    _expect(gcb.ERR_INVALID_ARG, dict(prob3(1, 1, 8, 8, (4, 4, 4), (1, 1, 1)), ndim=4))


def test_size_products_cannot_wrap():
    # lengths and strides of 2^20 on three axes: X would hold 2^64 elements,
    # which wraps int64 to a small number if the product is formed unchecked
    big = prob3(1, 1, 16, 16, (2 ** 20,) * 3, (1, 1, 1), stride=(2 ** 20,) * 3)
    assert "31 bits" in _expect(gcb.ERR_INVALID_ARG, big)
    # single fields beyond 31 bits are rejected before any product
    assert "31 bits" in _expect(gcb.ERR_INVALID_ARG, prob3(1, 1, 16, 16, (4, 4, 2 ** 40), (1, 1, 1)))
    assert "31 bits" in _expect(gcb.ERR_INVALID_ARG, prob3(1, 1, 16, 16, (4, 4, 4), (1, 1, 1),
                                                         pad=(0, 0, 2 ** 62)))
    assert "31 bits" in _expect(gcb.ERR_INVALID_ARG, prob3(1, 2 ** 33, 16, 16, (4, 4, 4), (1, 1, 1)))


def test_row_slab_forms_reject_inputs_of_2_gib():
    # 3D: X of 4096*64*64*64 bf16 elements is exactly 2 GiB, which the
    # row-slab kernels' 32-bit byte offsets cannot address; the depth axis
    # counts toward that size
    cfg = prob3(1, 1, 64, 64, (4096, 64, 64), (3, 3, 3), pad=(1, 1, 1))
    p = plan(cfg)
    assert p.info["variant"] != gcb.VARIANT_ROWSLAB, p.name
    assert "2 GiB" in _expect(gcb.ERR_UNSUPPORTED, cfg, variant=gcb.VARIANT_ROWSLAB)
    # one depth slice less fits and takes the row-slab kernel
    small = prob3(1, 1, 64, 64, (4095, 64, 64), (3, 3, 3), pad=(1, 1, 1))
    assert plan(small).info["variant"] == gcb.VARIANT_ROWSLAB


def dplan(cfg, **kw):
    return gcb.DgradPlan(cfg, hip_device=-1, **kw)


def test_dgrad_plans_sizes_and_tiles():
    import oracle
    cfg = workloads.CONFIGS["c2"]
    p = dplan(cfg, tile=2)                    # the flat MFMA kernel (auto takes the row ring)
    info = p.info
    assert info["variant"] == gcb.VARIANT_DGRAD
    assert info["gemm_m"] == 32 * 56 * 56 and info["gemm_n"] == 64 and info["gemm_k"] == 64 * 9
    assert info["split_k"] == 1 and info["workspace_bytes"] == 0 and info["grid_reduce"] == 0
    assert (info["tile_m"], info["tile_n"], info["tile_k"]) == (128, 64, 32)
    assert info["grid_main"] == (32 * 56 * 56 + 127) // 128
    assert info["vector_width"] == 8 and p.name.startswith("dgrad_mfma_bf16")
    # grouped: one grid slice per group; odd channel runs narrow the loads
    g = prob3(4, 1, 4 * 6, 4 * 10, (3, 5, 7), (2, 3, 3), stride=(1, 2, 1), pad=(0, 1, 1))
    p = dplan(g, group_merge=1)
    assert p.info["vector_width"] == 2 and p.info["tile_n"] == 32
    # h-stride 2: two stride phases, each over a 3 x 3 x 7 phase grid
    assert p.info["grid_main"] == 2 * ((3 * 3 * 7 + 127) // 128) * 4
    assert dplan(g).info["group_merge"] == 4 and dplan(g).info["grid_main"] == 2
    assert p.info["out_len"] == oracle.out_len(g)
    # explicit tiles; 128-wide channel tiles for wide groups
    wide = dict(cfg, C=256)
    wide = dict(cfg, C=256, pad_lo=(2, 1), pad_hi=(2, 1))   # out of the row ring's reach
    assert dplan(wide).info["tile_n"] == 128
    assert dplan(wide, tile=2).info["tile_n"] == 64
    # small groups merge until both merged runs reach 32 channels
    p = dplan(workloads.CONFIGS["c4a"], tile=1)
    assert p.info["group_merge"] == 4 and p.info["tile_n"] == 32 and p.name.endswith("gm4")
    assert p.info["grid_main"] == ((32 * 28 * 28 + 127) // 128) * 8
    assert dplan(workloads.CONFIGS["c4a"], group_merge=8).info["group_merge"] == 8
    for bad in (3, 64):
        with pytest.raises(gcb.WgradError):
            dplan(workloads.CONFIGS["c4a"], group_merge=bad)
    # depthwise shapes take the direct kernels; forcing them elsewhere is unsupported
    # 3x3 unit stride, C a multiple of 256: the tile form, 14 x 28 dX tiles of
    # 256 channels, 16 x 4 x 2 x 2 = 256 tiles, one per workgroup
    p = dplan(workloads.CONFIGS["c5"])
    assert p.info["tile"] == 7 and p.name == "dgrad_dwtile_bf16_t14x28" and p.info["grid_main"] == 256
    # more tiles than CUs: taller tiles first, then several per workgroup
    p = dplan(dict(workloads.CONFIGS["c5"], N=64))
    assert p.info["tile"] == 7 and p.info["grid_main"] == 256 and p.name.endswith("_t56x28")
    # C not a multiple of 256: the row-walking form
    assert dplan(dict(workloads.CONFIGS["c5"], G=96, C=96, K=96)).info["tile"] == 4
    with pytest.raises(gcb.WgradError) as e:
        dplan(dict(workloads.CONFIGS["c5"], G=96, C=96, K=96), tile=7)
    assert e.value.code == gcb.ERR_UNSUPPORTED
    # the row-walking form on c5: 256-channel blocks of 4-channel lanes, 4
    # strips per workgroup, row chunks per strip from the planner
    p = dplan(workloads.CONFIGS["c5"], tile=4)
    assert p.info["tile"] == 4 and p.name.startswith("dgrad_dwring") and p.info["tile_n"] == 256
    nch = int(p.name.rsplit("_ch", 1)[1])
    assert p.info["grid_main"] == 2 * ((16 * 14 * nch + 3) // 4)
    # the per-tap form: 512-channel blocks of 8-channel lanes, one strip of a row each
    p5 = dplan(workloads.CONFIGS["c5"], tile=5)
    assert p5.info["tile"] == 5 and p5.info["tile_n"] == 512
    assert p5.info["grid_main"] == (16 * 56 * 14 + 3) // 4
    assert dplan(workloads.CONFIGS["c5"], tile=1).info["tile"] == 1
    assert dplan(dict(workloads.CONFIGS["c5"], G=24, C=24, K=24)).info["tile_n"] == 8
    # strided depthwise keeps the per-tap form
    assert dplan(dict(workloads.CONFIGS["c5"], stride=(2, 2))).info["tile"] == 5
    with pytest.raises(gcb.WgradError) as e:
        dplan(cfg, tile=4)
    assert e.value.code == gcb.ERR_UNSUPPORTED
    # stride phases: one grid slice per phase; strides above 16 are refused
    p = dplan(workloads.CONFIGS["c3"])
    assert p.info["grid_main"] == 4 * ((16 * 28 * 28 + 127) // 128) * (128 // p.info["tile_n"])
    with pytest.raises(gcb.WgradError) as e:
        dplan(dict(cfg, stride=(17, 1), in_len=(70, 56)))
    assert e.value.code == gcb.ERR_UNSUPPORTED
    # the fp16 strided shape, fp32 output
    p = dplan(dict(workloads.CONFIGS["c3"], out_dtype="fp32"))
    assert p.info["gemm_m"] == 16 * 56 * 56 and p.info["gemm_k"] == 200 * 9 and "fp16" in p.name


def test_dgrad_plan_rejections_and_plan_kinds():
    lib = gcb.load_library()
    cfg = workloads.CONFIGS["c2"]
    for kw in ({"split_k": 2}, {"group_merge": 2}, {"variant": gcb.VARIANT_MFMA}, {"tile": 9}):
        with pytest.raises(gcb.WgradError) as e:
            dplan(cfg, **kw)
        assert e.value.code == gcb.ERR_UNSUPPORTED
    with pytest.raises(gcb.WgradError) as e:
        plan(cfg, variant=gcb.VARIANT_DGRAD)
    assert e.value.code == gcb.ERR_UNSUPPORTED
    with pytest.raises(gcb.WgradError) as e:
        dplan(dict(cfg, G=2, C=63))   # C not a multiple of G
    assert e.value.code == gcb.ERR_INVALID_ARG
    d, w = dplan(cfg), plan(cfg)
    # each run entry point refuses the other direction's plan
    assert lib.wgrad_dgrad_run(w.handle, 16, 16, 16, None) == gcb.ERR_INVALID_ARG
    assert "backward-data" in gcb.wgrad_last_error()
    assert lib.wgrad_run(d.handle, 16, 16, 16, None, 0, None) == gcb.ERR_INVALID_ARG
    assert lib.wgrad_dgrad_run(None, 16, 16, 16, None) == gcb.ERR_INVALID_ARG
    assert lib.wgrad_dgrad_run(d.handle, 16, 16, None, None) == gcb.ERR_INVALID_ARG
    assert lib.wgrad_dgrad_run(d.handle, 16, 24, 16, None) == gcb.ERR_INVALID_ARG
    assert "aligned" in gcb.wgrad_last_error()
    # an empty batch enqueues nothing and accepts NULL pointers
    e = dplan(dict(cfg, N=0))
    assert e.info["grid_main"] == 0
    assert lib.wgrad_dgrad_run(e.handle, None, None, None, None) == gcb.OK


def test_ring_form_plans():
    # the grouped 3x3 workload takes the filter-row ring form: one workgroup
    # per (group block, M block, 32-channel block) and split, all nine taps
    c4a = workloads.CONFIGS["c4a"]
    p = plan(c4a)
    assert p.info["variant"] == gcb.VARIANT_ROWSLAB and p.info["tile"] == 2
    assert p.name.startswith("wgrad_ring_bf16_m32c32x3x3") and p.name.endswith("gm4")
    Gm, S = p.info["group_merge"], p.info["split_k"]
    assert Gm == 4 and p.info["tile_n"] == 9 * 32
    assert p.info["grid_main"] == (c4a["G"] // Gm) * S
    rows = c4a["N"] * p.info["out_len"][0]
    rpw = -(-rows // S)
    assert -(-rows // rpw) == S and S <= 256
    assert p.workspace_bytes == S * c4a["K"] * 9 * (c4a["C"] // c4a["G"]) * 4
    # the one-filter-row form is still there by request
    p1 = plan(c4a, variant=gcb.VARIANT_ROWSLAB, tile=1)
    assert p1.info["tile"] == 0 and p1.name.startswith("wgrad_rowslab_")
    # dense shapes keep one filter row per workgroup unless asked
    c2 = workloads.CONFIGS["c2"]
    assert plan(c2).name.startswith("wgrad_rowslab_")
    p2 = plan(c2, variant=gcb.VARIANT_ROWSLAB, tile=2)
    assert p2.name.startswith("wgrad_ring_bf16_m64c32") and p2.info["grid_main"] == 2 * p2.info["split_k"]
    # stride 2 in w picks a stride-2 row tile; the split never exceeds the rows
    p3 = plan(workloads.CONFIGS["c3"], variant=gcb.VARIANT_ROWSLAB, tile=2)
    assert "_s2x2_" in p3.name
    assert plan(c4a, variant=gcb.VARIANT_ROWSLAB, tile=2, split_k=10 ** 6).info["split_k"] == rows


def test_ring_form_rejections():
    c4a = workloads.CONFIGS["c4a"]
    ring = dict(variant=gcb.VARIANT_ROWSLAB, tile=2)
    _expect(gcb.ERR_UNSUPPORTED, workloads.CONFIGS["c4b"], **ring)                  # 1D
    _expect(gcb.ERR_UNSUPPORTED, workloads.get("pw"), **ring)                       # 1x1 filter
    _expect(gcb.ERR_UNSUPPORTED, workloads.problem(c4a, dilation=(2, 1)), **ring)   # dilation
    _expect(gcb.ERR_UNSUPPORTED, workloads.problem(c4a, stride=(1, 3)), **ring)     # w-stride 3
    _expect(gcb.ERR_UNSUPPORTED, workloads.problem(c4a, stride=(4, 1)), **ring)     # h-stride 4
    _expect(gcb.ERR_UNSUPPORTED, workloads.problem(c4a, in_len=(28, 100)), **ring)  # rows wider than 62
    _expect(gcb.ERR_UNSUPPORTED, workloads.CONFIGS["c5"], **ring)                   # 1-channel groups
    _expect(gcb.ERR_UNSUPPORTED, c4a, variant=gcb.VARIANT_ROWSLAB, tile=3)
    # where the ring form does not apply, auto falls back to one filter row per workgroup
    assert plan(workloads.problem(c4a, in_len=(28, 100))).name.startswith("wgrad_rowslab_")


def test_dgrad_ring_form_plans():
    def dplan(cfg, **kw):
        return gcb.DgradPlan(cfg, hip_device=-1, **kw)
    # the dense and grouped 3x3 unit-stride workloads take the row-ring form
    p = dplan(workloads.CONFIGS["c2"])
    assert p.info["tile"] == 6 and p.name.startswith("dgrad_ring_bf16_m2x32_n64_k64")
    rows = 32 * (56 + 2)
    vpw = int(p.name.split("_v")[1].split("_")[0])
    assert vpw % 4 == 0 and p.info["grid_main"] == -(-rows // vpw) and p.info["grid_main"] <= 256
    p = dplan(workloads.CONFIGS["c4a"])
    assert p.info["tile"] == 6 and p.info["group_merge"] == 4 and p.name.endswith("gm4")
    # shapes it does not take fall back to the flat MFMA kernel, or fail when asked for
    for bad in (workloads.problem("c2", pad_lo=(2, 1), pad_hi=(2, 1)),     # Ho > Hi
                workloads.problem("c2", in_len=(56, 70)),                  # rows wider than 64
                workloads.CONFIGS["c3"], workloads.CONFIGS["c1"]):
        assert dplan(bad).info["tile"] in (1, 2, 3)
        with pytest.raises(gcb.WgradError):
            dplan(bad, tile=6)


def test_build_guard_rejects_scratch_in_counted_load_kernels():
    """build.py fails the build when a kernel in a source file that issues
    counted direct-to-LDS loads uses scratch memory or a dynamic stack: its
    exact vmcnt waits would then be short."""
    from grouped_convolution_backward_amd import build as b
    for f in ("rowslab.hip", "ring.hip", "dgrad_ring.hip"):
        assert b.uses_counted_lds_loads(f), f
    assert not b.uses_counted_lds_loads("plan.cpp")

    def remarks(name, scratch, dyn):
        return (f"x.hip:1:1: remark: Function Name: {name} [-Rpass-analysis=kernel-resource-usage]\n"
                f"x.hip:1:1: remark:     VGPRs: 90 [-Rpass-analysis=kernel-resource-usage]\n"
                f"x.hip:1:1: remark:     ScratchSize [bytes/lane]: {scratch} [-Rpass-analysis=kernel-resource-usage]\n"
                f"x.hip:1:1: remark:     Dynamic Stack: {dyn} [-Rpass-analysis=kernel-resource-usage]\n")
    clean = remarks("k0", 0, "False") + remarks("k1", 0, "False")
    assert b.scratch_violations(clean) == []
    assert b.scratch_violations(clean + remarks("k2", 16, "False")) == [("k2", 16, "False")]
    assert b.scratch_violations(remarks("k3", 0, "True") + clean) == [("k3", 0, "True")]


def test_missing_library_fails_loudly(tmp_path):
    """Without libwgrad.so the package raises instead of computing anything
    another way: a fresh interpreter whose package copy has no library."""
    import shutil
    import sys
    pkg = os.path.dirname(gcb.__file__)
    dst = tmp_path / "grouped_convolution_backward_amd"
    shutil.copytree(pkg, dst, ignore=shutil.ignore_patterns("*.so", "_build", "__pycache__"))
    root = os.path.dirname(pkg)
    code = ("import grouped_convolution_backward_amd as g, workloads\n"
            "try:\n"
            "    g.Plan(workloads.get('c2'), hip_device=-1)\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n"
            "else:\n"
            "    print('no error')\n")
    env = dict(os.environ, PYTHONPATH=os.pathsep.join([str(tmp_path), root]))
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, cwd=str(tmp_path),
                         timeout=120)
    assert out.returncode == 0, out.stderr
    assert "raised:" in out.stdout and "is not built" in out.stdout, out.stdout
