"""Host-side parts of bench.py: the one-GPU guard, the algorithmic work of
the headline workload, the kernel-source hashing that keys the committed
traffic records, and the rule that a traffic record counts only for the
plan and sources it was taken on. No GPU is touched."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_algorithmic_work_of_the_dense_workload():
    # 2*G*(K/G)*(C/G)*Y*X*N*Ho*Wo and |X| + |dY| + |dW| for N=32 56x56 C=K=64 3x3
    cfg = workloads.get("c2")
    flops, nbytes = bench.algorithmic(cfg, {"gemm_k": 32 * 56 * 56})
    assert flops == 2 * 64 * 64 * 9 * 32 * 56 * 56 == 7_398_752_256
    assert nbytes == 12_845_056 + 12_845_056 + 73_728


def test_algorithmic_bytes_count_fp32_output():
    cfg = dict(workloads.get("c1"), out_dtype="fp32")
    _, nbytes = bench.algorithmic(cfg, {"gemm_k": 64})
    assert nbytes == 2 * (8 * 8 * 16) + 2 * (64 * 32) + 4 * 32 * 9 * 16


@pytest.mark.parametrize("plan,own", [
    ("wgrad_rowslab_bf16_m64c64x3_k32_slab1x32_kouter_spk82_gm1", "rowslab.hip"),
    ("wgrad_ring_bf16_m32c32x3x3_k32_w32_s1x1_kouter_spk32_gm4", "ring.hip"),
    ("dgrad_ring_bf16_m2x32_n64_k64_v8_gm1", "dgrad_ring.hip"),
    ("dgrad_mfma_fp16_t2_128x64x32_v8_kouterB_gm1", "dgrad.hip"),
])
def test_source_hash_follows_the_kernel_family(plan, own, tmp_path, monkeypatch):
    """The hash changes with the family's own source and with the shared
    headers, and not with another family's source."""
    csrc = tmp_path / "grouped_convolution_backward_amd" / "csrc"
    csrc.mkdir(parents=True)
    names = {f for _, f in bench._FAMILY_SOURCES} | set(bench._SHARED_SOURCES)
    for f in names:
        (csrc / f).write_text(f"// {f}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash(plan)
    other = next(f for f in sorted(names - {own} - set(bench._SHARED_SOURCES)))
    (csrc / other).write_text("// changed\n")
    assert bench.kernel_source_hash(plan) == h0
    (csrc / own).write_text("// changed\n")
    h1 = bench.kernel_source_hash(plan)
    assert h1 != h0
    (csrc / "device_common.hpp").write_text("// changed\n")
    assert bench.kernel_source_hash(plan) != h1


def test_traffic_record_needs_same_plan_and_sources(tmp_path, monkeypatch):
    plan = "wgrad_rowslab_bf16_m64c64x3_k32_slab1x32_kouter_spk82_gm1"
    (tmp_path / "profiles").mkdir()
    csrc = tmp_path / "grouped_convolution_backward_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in {f for _, f in bench._FAMILY_SOURCES} | set(bench._SHARED_SOURCES):
        (csrc / f).write_text(f"// {f}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    rec = {"c2": {"kernel": plan, "source_hash": bench.kernel_source_hash(plan), "bytes_per_launch": 123}}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("c2", plan) == 123
    assert bench.measured_traffic("c2", plan.replace("spk82", "spk41")) is None
    assert bench.measured_traffic("c3", plan) is None
    (csrc / "rowslab.hip").write_text("// edited kernel\n")
    assert bench.measured_traffic("c2", plan) is None


def test_mfma_counter_record_needs_same_plan_and_sources(tmp_path, monkeypatch):
    plan = "wgrad_rowslab_bf16_m64c64x3_k32_slab1x32_kouter_spk82_gm1"
    (tmp_path / "profiles").mkdir()
    csrc = tmp_path / "grouped_convolution_backward_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in {f for _, f in bench._FAMILY_SOURCES} | set(bench._SHARED_SOURCES):
        (csrc / f).write_text(f"// {f}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    rec = {"c2": {"kernel": plan, "source_hash": bench.kernel_source_hash(plan), "mfma_insts": 258048,
                  "useful_frac": 0.875, "busy_frac_of_simd_cycles": 0.24, "other": 1}}
    (tmp_path / "profiles" / "mfma_counters.json").write_text(json.dumps(rec))
    got = bench.measured_mfma("c2", plan)
    assert got == {"mfma_insts": 258048, "useful_frac": 0.875, "busy_frac_of_simd_cycles": 0.24}
    assert bench.measured_mfma("c2", plan.replace("spk82", "spk41")) is None
    (csrc / "rowslab.hip").write_text("// edited kernel\n")
    assert bench.measured_mfma("c2", plan) is None


def test_dense_workloads_are_reported_against_mfma():
    # the dense split-K shape sits just under the ridge (HBM floor 3.22 us,
    # MFMA floor 2.96 us) but is a dense contraction: reported against MFMA
    cfg = workloads.get("c2")
    flops, nbytes = bench.algorithmic(cfg, {"gemm_k": 32 * 56 * 56})
    assert flops / bench.PEAK_MFMA_16 < nbytes / bench.PEAK_HBM
    assert bench.reported_bound("c2", flops, nbytes) == "mfma"
    assert bench.reported_bound("dgrad:c3", flops, nbytes) == "mfma"
    cfg5 = workloads.get("c5")
    f5, b5 = bench.algorithmic(cfg5, {"gemm_k": 16 * 56 * 56})
    assert bench.reported_bound("c5", f5, b5) == "hbm"


def test_median_of_even_and_odd_counts():
    assert bench._median([3.0, 1.0, 2.0]) == 2.0
    assert bench._median([4.0, 1.0, 3.0, 2.0]) == 2.5


def _counter_csv(path, dispatches):
    import csv
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Correlation_Id", "Dispatch_Id", "Agent_Id", "Grid_Size", "Kernel_Name", "Workgroup_Size",
                    "Counter_Name", "Counter_Value"])
        for i, (kernel, wgs, wg_size, counters) in enumerate(dispatches):
            for name, val in counters.items():
                w.writerow([i + 1, i + 1, 1, wgs * wg_size, kernel, wg_size, name, val])


def test_counter_ingestion_finds_main_kernels_and_scales_by_the_copy(tmp_path, monkeypatch):
    """traffic.json and mfma_counters.json from rocprofv3 counter CSVs: the
    main kernel is found by function and workgroup count (a dgrad kernel of
    a similar name and a dispatch of another grid are ignored), FETCH_SIZE is
    scaled by what it reads for the 256 MiB copy, MFMA fractions follow from
    the counts."""
    import grouped_convolution_backward_amd as gcb
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", ROOT)
    p2 = gcb.Plan(workloads.get("c2"), hip_device=-1)
    p4 = gcb.Plan(workloads.get("c4a"), hip_device=-1)
    g2, g4 = p2.info["grid_main"], p4.info["grid_main"]
    assert bench.kernel_fn(p2.name) == "rowslab_kernel" and bench.kernel_fn(p4.name) == "ring_kernel"
    rs = "void wgrad::(anonymous namespace)::rowslab_kernel<64, 64, 3>(wgrad::RowSlabArgs)"
    ring = "void wgrad::(anonymous namespace)::ring_kernel<32, 2>(wgrad::RingArgs)"
    dring = "void wgrad::(anonymous namespace)::dgrad_ring_kernel<1>(wgrad::DgradRingArgs)"
    neg = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>(int)"
    # FETCH_SIZE reads half the true bytes here: the copy of 256 MiB reads 131072 KiB
    fetch = tmp_path / "fetch.csv"
    _counter_csv(fetch, [(neg, 4096, 256, {"FETCH_SIZE": 131072.0}),
                         (rs, g2, 768, {"FETCH_SIZE": 13000.0}), (rs, g2, 768, {"FETCH_SIZE": 15000.0}),
                         (rs, g2 + 8, 768, {"FETCH_SIZE": 99999.0}),
                         (dring, g4, 320, {"FETCH_SIZE": 77777.0}), (ring, g4, 320, {"FETCH_SIZE": 12000.0})])
    write = tmp_path / "write.csv"
    _counter_csv(write, [(neg, 4096, 256, {"WRITE_SIZE": 262144.0}), (rs, g2, 768, {"WRITE_SIZE": 11808.0}),
                         (ring, g4, 320, {"WRITE_SIZE": 2304.0})])
    flops2, _ = bench.algorithmic(workloads.get("c2"), p2.info)
    mf = tmp_path / "mfma.csv"
    _counter_csv(mf, [(rs, g2, 768, {"SQ_INSTS_MFMA": 258048.0, "SQ_INSTS_VALU_MFMA_MOPS_BF16": flops2 / 512 / 0.875,
                                    "SQ_VALU_MFMA_BUSY_CYCLES": 8257536.0, "SQ_BUSY_CU_CYCLES": 7805507.0})])
    traffic, mfma = bench.ingest_counters([("c2", str(fetch)), ("c4a", str(fetch)), ("c2", str(write)),
                                           ("c4a", str(write)), ("c2", str(mf))], out_dir=str(tmp_path / "profiles"))
    t = json.loads((tmp_path / "profiles" / "traffic.json").read_text())
    assert t["c2"]["fetch_bytes"] == 14000 * 1024 * 2 and t["c2"]["write_bytes"] == 11808 * 1024
    assert t["c2"]["bytes_per_launch"] == t["c2"]["fetch_bytes"] + t["c2"]["write_bytes"]
    assert t["c4a"]["fetch_bytes"] == 12000 * 1024 * 2
    assert t["c2"]["source_hash"] == bench.kernel_source_hash(p2.name) and t["c2"]["kernel"] == p2.name
    m = json.loads((tmp_path / "profiles" / "mfma_counters.json").read_text())["c2"]
    assert m["mfma_insts"] == 258048 and m["useful_frac"] == 0.875
    assert m["busy_frac_of_simd_cycles"] == round(8257536.0 / (4 * 7805507.0), 4)
    with pytest.raises(ValueError):
        bench.ingest_counters([("c3", str(fetch))], out_dir=str(tmp_path / "profiles"))


def test_every_benchmarked_plan_maps_to_its_kernel_and_sources():
    """The trace and counter summaries find each workload's main kernel by
    the function its plan name maps to, and traffic records are keyed by
    that kernel's source files: every plan the bench runs (both directions)
    must map to both."""
    import grouped_convolution_backward_amd as gcb
    for name in list(workloads.CONFIGS) + list(workloads.WIDER):
        cfg = workloads.get(name)
        for plan in (gcb.Plan(cfg, hip_device=-1), gcb.DgradPlan(cfg, hip_device=-1)):
            fn = bench.kernel_fn(plan.name)
            assert fn.endswith("_kernel"), (name, plan.name, fn)
            assert [f for pre, f in bench._FAMILY_SOURCES if plan.name.startswith(pre)], plan.name
    # the depthwise forms bench.py reaches through overrides
    c5 = workloads.get("c5")
    for tile, fn in ((3, "dw3_kernel"), (4, "dwtile_kernel")):
        assert bench.kernel_fn(gcb.Plan(c5, hip_device=-1, variant=gcb.VARIANT_DEPTHWISE, tile=tile).name) == fn
    for tile, fn in ((4, "dgrad_dw_ring_kernel"), (7, "dgrad_dwtile_kernel")):
        assert bench.kernel_fn(gcb.DgradPlan(c5, hip_device=-1, tile=tile).name) == fn
