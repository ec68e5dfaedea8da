"""Benchmark of grouped convolution backward-weight (wgrad) on one MI355X,
with backward-data (dgrad) rows beside it.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--configs c2,c5,...]

One step is one pass of the whole path (the main kernel, plus the reduce /
convert kernel when the plan splits the reduction) over one batch of
synthetic, seeded input already resident in HBM. The headline workload is
the dense split-K shape (G=1 N=32 56x56 C=64 K=64 3x3 s1 p1, bf16): value =
its TFLOP/s over exactly K timed steps. Every other configuration is timed
the same way and reported under "per_config"; "dgrad:<name>" rows time
backward data (dX from dY and W) of that workload's convolution.

Every workload does its W warmup steps, then its K timed steps: captured in
HIP graphs (up to 512 steps per graph, cycling through the input copies),
replayed untimed for 0.3 s (graph upload, and the GPU clocks back at their
loaded state after the host has built the workload's inputs), then replayed
with HIP events recorded on the replay stream around exactly K steps, behind
a short GPU spin so that the host's graph submission is not on the clock;
torch.cuda.synchronize() on both sides. Neither the host's launch rate nor
a graph replay's own start-up sets the time.

Honest memory: each configuration cycles through enough copies of its inputs
(> 512 MB in total) that no step finds its inputs in the 256 MB MALL left
behind by the previous steps.

Dominant-kernel roofline: the per-launch duration of the main kernel comes
from HIP events recorded on the launch stream around replays of a graph that
holds only wgrad_run_stage(1) launches (at least 64, cycling through the
input sets), divided by the launch count; achieved = algorithmic FLOPs or bytes per launch / that
duration. traffic = HBM bytes per launch from committed rocprofv3 FETCH_SIZE
and WRITE_SIZE runs, each scaled by what the counter reads for a plain
device copy of known size (--copy-calibration), when they were taken on the
current kernel sources.

Per configuration, beside the graph-replayed steady state (us_per_step):
* "iters": 10 warmup calls, then 50 timed calls of the whole path, each
  bracketed by HIP events on the launch stream, with a 512 MiB fill kernel
  between calls (outside the events) so that no call finds its inputs or
  workspace in the L2 or the 256 MB MALL; median and min in us;
* "hot": the same 50 events-bracketed calls with no fill in between (inputs
  and workspace warm in the caches), labelled as such;
* MFMA counters of the main kernel from the committed rocprofv3 record
  profiles/mfma_counters.json, when it was taken on the same plan and
  kernel sources (else null);
* "cpu_oracle_s": the CPU oracle's wall time for the full dW of that
  configuration on this host, with its thread count.

cpu_baseline: the CPU oracle (fp64 direct loop, OpenMP) over the full
headline dW, timed on this host.

Roofline bound: the dense configurations (the dense split-K shape and the
strided fp16 shape, and the 3D dense shape) are reported against MFMA throughput,
the others on HBM bandwidth where their arithmetic intensity puts them;
the headline roofline block also carries the HBM fraction of the same
kernel and the MFMA and HBM fractions of the whole step.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_16 = 2.5e15     # dense bf16/fp16 MFMA, FLOP/s
PEAK_HBM = 8.0e12         # HBM3E, B/s
METRIC = "wgrad TFLOP/s (GB/s for depthwise) and % of roofline, 1 MI355X"
HEADLINE = "c2"
ROTATE_BYTES = 600 * 2 ** 20
GRAPH_MIN_LAUNCHES = 64
MAX_GRAPH = 512           # steps per captured graph in the timed region
FLUSH_BYTES = 512 * 2 ** 20
ITER_WARMUP, ITER_TIMED = 10, 50
# workloads reported against MFMA throughput whatever their exact arithmetic
# intensity (the dense contractions); the others by intensity
DENSE = ("c2", "c3", "c3d")


def reported_bound(name, flops, nbytes):
    if name.split(":")[-1] in DENSE:
        return "mfma"
    return "mfma" if flops / PEAK_MFMA_16 >= nbytes / PEAK_HBM else "hbm"


def algorithmic(cfg, info):
    """FLOPs = 2*G*(K/G)*(C/G)*Y*X*N*Ho*Wo; bytes = |X| + |dY| + |dW|, each once."""
    G = cfg["G"]
    taps = 1
    for f in cfg["filt_len"][: cfg["ndim"]]:
        taps *= f
    R = info["gemm_k"]
    flops = 2 * G * (cfg["K"] // G) * (cfg["C"] // G) * taps * R
    nx = cfg["N"] * math.prod(cfg["in_len"][: cfg["ndim"]]) * cfg["C"]
    ndy = R * cfg["K"]
    out_bytes = 4 if cfg["out_dtype"] == "fp32" else 2
    nbytes = 2 * (nx + ndy) + out_bytes * cfg["K"] * taps * (cfg["C"] // G)
    return flops, nbytes


# the source files each kernel family is built from (besides the shared
# device helpers and argument headers); a traffic record is valid only for
# the exact bytes of these files
_FAMILY_SOURCES = (("wgrad_rowslab", "rowslab.hip"), ("wgrad_ring", "ring.hip"), ("wgrad_mfma", "kernels.hip"),
                   ("wgrad_dwtile", "dwtile.hip"), ("wgrad_dw", "depthwise.hip"), ("dgrad_ring", "dgrad_ring.hip"),
                   ("dgrad_dwtile", "dwtile.hip"), ("dgrad_", "dgrad.hip"))
_SHARED_SOURCES = ("device_common.hpp", "wgrad_internal.hpp", "dgrad_internal.hpp", "magic.hpp")


def kernel_source_hash(plan_name):
    """Hash of the sources the named plan's main kernel is compiled from."""
    own = [f for pre, f in _FAMILY_SOURCES if plan_name.startswith(pre)][:1]
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "grouped_convolution_backward_amd", "csrc")
    for f in sorted(own + list(_SHARED_SOURCES)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, plan_name):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the same plan (kernel, split, merge) built from the current
    sources of its kernel (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
        e = t[workload]
        if e.get("kernel") != plan_name or e.get("source_hash") != kernel_source_hash(plan_name):
            return None
        return e["bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def measured_mfma(workload, plan_name):
    """MFMA counters of the workload's main kernel from the committed
    rocprofv3 record (profiles/mfma_counters.json), if taken on the same
    plan built from the current sources of its kernel (else None)."""
    path = os.path.join(ROOT, "profiles", "mfma_counters.json")
    try:
        with open(path) as f:
            t = json.load(f)
        e = t[workload]
        if e.get("kernel") != plan_name or e.get("source_hash") != kernel_source_hash(plan_name):
            return None
        return {k: e[k] for k in ("mfma_insts", "useful_frac", "mfma_busy_cycles", "busy_frac_of_simd_cycles",
                                  "launch_us") if k in e}
    except (OSError, KeyError, ValueError):
        return None


# plan-name prefix -> the main kernel's function (longer prefixes first)
_KERNEL_FN = (("wgrad_rowslab_", "rowslab_kernel"), ("wgrad_ring_", "ring_kernel"), ("wgrad_mfma_", "mfma_kernel"),
              ("wgrad_dwtile_", "dwtile_kernel"), ("wgrad_dwstrip_", "dw3_kernel"), ("wgrad_dwwin_", "dw2_kernel"),
              ("wgrad_dw_", "dw_kernel"),
              ("dgrad_ring_", "dgrad_ring_kernel"), ("dgrad_dwtile_", "dgrad_dwtile_kernel"),
              ("dgrad_dwring_", "dgrad_dw_ring_kernel"),
              ("dgrad_dw_", "dgrad_dw_kernel"), ("dgrad_mfma_", "dgrad_kernel"))
COPY_BYTES = 256 * 2 ** 20   # --copy-calibration: torch.neg over this many bytes, read and written


def kernel_fn(plan_name):
    for pre, fn in _KERNEL_FN:
        if plan_name.startswith(pre):
            return fn
    raise ValueError(plan_name)


def _kernel_parts(name):
    """(function, template arguments) of a demangled kernel name."""
    import re
    name = name.replace("(anonymous namespace)", "")
    cut = min([i for i in (name.find("<"), name.find("(")) if i >= 0] or [len(name)])
    fn = re.split(r"[\s:]+", name[:cut].strip())[-1]
    targs = ""
    if "<" in name:
        depth, start = 0, name.index("<")
        for i in range(start, len(name)):
            depth += name[i] == "<"
            depth -= name[i] == ">"
            if depth == 0:
                targs = name[start:i + 1]
                break
    return fn, targs


def _targs_match(plan_name, targs):
    """Row-slab and ring kernels: the template arguments start with the M
    block, C block and (row slab) filter width the plan name states."""
    import re
    m = re.search(r"_m(\d+)c(\d+)x(\d+)", plan_name)
    if not m or not plan_name.startswith(("wgrad_rowslab_", "wgrad_ring_")):
        return True
    want = [m.group(1)] if plan_name.startswith("wgrad_ring_") else [m.group(1), m.group(2), m.group(3)]
    got = [x.strip() for x in targs.strip("<>").split(",")]
    return got[:len(want)] == want


def summarize_trace(path, names):
    """Markdown table of the main and reduce kernels of each workload from a
    rocprofv3 kernel-trace CSV: dispatches matched by kernel function and
    workgroup count (from the host plans), with their count and mean,
    median and min duration. For split-K workloads the main kernel's
    dispatches are also split by what runs next: its own reduce (whole
    steps) or another main launch (the stage-only replays that
    roofline.kernel_us is measured on)."""
    import csv
    import grouped_convolution_backward_amd as gcb
    import workloads
    disp = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            gx = int(r.get("Grid_Size_X") or r.get("Grid_Size"))
            wx = int(r.get("Workgroup_Size_X") or r.get("Workgroup_Size"))
            fn, targs = _kernel_parts(r["Kernel_Name"])
            t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
            disp.append((fn, targs, gx // max(1, wx), (t1 - t0) / 1e3, t0, t1))
    disp.sort(key=lambda d: d[4])
    following = {id(d): disp[i + 1] if i + 1 < len(disp) else None for i, d in enumerate(disp)}
    lines = ["| workload | plan | kernel | workgroups | dispatches | mean us | median us | min us |",
             "|---|---|---|---|---|---|---|---|"]
    for name in names:
        dgrad = name.startswith("dgrad:")
        cfg = workloads.get(name.split(":", 1)[-1])
        plan = (gcb.DgradPlan if dgrad else gcb.Plan)(cfg, hip_device=-1)
        fn = kernel_fn(plan.name)
        main = [d for d in disp if d[0] == fn and d[2] == plan.info["grid_main"] and _targs_match(plan.name, d[1])]
        parts = [(fn, plan.info["grid_main"], main)]
        if plan.info["split_k"] > 1 and not dgrad and main:
            # the reduce launches of this workload: inside the time span of its main launches
            lo, hi = min(d[4] for d in main), max(d[5] for d in main)
            red = [d for d in disp if d[0] == "reduce_kernel" and d[2] == plan.info["grid_reduce"] and lo <= d[4] <= hi]
            parts.append(("reduce_kernel", plan.info["grid_reduce"], red))
            nxt = lambda d: following[id(d)]
            in_steps = [d for d in main if nxt(d) is not None and nxt(d)[0] == "reduce_kernel"]
            alone = [d for d in main if nxt(d) is not None and nxt(d)[0] == fn and nxt(d)[2] == d[2]]
            parts.insert(1, (fn, plan.info["grid_main"], in_steps, " (followed by its reduce: steps)"))
            parts.insert(2, (fn, plan.info["grid_main"], alone, " (followed by another main launch)"))
        for part in parts:
            fn, wgs, sel = part[:3]
            note = part[3] if len(part) > 3 else ""
            if not sel:
                lines.append(f"| {name} | `{plan.name}` | `{fn}`{note} | {wgs} | 0 | | | |")
                continue
            t = sorted(d[3] for d in sel)
            targs = sorted({d[1] for d in sel})
            lines.append(f"| {name} | `{plan.name}` | `{fn}{targs[0] if len(targs) == 1 else ''}`{note} | {wgs} | "
                         f"{len(t)} | {sum(t) / len(t):.2f} | {t[len(t) // 2]:.2f} | {t[0]:.2f} |")
    return "\n".join(lines)


def read_counter_csv(path):
    """Dispatches of a rocprofv3 counter-collection CSV: a list of
    {"kernel", "wgs", "counters": {name: value}} in dispatch order (one row
    per dispatch and counter in the file)."""
    import csv
    rows = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            grid = int(r.get("Grid_Size") or r.get("Grid_Size_X"))
            wgsz = int(r.get("Workgroup_Size") or r.get("Workgroup_Size_X"))
            d = rows.setdefault(int(r["Dispatch_Id"]), {
                "kernel": r["Kernel_Name"], "wgs": grid // max(1, wgsz), "counters": {},
                "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) if r.get("End_Timestamp") else 0})
            name = r["Counter_Name"]
            d["counters"][name] = d["counters"].get(name, 0.0) + float(r["Counter_Value"])
    return [rows[k] for k in sorted(rows)]


def _calls(dispatches, fn, wgs, plan_name=""):
    out = []
    for d in dispatches:
        kfn, targs = _kernel_parts(d["kernel"])
        if kfn == fn and d["wgs"] == wgs and _targs_match(plan_name, targs):
            out.append(d)
    return out


def ingest_counters(pairs, out_dir=None):
    """Build profiles/traffic.json and profiles/mfma_counters.json from
    rocprofv3 counter CSVs: pairs of (workload, csv path). Each workload's
    main-kernel dispatches are found by kernel function and workgroup count
    (from the host plan) and averaged. FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch) are scaled by what they read for the copy-calibration kernel
    (torch neg over COPY_BYTES) in the same file; MFMA counters are kept as
    read, with the useful fraction 2*M*N*R / (MOPS * 512) and the busy
    fraction MFMA-busy cycles / (4 SIMDs * CU-busy cycles)."""
    import grouped_convolution_backward_amd as gcb
    import workloads
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    traffic, mfma = {}, {}
    for workload, path in pairs:
        disp = read_counter_csv(path)
        dgrad = workload.startswith("dgrad:")
        cfg = workloads.get(workload.split(":", 1)[-1])
        plan = (gcb.DgradPlan if dgrad else gcb.Plan)(cfg, hip_device=-1)
        fn = kernel_fn(plan.name)
        calls = _calls(disp, fn, plan.info["grid_main"], plan.name)
        if not calls:
            raise ValueError(f"{workload}: no {fn} dispatch with {plan.info['grid_main']} workgroups in {path}")
        avg = {}
        for d in calls:
            for k, v in d["counters"].items():
                avg[k] = avg.get(k, 0.0) + v / len(calls)
        base = {"kernel": plan.name, "source_hash": kernel_source_hash(plan.name), "kernel_fn": fn,
                "dispatches": len(calls)}
        if "FETCH_SIZE" in avg or "WRITE_SIZE" in avg:
            rec = dict(base)
            for cname, key in (("FETCH_SIZE", "fetch_bytes"), ("WRITE_SIZE", "write_bytes")):
                if cname not in avg:
                    continue
                cal = [d["counters"][cname] for d in disp if "neg" in d["kernel"] and cname in d["counters"]]
                if not cal:
                    raise ValueError(f"{path}: no copy-calibration dispatch for {cname}")
                scale = COPY_BYTES / (_median(cal) * 1024.0)
                rec[key] = int(round(avg[cname] * 1024.0 * scale))
                rec[key.replace("bytes", "scale")] = round(scale, 4)
            prev = traffic.get(workload, {})
            prev.update(rec)
            traffic[workload] = prev
        if "SQ_INSTS_MFMA" in avg:
            flops, _ = algorithmic(cfg, gcb.Plan(cfg, hip_device=-1).info)
            mops = avg.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) + avg.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0)
            rec = dict(base, mfma_insts=int(round(avg["SQ_INSTS_MFMA"])),
                       mfma_busy_cycles=int(round(avg.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0))))
            if mops:
                rec["useful_frac"] = round(flops / (mops * 512.0), 4)
            if avg.get("SQ_BUSY_CU_CYCLES"):
                # both counters are sums over the chip; a CU has 4 SIMDs
                rec["cu_busy_cycles"] = int(round(avg["SQ_BUSY_CU_CYCLES"]))
                rec["busy_frac_of_simd_cycles"] = round(
                    avg.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (4 * avg["SQ_BUSY_CU_CYCLES"]), 4)
            ns = sorted(d["ns"] for d in calls if d["ns"])
            if ns:
                rec["launch_us"] = round(ns[len(ns) // 2] / 1e3, 2)
            mfma[workload] = rec
    for fname, recs, about in (
            ("traffic.json", traffic,
             "HBM bytes per launch of each workload's main kernel: rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per "
             "dispatch, one counter per run), each scaled by what it reads for a plain device copy of known size "
             "(torch neg over 256 MiB) in the same run; source_hash: kernel sources the counters were taken on"),
            ("mfma_counters.json", mfma,
             "MFMA counters of each dense workload's main kernel from one rocprofv3 --pmc run, averaged over its "
             "dispatches: instruction count, MFMA-busy cycles summed over SIMDs, useful fraction 2*M*N*R / "
             "(MOPS * 512), busy fraction MFMA-busy cycles / (4 SIMDs * CU-busy cycles, SQ_BUSY_CU_CYCLES), launch_us the "
             "median dispatch duration under the counter run")):
        if not recs:
            continue
        path = os.path.join(out_dir, fname)
        try:
            with open(path) as f:
                old = json.load(f)
        except (OSError, ValueError):
            old = {}
        old["_about"] = about
        for k, v in recs.items():
            merged = dict(old.get(k, {})) if old.get(k, {}).get("source_hash") == v["source_hash"] and \
                old.get(k, {}).get("kernel") == v["kernel"] else {}
            merged.update(v)
            if "fetch_bytes" in merged and "write_bytes" in merged:
                merged["bytes_per_launch"] = merged["fetch_bytes"] + merged["write_bytes"]
            old[k] = merged
        with open(path, "w") as f:
            json.dump(old, f, indent=1, sort_keys=True)
    return traffic, mfma


def _median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


class Timer:
    """Events-bracketed calls on the current stream: 'flushed' with a large
    fill kernel before each call (outside the events), or 'hot'."""

    def __init__(self, torch):
        self.torch = torch
        self.flush_buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        # GPU spin used to let the host queue a batch of calls ahead of the GPU
        s = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        e0.record(s)
        torch.cuda._sleep(1_000_000)
        e1.record(s)
        torch.cuda.synchronize()
        self.spin_per_ms = 1_000_000 / max(1e-3, e0.elapsed_time(e1))

    def spin(self, ms):
        """Keep the GPU busy for about ms milliseconds (lets the host queue
        work behind it)."""
        self.torch.cuda._sleep(int(self.spin_per_ms * ms))

    def calls(self, fn, n, flush):
        torch = self.torch
        s = torch.cuda.current_stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        torch.cuda.synchronize()
        self.spin(20.0)      # for the host to run ahead
        for i in range(n):
            if flush:
                self.flush_buf.fill_(float(i & 7))
            ev[i][0].record(s)
            fn(i)
            ev[i][1].record(s)
        torch.cuda.synchronize()
        us = [a.elapsed_time(b) * 1e3 for a, b in ev]
        return {"median_us": round(_median(us), 3), "min_us": round(min(us), 3), "n": n}


class Case:
    def __init__(self, torch, gcb, workloads, name, cfg, overrides=None):
        self.name, self.cfg = name, cfg
        self.torch = torch
        self.plan = gcb.Plan(cfg, **(overrides or {}))
        x_bits, dy_bits = workloads.inputs(cfg)
        dt = torch.bfloat16 if cfg["in_dtype"] == "bf16" else torch.float16
        out_t = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[cfg["out_dtype"]]
        import numpy as np
        x0 = torch.from_numpy(x_bits.view(np.int16).reshape(-1).copy()).view(dt).cuda()
        dy0 = torch.from_numpy(dy_bits.view(np.int16).reshape(-1).copy()).view(dt).cuda()
        set_bytes = (x0.numel() + dy0.numel()) * 2
        self.nsets = max(2, min(64, math.ceil(ROTATE_BYTES / max(1, set_bytes))))
        self.xs = [x0] + [x0.clone() for _ in range(self.nsets - 1)]
        self.dys = [dy0] + [dy0.clone() for _ in range(self.nsets - 1)]
        self.dw = torch.empty(self.plan.dw_shape(), dtype=out_t, device="cuda")
        self.ws = self.plan.new_workspace() if self.plan.workspace_bytes else None
        self.flops, self.bytes = algorithmic(cfg, self.plan.info)

    def step(self, i, stage=0):
        j = i % self.nsets
        self.plan.run(self.xs[j], self.dys[j], self.dw, self.ws, stage=stage)

    def capture(self, nsteps, stage=0):
        """A HIP graph of nsteps launches (cycling through the input sets)."""
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for i in range(nsteps):
                    self.step(i, stage=stage)
        torch.cuda.current_stream().wait_stream(s)
        return g

    def graph_len(self):
        # enough launches per graph that the replay's own cost is spread thin
        return self.nsets * max(1, math.ceil(GRAPH_MIN_LAUNCHES / self.nsets))

    def time_steps(self, steps, warmup, use_graphs=True, timer=None):
        """Seconds per step over exactly `steps` steps after `warmup` untimed
        ones. With graphs: the steps are captured (one graph of up to
        MAX_GRAPH steps, cycling through the input sets, replayed as often as
        needed plus a tail graph), replayed untimed for SETTLE_S seconds (graph
        upload, and the GPU clocks back at their loaded state after the host
        work of building this workload's inputs), then timed by HIP events on
        the replay stream, recorded behind a GPU spin so that the host's graph
        submission is not on the clock; synchronized on both sides. Without
        graphs (for profilers): host wall clock around eager launches."""
        torch = self.torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        if use_graphs:
            glen = min(steps, MAX_GRAPH)
            full = self.capture(glen)
            rem = steps % glen
            tail = self.capture(rem) if rem else None
            t0 = time.perf_counter()
            while True:                        # untimed: upload, settle
                full.replay()
                if tail is not None:
                    tail.replay()
                torch.cuda.synchronize()
                if time.perf_counter() - t0 >= SETTLE_S:
                    break
            s = torch.cuda.current_stream()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            if timer is not None:
                timer.spin(5.0)
            e0.record(s)
            for _ in range(steps // glen):
                full.replay()
            if tail is not None:
                tail.replay()
            e1.record(s)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e-3 / steps
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(i)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return (t1 - t0) / steps

    def kernel_times(self, reps=4):
        """Average per-launch durations (s) of stage 1 (main kernel) and stage 2
        (reduce), each from HIP events on the launch stream around replays of a
        graph that holds graph_len() launches of that stage alone."""
        torch = self.torch
        out = []
        glen = self.graph_len()
        for stage in (1, 2):
            if stage == 2 and self.plan.info["split_k"] <= 1:
                out.append(0.0)
                continue
            g = self.capture(glen, stage=stage)
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                g.replay()                       # untimed: graph upload
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(s)
                for _ in range(reps):
                    g.replay()
                e1.record(s)
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) * 1e-3 / (reps * glen))
        return out[0], out[1]

    def iteration_stats(self, timer):
        """Median and min of 50 events-bracketed calls of the whole path,
        flushed between calls and hot."""
        for i in range(ITER_WARMUP):
            self.step(i)
        flushed = timer.calls(lambda i: self.step(i), ITER_TIMED, flush=True)
        hot = timer.calls(lambda i: self.step(0), ITER_TIMED, flush=False)
        return flushed, hot

    def row(self, sec_per_step, t_main, t_red, flushed=None, hot=None):
        flops, nbytes = self.flops, self.bytes
        floor = max(flops / PEAK_MFMA_16, nbytes / PEAK_HBM)
        r = {
            "kernel": self.plan.name,
            "us_per_step": round(sec_per_step * 1e6, 3),
            "tflops": round(flops / sec_per_step / 1e12, 3),
            "gbps": round(nbytes / sec_per_step / 1e9, 1),
            "frac_mfma_peak": round(flops / sec_per_step / PEAK_MFMA_16, 4),
            "frac_hbm_peak": round(nbytes / sec_per_step / PEAK_HBM, 4),
            "frac_attainable": round(floor / sec_per_step, 4),
            "bound": reported_bound(self.name, flops, nbytes),
            "main_kernel_us": round(t_main * 1e6, 3),
            "reduce_kernel_us": round(t_red * 1e6, 3),
            "main_kernel_frac_mfma_peak": round(flops / t_main / PEAK_MFMA_16, 4) if t_main else None,
            "main_kernel_frac_hbm_peak": round(nbytes / t_main / PEAK_HBM, 4) if t_main else None,
            "split_k": self.plan.info["split_k"],
            "group_merge": self.plan.info["group_merge"],
            "input_sets": self.nsets,
            "hbm_bytes_measured": measured_traffic(self.name, self.plan.name),
            "mfma_counters": measured_mfma(self.name, self.plan.name),
        }
        if flushed is not None:
            r["iters"] = dict(flushed, flush="512 MiB fill between calls, outside the events",
                              tflops_at_median=round(flops / flushed["median_us"] / 1e6, 3),
                              frac_attainable_at_median=round(floor / (flushed["median_us"] * 1e-6), 4))
            r["hot"] = dict(hot, note="no flush between calls: inputs and workspace warm in L2/MALL")
        return r


class DgradCase(Case):
    """Backward data of a workload's convolution: dX = dgrad(dY, W), one
    kernel per step. FLOPs as for wgrad (the same multiply-adds); bytes =
    |dY| + |W| + |dX|, each once."""

    def __init__(self, torch, gcb, workloads, name, cfg, overrides=None):
        import numpy as np
        self.name, self.cfg = name, cfg
        self.torch = torch
        self.plan = gcb.DgradPlan(cfg, **(overrides or {}))
        dt = torch.bfloat16 if cfg["in_dtype"] == "bf16" else torch.float16
        out_t = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[cfg["out_dtype"]]
        s0, s1 = cfg["seeds"]
        dy_bits = workloads.draw(self.plan.dy_shape(), cfg["in_dtype"], cfg["dist"], s0 + 100)
        w_bits = workloads.draw(self.plan.w_shape(), cfg["in_dtype"], cfg["dist"], s1 + 100)
        dy0 = torch.from_numpy(dy_bits.view(np.int16).reshape(-1).copy()).view(dt).cuda()
        self.w = torch.from_numpy(w_bits.view(np.int16).reshape(-1).copy()).view(dt).cuda()
        self.nsets = max(2, min(64, math.ceil(ROTATE_BYTES / max(1, dy0.numel() * 2))))
        self.dys = [dy0] + [dy0.clone() for _ in range(self.nsets - 1)]
        self.dx = torch.empty(self.plan.dx_shape(), dtype=out_t, device="cuda")
        self.ws = None
        flops, _ = algorithmic(cfg, gcb.Plan(cfg, hip_device=-1).info)
        out_bytes = 4 if cfg["out_dtype"] == "fp32" else 2
        self.flops = flops
        self.bytes = 2 * (dy0.numel() + self.w.numel()) + out_bytes * self.dx.numel()

    def step(self, i, stage=0):
        self.plan.run(self.dys[i % self.nsets], self.w, self.dx)

    def kernel_times(self, reps=4):
        torch = self.torch
        glen = self.graph_len()
        g = self.capture(glen)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            g.replay()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(s)
            for _ in range(reps):
                g.replay()
            e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / (reps * glen), 0.0


SETTLE_S = 0.3   # untimed replays before each workload's timed steps


def oracle_time(workloads, cfg, dgrad=False):
    """Wall time of the CPU oracle over the full output of one configuration
    (the same seeded inputs as the GPU), with the threads it ran on."""
    import oracle
    if dgrad:
        s0, s1 = cfg["seeds"]
        dy_bits = workloads.draw(workloads.dy_shape(cfg), cfg["in_dtype"], cfg["dist"], s0 + 100)
        w_bits = workloads.draw(oracle.dw_shape(cfg), cfg["in_dtype"], cfg["dist"], s1 + 100)
        t0 = time.perf_counter()
        out, _ = oracle.dgrad(cfg, dy_bits, w_bits)
    else:
        x_bits, dy_bits = workloads.inputs(cfg)
        t0 = time.perf_counter()
        out, _ = oracle.wgrad(cfg, x_bits, dy_bits)
    dt = time.perf_counter() - t0
    return dt, oracle.last_threads(), out.size


def cpu_baseline(workloads, cfg):
    dt, threads, n = oracle_time(workloads, cfg)
    G = cfg["G"]
    taps = math.prod(cfg["filt_len"][: cfg["ndim"]])
    R = cfg["N"] * math.prod(cfg["out_len"][: cfg["ndim"]])
    flops = 2 * G * (cfg["K"] // G) * (cfg["C"] // G) * taps * R
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"full dW of the headline workload ({n} elements, {flops/2:.3g} MACs) in "
                      f"{dt:.2f} s, fp64, {threads} OpenMP threads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--configs", default="c1,c2,c3,c4a,c4b,c5,pw,c3d,dgrad:c2,dgrad:c3,dgrad:c4a,dgrad:c5,dgrad:c3d",
                    help="workload names; dgrad:<name> times backward data of that workload")
    ap.add_argument("--eager", action="store_true", help="launch steps one by one (for profilers)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep-merge", action="store_true", help="also time the depthwise shape over Gm and S")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 256 MiB device copy (torch neg), the reference for HBM byte counters")
    ap.add_argument("--ingest-counters", nargs="+", metavar="WORKLOAD=CSV",
                    help="host only: write profiles/traffic.json and profiles/mfma_counters.json from rocprofv3 "
                         "counter CSVs of eager bench runs, then exit")
    ap.add_argument("--summarize-trace", metavar="CSV",
                    help="host only: print the per-workload kernel table of a rocprofv3 kernel-trace CSV, then exit")
    args = ap.parse_args()
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, [n for n in args.configs.split(",") if n]
                              if HEADLINE in args.configs.split(",") else [HEADLINE] + args.configs.split(",")))
        return
    if args.ingest_counters:
        traffic, mfma = ingest_counters([tuple(x.split("=", 1)) for x in args.ingest_counters])
        print(json.dumps({"traffic": traffic, "mfma": mfma}, indent=1))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU only; run with --gpus 1"}))
        sys.exit(2)
    import torch
    import grouped_convolution_backward_amd as gcb
    import workloads

    torch.cuda.init()
    timer = Timer(torch)
    if args.copy_calibration:
        src = torch.ones(128 * 2 ** 20, dtype=torch.bfloat16, device="cuda")   # 256 MiB
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(f"[bench] copy calibration: neg over {src.numel() * 2} bytes read and written", file=sys.stderr)
        del src, dst
    names = [n for n in args.configs.split(",") if n]
    if HEADLINE not in names:
        names.insert(0, HEADLINE)
    per = {}
    head = None
    for name in names:
        if name.startswith("dgrad:"):
            case = DgradCase(torch, gcb, workloads, name, workloads.get(name.split(":", 1)[1]))
        else:
            case = Case(torch, gcb, workloads, name, workloads.get(name))
        sec = case.time_steps(args.steps, args.warmup, use_graphs=not args.eager, timer=timer)
        t_main, t_red = case.kernel_times()
        flushed, hot = (None, None) if args.eager else case.iteration_stats(timer)
        per[name] = case.row(sec, t_main, t_red, flushed, hot)
        if not args.no_cpu_baseline and not args.eager:
            base = name.split(":", 1)[-1]
            dt, th, _ = oracle_time(workloads, workloads.get(base), dgrad=name.startswith("dgrad:"))
            per[name]["cpu_oracle_s"] = round(dt, 3)
            per[name]["cpu_oracle_threads"] = th
            per[name]["gpu_speedup_vs_cpu_oracle"] = round(dt / sec, 1)
        print(f"[bench] {name}: {per[name]}", file=sys.stderr, flush=True)
        if name == HEADLINE:
            head = (case, sec, t_main)
        else:
            del case
        torch.cuda.empty_cache()
    sweep = {}
    if args.sweep_merge:
        cfg = workloads.CONFIGS["c5"]
        for gm in (1, 2, 4, 8):
            for s in (0, 8, 32, 128):
                case = Case(torch, gcb, workloads, "c5", cfg, {"variant": gcb.VARIANT_MFMA, "group_merge": gm, "split_k": s})
                sec = case.time_steps(max(20, args.steps // 4), 5, use_graphs=not args.eager)
                sweep[f"mfma_gm{gm}_spk{case.plan.info['split_k']}"] = round(sec * 1e6, 2)
                del case
                torch.cuda.empty_cache()
        print(f"[bench] c5 merge sweep (us): {sweep}", file=sys.stderr, flush=True)

    case, sec, t_main = head
    cfg = case.cfg
    flops, nbytes = case.flops, case.bytes
    hb = per[HEADLINE]
    bound = hb["bound"]
    if bound == "mfma":
        achieved, peak, unit = flops / t_main / 1e12, PEAK_MFMA_16 / 1e12, "TFLOP/s"
    else:
        achieved, peak, unit = nbytes / t_main / 1e9, PEAK_HBM / 1e9, "GB/s"
    # contract fields first (dominant kernel: the main kernel), then the
    # secondary fractions: the same kernel against the other peak, and the
    # whole step (main + reduce + launch gaps) against both
    roof = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4),
            "traffic": measured_traffic(HEADLINE, case.plan.name),
            "kernel": case.plan.name, "kernel_us": round(t_main * 1e6, 3),
            "kernel_frac_mfma": round(flops / t_main / PEAK_MFMA_16, 4),
            "kernel_frac_hbm": round(nbytes / t_main / PEAK_HBM, 4),
            "step_us": round(sec * 1e6, 3),
            "step_frac_mfma": round(flops / sec / PEAK_MFMA_16, 4),
            "step_frac_hbm": round(nbytes / sec / PEAK_HBM, 4),
            "mfma_counters": hb.get("mfma_counters")}
    out = {
        "metric": METRIC,
        "value": round(flops / sec / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "dense split-K wgrad G=1 N=32 56x56 C=64 K=64 3x3 s1 p1 bf16 (NHWGC/NHWGK/GKYXC)",
                   "G": 1, "N": 32, "C": 64, "K": 64, "H": 56, "W": 56, "filter": "3x3", "stride": 1, "pad": 1,
                   "gemm": "M=64 N=576 K=100352", "parallelism": "single GPU"},
        "roofline": roof,
        "per_config": per,
    }
    if sweep:
        out["c5_merge_sweep_us"] = sweep
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(workloads, cfg)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
