"""Build libwgrad.so (HIP kernels + host planner + C ABI) in-tree for gfx950.

    python -m grouped_convolution_backward_amd.build

Objects are compiled in parallel into csrc/_build/ and linked into
grouped_convolution_backward_amd/libwgrad.so.
"""

from __future__ import annotations

import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(CSRC, "_build")
LIB = os.path.join(HERE, "libwgrad.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["kernels.hip", "rowslab.hip", "ring.hip", "depthwise.hip", "dwtile.hip", "dgrad.hip", "dgrad_ring.hip", "noalloc.hip",
           "probe.hip", "plan.cpp", "abi.cpp"]

# Packed fp32 instructions are kept out of every code object.
COMMON = ["-O3", "-fPIC", "-std=c++17", "--offload-arch=gfx950", "-mcode-object-version=5", "-I", INCLUDE,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]


# Kernels that load straight into LDS with inline-assembly buffer loads wait
# for them with exact vector-memory counts (s_waitcnt vmcnt(N)). A load or
# store the compiler adds to such a wave, such as a register spill to
# scratch, would make those counts short and the waits race. Every kernel in
# a source file that issues such loads must therefore compile without scratch
# memory and without a dynamic stack; the build fails otherwise.
_DMA_MARK = "dma_load16("
_REMARK = re.compile(r"remark:\s+(Function Name|ScratchSize \[bytes/lane\]|Dynamic Stack):\s*(\S+)")


def uses_counted_lds_loads(src: str) -> bool:
    with open(os.path.join(CSRC, src)) as f:
        return _DMA_MARK in f.read()


def scratch_violations(remarks: str):
    """(kernel, scratch bytes, dynamic stack) of every kernel in the
    kernel-resource-usage remarks that uses scratch or a dynamic stack."""
    bad, name, scratch = [], None, 0
    for key, val in _REMARK.findall(remarks):
        if key == "Function Name":
            name, scratch = val, 0
        elif key.startswith("ScratchSize"):
            scratch = int(val)
        elif key == "Dynamic Stack":
            if scratch or val != "False":
                bad.append((name, scratch, val))
    return bad


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, "-x", "hip" if src.endswith(".hip") else "c++", "-c",
           os.path.join(CSRC, src), "-o", obj]
    if not src.endswith(".hip"):
        # host-only translation units still go through hipcc for the HIP headers
        cmd = [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    guard = src.endswith(".hip") and uses_counted_lds_loads(src)
    if guard:
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    text = r.stdout + r.stderr
    if guard and r.returncode == 0:
        bad = scratch_violations(text)
        names = set(re.findall(r"Function Name:\s*(\S+)", text))
        if not names:
            raise RuntimeError(f"{src}: no kernel resource usage reported; cannot check scratch use")
        if bad:
            raise RuntimeError(f"{src}: kernels with counted direct-to-LDS loads use scratch memory "
                               f"(their vmcnt waits would be short): {bad}")
    out = "\n".join(l for l in text.splitlines()
                    if "packed-fp32-ops" not in l and "kernel-resource-usage" not in l
                    and not re.match(r"^\s*\d+ \|", l) and not re.match(r"^\s*\|\s*\^", l))
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{out}")
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
