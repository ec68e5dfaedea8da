"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code, on
the CPU:

* the planner and C ABI (csrc/plan.cpp, csrc/abi.cpp) linked with stub
  launchers (tests/sanitize/hip_stubs.cpp) and driven over every workload,
  the widened shapes, edge and invalid problems, overflow probes and override
  sweeps in both directions (tests/sanitize/plan_driver.cpp). Each plan's
  decisions must equal the regular library's, and the run entry points must
  reject bad arguments without launching;
* the CPU oracle (oracle/wgrad_oracle.c) on small problems, whose results
  must equal the regular oracle's bit for bit.

Any sanitizer report fails the test (halt_on_error)."""

import os
import shutil
import subprocess

import numpy as np
import pytest

import grouped_convolution_backward_amd as gcb
import oracle
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "grouped_convolution_backward_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
SAN_ENV = {"ASAN_OPTIONS": "halt_on_error=1:detect_leaks=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                                reason="needs gcc and g++")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    if r.returncode != 0:
        raise AssertionError(f"{' '.join(cmd[:3])} ... failed ({r.returncode}):\n{r.stdout[-2000:]}\n{r.stderr[-4000:]}")
    return r


@pytest.fixture(scope="module")
def drivers(tmp_path_factory):
    d = tmp_path_factory.mktemp("san")
    plan_exe, oracle_exe = str(d / "plan_driver"), str(d / "oracle_driver")
    _run(["g++", "-std=c++17", *SAN_FLAGS, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
          "-I", os.path.join(ROOT, "include"),
          os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "abi.cpp"),
          os.path.join(SAN, "hip_stubs.cpp"), os.path.join(SAN, "plan_driver.cpp"), "-o", plan_exe])
    _run(["gcc", "-std=c11", *SAN_FLAGS, "-fopenmp", os.path.join(ROOT, "oracle", "wgrad_oracle.c"),
          os.path.join(SAN, "oracle_driver.c"), "-o", oracle_exe, "-lm"])
    return plan_exe, oracle_exe, d


def _env():
    e = dict(os.environ)
    e.update(SAN_ENV)
    return e


def _fields(cfg):
    nd = int(cfg["ndim"])
    f = [nd, gcb.DTYPES[cfg["in_dtype"]], gcb.DTYPES[cfg.get("out_dtype", cfg["in_dtype"])],
         cfg["G"], cfg["N"], cfg["C"], cfg["K"]]
    for name in ("in_len", "filt_len", "stride", "dilation", "pad_lo", "pad_hi"):
        v = list(cfg[name])[:nd]
        f += [int(x) for x in v] + [0] * (3 - len(v))
    return [int(x) for x in f]


def _p(ndim, G, N, C, K, in_len, filt, stride=None, pad=None, dil=None, dtype="bf16", out=None, pad_hi=None):
    one = (1,) * ndim
    pad = pad or (0,) * ndim
    return {"ndim": ndim, "G": G, "N": N, "C": C, "K": K, "in_len": in_len, "filt_len": filt,
            "stride": stride or one, "dilation": dil or one, "pad_lo": pad, "pad_hi": pad_hi or pad,
            "in_dtype": dtype, "out_dtype": out or dtype}


def _cases():
    """(op, problem, overrides) triples: every workload and widened shape,
    override sweeps, edge and invalid problems, overflow probes, random small
    problems."""
    cases = []
    named = dict(workloads.CONFIGS)
    named.update(workloads.WIDER)
    for cfg in named.values():
        for op in (0, 1):
            cases.append((op, cfg, (0, 0, 0, 0)))
    for name in ("c2", "c3", "c4a", "c4b", "c5"):
        cfg = workloads.CONFIGS[name]
        for ov in ((1, 0, 0, 0), (3, 0, 0, 0), (0, 0, 1, 0), (0, 0, 1, 3), (0, 0, 3, 1), (0, 0, 3, 2),
                   (7, 0, 3, 0), (0, 2, 1, 0), (0, 0, 2, 0), (0, 0, 2, 1), (0, 0, 2, 2), (0, 0, 2, 3),
                   (100000, 0, 0, 0), (0, 3, 0, 0), (0, 0, 9, 0), (0, 0, 1, 99)):
            cases.append((0, cfg, ov))
        for ov in ((0, 0, 4, 1), (0, 0, 4, 2), (0, 0, 4, 3), (0, 0, 4, 4), (0, 0, 4, 5), (0, 0, 4, 6),
                   (2, 0, 0, 0), (0, 2, 0, 0), (0, 0, 1, 0)):
            cases.append((1, cfg, ov))
    for n in (0, 1):
        cases.append((0, workloads.problem("c2", N=n), (0, 0, 0, 0)))
        cases.append((1, workloads.problem("c5", N=n), (0, 0, 0, 0)))
    # the depthwise tile form: a workgroup over several tiles, and every form override
    cases.append((0, workloads.problem("c5", N=64), (0, 0, 0, 0)))
    for form in (1, 2, 3, 4, 5):
        cases.append((0, workloads.problem("c5", N=3, in_len=(9, 31), out_len=(9, 31)), (5, 0, 2, form)))
    # backward data: the depthwise tile form (taller tiles, several per
    # workgroup) and every depthwise form override
    cases.append((1, workloads.problem("c5", N=64), (0, 0, 0, 0)))
    for form in (4, 5, 7, 8):
        cases.append((1, workloads.problem("c5", N=3, in_len=(9, 31), out_len=(9, 31)), (0, 0, 0, form)))
    bad = [
        workloads.problem("c1", G=3), workloads.problem("c1", N=-1), workloads.problem("c2", N=20000),
        workloads.problem("c1", in_len=(1, 1), pad_lo=(0, 0), pad_hi=(0, 0)),
        _p(3, 1, 1, 16, 16, (2 ** 20,) * 3, (1, 1, 1), stride=(2 ** 20,) * 3),
        _p(3, 1, 1, 16, 16, (4, 4, 2 ** 40), (1, 1, 1)),
        _p(3, 1, 1, 16, 16, (4, 4, 4), (1, 1, 1), pad=(0, 0, 2 ** 62)),
        _p(3, 1, 2 ** 33, 16, 16, (4, 4, 4), (1, 1, 1)),
        _p(3, 1, 1, 64, 64, (4096, 64, 64), (3, 3, 3), pad=(1, 1, 1)),
        _p(2, 1, 1, 8, 8, (2 ** 31 - 1, 2), (1, 1), stride=(2 ** 31 - 1, 1)),
        _p(1, 1, 1, 8, 8, (16,), (3,), dil=(2 ** 31 - 1,)),
    ]
    for cfg in bad:
        for op in (0, 1):
            cases.append((op, cfg, (0, 0, 0, 0)))
    rng = np.random.default_rng(77)
    for _ in range(60):
        nd = int(rng.integers(1, 4))
        G = int(rng.choice([1, 2, 4, 8, 32]))
        cpg, kpg = int(rng.choice([1, 3, 8, 16, 32, 64])), int(rng.choice([1, 5, 8, 32, 64]))
        in_len = tuple(int(x) for x in rng.integers(1, 40, nd))
        filt = tuple(int(x) for x in rng.integers(1, 6, nd))
        stride = tuple(int(x) for x in rng.integers(1, 4, nd))
        dil = tuple(int(x) for x in rng.integers(1, 3, nd))
        pad = tuple(int(x) for x in rng.integers(0, 3, nd))
        padh = tuple(int(x) for x in rng.integers(0, 3, nd))
        dt = str(rng.choice(["bf16", "fp16"]))
        out = str(rng.choice([dt, "fp32"]))
        cfg = _p(nd, G, int(rng.integers(0, 5)), G * cpg, G * kpg, in_len, filt, stride, pad, dil, dt, out, padh)
        ov = (int(rng.choice([0, 0, 1, 2, 5])), int(rng.choice([0, 0, 1, 2, 4])), int(rng.choice([0, 0, 1, 2, 3])), 0)
        cases.append((int(rng.integers(0, 2)), cfg, ov))
    return cases


def _regular(op, cfg, ov):
    """The same plan through the regular library, in the line format plan_driver prints."""
    kw = dict(split_k=ov[0], group_merge=ov[1], variant=ov[2], tile=ov[3])
    try:
        p = (gcb.Plan if op == 0 else gcb.DgradPlan)(cfg, hip_device=-1, **kw)
    except gcb.WgradError as e:
        return f"{e.code}|||||||||"
    i = p.info
    return (f"0|{p.name}|{i['variant']}|{i['tile']}|{i['split_k']}|{i['group_merge']}|{i['grid_main']}|"
            f"{i['grid_reduce']}|{i['workspace_bytes']}")


def test_planner_and_abi_under_sanitizers(drivers):
    plan_exe, _, _ = drivers
    cases = _cases()
    lines = "\n".join(" ".join(str(v) for v in [op] + _fields(cfg) + list(ov)) for op, cfg, ov in cases)
    r = _run([plan_exe], input=lines + "\n", env=_env())
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-3000:]
    got = r.stdout.strip().splitlines()
    assert len(got) == len(cases)
    made = 0
    for (op, cfg, ov), line in zip(cases, got):
        want = _regular(op, cfg, ov)
        assert line == want, (op, cfg, ov, line, want)
        made += line.startswith("0|")
    assert made >= len(cases) // 3, made


def _oracle_case(drivers, op, cfg, seed):
    _, oracle_exe, d = drivers
    nd = int(cfg["ndim"])
    cfg = dict(cfg, out_len=tuple(oracle.out_len(cfg)))
    if op == 0:
        a = workloads.draw(workloads.x_shape(cfg), cfg["in_dtype"], "uniform", seed)
        b = workloads.draw(workloads.dy_shape(cfg), cfg["in_dtype"], "uniform", seed + 1)
        ref, ab = oracle.wgrad(cfg, a, b)
    else:
        a = workloads.draw(workloads.dy_shape(cfg), cfg["in_dtype"], "uniform", seed)
        b = workloads.draw(oracle.dw_shape(cfg), cfg["in_dtype"], "uniform", seed + 1)
        ref, ab = oracle.dgrad(cfg, a, b)
    inp, outp = str(d / f"in{op}_{seed}.bin"), str(d / f"out{op}_{seed}.bin")
    np.concatenate([np.asarray(a, np.uint16).reshape(-1), np.asarray(b, np.uint16).reshape(-1)]).tofile(inp)
    f = [nd, cfg["G"], cfg["N"], cfg["C"], cfg["K"]]
    for name in ("in_len", "filt_len", "stride", "dilation", "pad_lo", "pad_hi"):
        v = list(cfg[name])[:nd]
        f += [int(x) for x in v] + [0] * (3 - len(v))
    f.append(oracle.DTYPE_CODE[cfg["in_dtype"]])
    r = _run([oracle_exe, str(op), "3", inp, outp] + [str(int(x)) for x in f], env=_env())
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-3000:]
    out = np.fromfile(outp, np.float64)
    n = ref.size
    assert out.size == 2 * n
    assert np.array_equal(out[:n], ref.reshape(-1)) and np.array_equal(out[n:], ab.reshape(-1))


@pytest.mark.parametrize("op", [0, 1])
def test_oracle_under_sanitizers(drivers, op):
    cases = [workloads.CONFIGS["c1"],
             _p(1, 2, 2, 6, 4, (13,), (3,), (2,), (1,), (2,), "fp16"),
             _p(2, 4, 1, 8, 8, (7, 9), (3, 2), (2, 1), (1, 0), (1, 2)),
             _p(3, 1, 1, 4, 6, (4, 5, 6), (2, 3, 3), (1, 2, 1), (1, 1, 0), (2, 1, 1), "fp16"),
             _p(2, 8, 2, 8, 8, (6, 6), (3, 3), pad=(1, 1)),
             _p(2, 1, 0, 4, 4, (5, 5), (3, 3), pad=(1, 1))]
    for i, cfg in enumerate(cases):
        _oracle_case(drivers, op, cfg, 900 + 10 * i)
