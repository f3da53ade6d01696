"""CPU sanitizer builds: the oracle (plain C, gcc) and the library's host-only
entry points (the planner and the argument checks; host code built by hipcc
with AddressSanitizer and UndefinedBehaviorSanitizer, device code as usual),
each driven by a stand-alone program under tests/native that checks its
contract and exits 0.  Any out-of-bounds access, leak (oracle) or undefined
behaviour aborts the program."""
import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

from consumer_gemm_chain_amd import build as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout, env=env)
    assert r.returncode == 0, (" ".join(cmd), r.stdout[-2000:], r.stderr[-4000:])
    return r


def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_selftest")
    _run(["gcc", "-O1", "-g", "-fopenmp", "-ffp-contract=off", "-std=c11", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", os.path.join(ROOT, "oracle", "mlp_oracle.c"),
          os.path.join(NATIVE, "oracle_selftest.c"), "-o", exe, "-lm"])
    r = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1"})
    assert "0 failures" in r.stdout and "runtime error" not in r.stderr


def test_planner_under_address_and_undefined_sanitizers(tmp_path):
    if not os.path.exists(b.hipcc()):
        pytest.skip("hipcc not available")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    inc = [f"-I{os.path.join(ROOT, 'include')}", f"-I{b.CSRC}"]
    base = [b.hipcc(), "-x", "hip", f"--offload-arch={b.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC",
            "-ffp-contract=off", *san, *inc]
    jobs = [(os.path.join(b.CSRC, s), str(tmp_path / f"{s}.o"), []) for s in b.SOURCES]
    jobs += [(os.path.join(b.CSRC, b.KERNELS), str(tmp_path / f"k{c}.o"), [f"-DMLPC_CFG={c}"])
             for c in range(b.num_configs())]

    def one(job):
        src, obj, defs = job
        _run(base + defs + ["-c", src, "-o", obj])
        return obj
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(one, jobs))
    drv = str(tmp_path / "driver.o")
    _run([b.hipcc(), "-O1", "-g", "-std=c++17", *san, *inc, "-c", os.path.join(NATIVE, "plan_selftest.cpp"),
          "-o", drv])
    exe = str(tmp_path / "plan_selftest")
    _run([b.hipcc(), f"--offload-arch={b.ARCH}", *san, *objs, drv, "-o", exe])
    # leaks are not checked: the HIP runtime keeps allocations until exit
    r = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=0"})
    assert "0 failures" in r.stdout and "runtime error" not in r.stderr
