"""Build the HIP library libmlp_chain.so for gfx950 (in-tree).

    python -m consumer_gemm_chain_amd.build

Every source is compiled with hipcc for gfx950 only, with floating-point
contraction off (identical epilogue arithmetic in every kernel) and packed
fp32 instructions disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libmlp_chain.so")
# the same library with pseudo-random pauses before every publication
# (-DMLPC_CHAOS=1), loaded only by the tests
CHAOS_LIB = os.path.join(LIBDIR, "libmlp_chain_chaos.so")
BUILD = os.path.join(ROOT, "_build")
ARCH = "gfx950"

SOURCES = ["chain_api.cpp", "chain_dispatch.cpp", "chain_scratch.hip", "chain_litmus.hip"]
KERNELS = "chain_kernels.hip"     # compiled once per tile configuration


def num_configs() -> int:
    text = open(os.path.join(CSRC, "chain_configs.h")).read()
    import re
    return len(re.findall(r"^\s*X\(\d+,", text, flags=re.M))

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _compile(job, verbose: bool) -> str:
    src, cfg, chaos = job
    tag = os.path.basename(src) + ("" if cfg is None else f".cfg{cfg}") + (".chaos" if chaos else "")
    obj = os.path.join(BUILD, tag + ".o")
    defs = ([] if cfg is None else [f"-DMLPC_CFG={cfg}"]) + (["-DMLPC_CHAOS=1"] if chaos else [])
    cmd = [hipcc(), "-x", "hip", *FLAGS, *defs, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return obj


def _link(objs, lib, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Build the library and its test variant with chaos pauses."""
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    kern = [(KERNELS, c, False) for c in range(num_configs())]
    chaos = [(KERNELS, c, True) for c in range(num_configs())]
    api = [(src, None, False) for src in SOURCES]
    jobs = kern + chaos + api
    workers = min(len(jobs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        objs = dict(zip(jobs, ex.map(lambda j: _compile(j, verbose), jobs)))
    _link([objs[j] for j in kern + api], LIB, verbose)
    _link([objs[j] for j in chaos + api], CHAOS_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
