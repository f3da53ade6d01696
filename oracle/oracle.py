"""ctypes wrapper around the plain C oracle (mlp_oracle.c).

TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the CPU
baseline leg of the benchmark are the only callers; the GPU library and its
Python binding never import this module.  It shares no code with them.

All arrays are numpy ``uint16`` bit patterns of fp16 or bf16 values.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mlp_oracle.c")
LIB = os.path.join(HERE, "libmlp_oracle.so")

ACT = {"none": 0, "gelu_tanh": 1, "swiglu": 2}
DTYPE = {"f16": 0, "bf16": 1}

_lib = None


def build(force: bool = True) -> str:
    """Compile mlp_oracle.c with gcc into libmlp_oracle.so (strict IEEE fp32)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-std=c11", "-shared", "-fPIC", SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build(force=True)
        lib = ctypes.CDLL(LIB)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        ci = ctypes.c_int
        lib.oracle_mlp_chain.argtypes = [p, p, p, p, p, i64, i64, i64, ci, ci, ci]
        lib.oracle_mlp_chain.restype = ci
        lib.oracle_widen.argtypes = [p, p, i64, ci]
        lib.oracle_widen.restype = None
        lib.oracle_round.argtypes = [p, p, i64, ci]
        lib.oracle_round.restype = None
        lib.oracle_act.argtypes = [p, p, p, i64, ci]
        lib.oracle_act.restype = None
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ci
        _lib = lib
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _dt(dtype) -> int:
    return DTYPE[dtype] if isinstance(dtype, str) else int(dtype)


def _act(act) -> int:
    return ACT[act] if isinstance(act, str) else int(act)


def widen(bits: np.ndarray, dtype) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, np.float32)
    _load().oracle_widen(_ptr(bits), _ptr(out), bits.size, _dt(dtype))
    return out


def round_to(vals: np.ndarray, dtype) -> np.ndarray:
    vals = np.ascontiguousarray(vals, dtype=np.float32)
    out = np.empty(vals.shape, np.uint16)
    _load().oracle_round(_ptr(vals), _ptr(out), vals.size, _dt(dtype))
    return out


def act(g: np.ndarray, act, u: np.ndarray | None = None) -> np.ndarray:
    g = np.ascontiguousarray(g, dtype=np.float32)
    if u is not None:
        u = np.ascontiguousarray(u, dtype=np.float32)
        assert u.shape == g.shape
    out = np.empty(g.shape, np.float32)
    _load().oracle_act(_ptr(g), _ptr(u), _ptr(out), g.size, _act(act))
    return out


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def mlp_chain(x: np.ndarray, w1: np.ndarray, w2: np.ndarray, act, dtype,
              want_t: bool = False, nthreads: int = 0):
    """Run the oracle chain.  x [M,H], w1 [H,g*I], w2 [I,H] (uint16 bits).

    Returns y [M,H] (and t [M,I] if want_t)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    w1 = np.ascontiguousarray(w1, dtype=np.uint16)
    w2 = np.ascontiguousarray(w2, dtype=np.uint16)
    M, H = x.shape
    I, H2 = w2.shape
    g = 2 if _act(act) == ACT["swiglu"] else 1
    if H2 != H or w1.shape != (H, g * I):
        raise ValueError(f"shape mismatch: x{x.shape} w1{w1.shape} w2{w2.shape} act={act}")
    y = np.empty((M, H), np.uint16)
    t = np.empty((M, I), np.uint16) if want_t else None
    rc = _load().oracle_mlp_chain(_ptr(x), _ptr(w1), _ptr(w2), _ptr(t), _ptr(y),
                                  M, H, I, _act(act), _dt(dtype), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_mlp_chain failed with {rc}")
    return (y, t) if want_t else y


def mlp_layers(x: np.ndarray, w1s, w2s, act, dtype) -> np.ndarray:
    """A chain of MLP layers, the plain composition: layer l's input is layer
    l-1's output Y (already rounded to the storage dtype, as every chain
    output is), Y_l = mlp_chain(Y_{l-1}, W1_l, W2_l), Y_{-1} = x.  Chaining
    consecutive layers in one kernel (the Hacker News thread on megakernels
    vs CUDA graphs: overlapping work across layers) changes when tiles run,
    not what each layer computes.  Returns the last layer's Y."""
    if len(w1s) != len(w2s) or len(w1s) < 1:
        raise ValueError("need the same number (>= 1) of W1 and W2 matrices")
    y = np.ascontiguousarray(x, dtype=np.uint16)
    for w1, w2 in zip(w1s, w2s):
        y = mlp_chain(y, w1, w2, act, dtype)
    return y
