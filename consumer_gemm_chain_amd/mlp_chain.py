"""Thin Python binding of the C ABI in include/mlp_chain.h (ctypes).

Only argument marshalling happens here: every step of the chain runs in the
HIP library libmlp_chain.so.  torch supplies device memory (tensor
data_ptr()) and streams (torch.cuda.current_stream().cuda_stream, a
hipStream_t on ROCm).  There is no fallback: if the library is not built,
loading fails with an error that says how to build it.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "lib", "libmlp_chain.so")

MLP_ACT_NONE, MLP_ACT_GELU_TANH, MLP_ACT_SWIGLU = 0, 1, 2
MLP_DTYPE_F16, MLP_DTYPE_BF16 = 0, 1
MLP_POLICY_STREAM_ORDERED, MLP_POLICY_ROW_SYNC, MLP_POLICY_TILE_SYNC = 0, 1, 2
MLP_OK, MLP_EINVAL, MLP_ENOMEM, MLP_EHIP, MLP_ETIMEOUT = 0, -1, -2, -3, -4

ACTS = {"none": MLP_ACT_NONE, "gelu_tanh": MLP_ACT_GELU_TANH, "swiglu": MLP_ACT_SWIGLU}
DTYPES = {"f16": MLP_DTYPE_F16, "bf16": MLP_DTYPE_BF16}
POLICIES = {"stream_ordered": MLP_POLICY_STREAM_ORDERED, "row_sync": MLP_POLICY_ROW_SYNC,
            "tile_sync": MLP_POLICY_TILE_SYNC}

EXPORTS = ("mlp_chain_create", "mlp_chain_run", "mlp_chain_destroy", "mlp_chain_run_phase",
           "mlp_chain_status", "mlp_chain_last_error", "mlp_chain_info", "mlp_chain_plan",
           "mlp_chain_debug_set_spin_limit", "mlp_chain_debug_skip_producer",
           "mlp_chain_debug_set_config", "mlp_chain_debug_set_split", "mlp_chain_debug_set_grid",
           "mlp_chain_debug_set_order", "mlp_chain_debug_set_trace", "mlp_chain_debug_read_intermediate",
           "mlp_chain_run_noalloc", "mlp_chain_create_layers", "mlp_chain_run_layers", "mlp_chain_debug_litmus",
           "mlp_chain_debug_set_epoch", "mlp_chain_set_weight_ld", "mlp_chain_weight_ld")

INFO_FIELDS = ("BM", "BN1", "BN2", "BK", "Mt", "N1t", "N2t", "T1", "T2", "grid", "wg_per_cu",
               "threads", "cus", "epoch", "config", "workspace_bytes", "S1", "S2", "ksp1", "ksp2", "layers")

_lib = None


class MlpChainError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"mlp_chain error {code}: {msg}")
        self.code = code


def load_library(path: str | None = None):
    """Load libmlp_chain.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = _bind(path or LIB_PATH)
    return _lib


def load_chaos_library():
    """The test build of the library (pauses before every publication), as a
    separate ctypes handle with the same signatures."""
    return _bind(os.path.join(PKG, "lib", "libmlp_chain_chaos.so"))


def _bind(path: str):
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library not found at {path}; build it with "
                           "`python -m consumer_gemm_chain_amd.build` (needs hipcc)")
    lib = ctypes.CDLL(path)
    vp, i64, ci, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint32
    lib.mlp_chain_create.argtypes = [i64, i64, i64, ci, ci, ci]
    lib.mlp_chain_create.restype = vp
    lib.mlp_chain_run.argtypes = [vp, vp, vp, vp, vp, vp]
    lib.mlp_chain_run.restype = ci
    lib.mlp_chain_destroy.argtypes = [vp]
    lib.mlp_chain_destroy.restype = ci
    lib.mlp_chain_run_phase.argtypes = [vp, ci, vp, vp, vp, vp, vp]
    lib.mlp_chain_run_phase.restype = ci
    lib.mlp_chain_status.argtypes = [vp]
    lib.mlp_chain_status.restype = ci
    lib.mlp_chain_last_error.argtypes = []
    lib.mlp_chain_last_error.restype = ctypes.c_char_p
    lib.mlp_chain_info.argtypes = [vp, ctypes.POINTER(i64), ci]
    lib.mlp_chain_info.restype = ci
    lib.mlp_chain_plan.argtypes = [i64, i64, i64, ci, ci, ci, ctypes.POINTER(ctypes.c_int64), ci]
    lib.mlp_chain_plan.restype = ci
    lib.mlp_chain_debug_set_spin_limit.argtypes = [vp, u32]
    lib.mlp_chain_debug_set_spin_limit.restype = ci
    lib.mlp_chain_debug_skip_producer.argtypes = [vp, i64]
    lib.mlp_chain_debug_skip_producer.restype = ci
    lib.mlp_chain_debug_set_config.argtypes = [vp, ci]
    lib.mlp_chain_debug_set_config.restype = ci
    lib.mlp_chain_debug_set_split.argtypes = [vp, ci, ci]
    lib.mlp_chain_debug_set_split.restype = ci
    lib.mlp_chain_debug_set_grid.argtypes = [vp, ci]
    lib.mlp_chain_debug_set_grid.restype = ci
    lib.mlp_chain_debug_set_order.argtypes = [vp, ci]
    lib.mlp_chain_debug_set_order.restype = ci
    lib.mlp_chain_debug_set_trace.argtypes = [vp, vp]
    lib.mlp_chain_debug_set_trace.restype = ci
    lib.mlp_chain_debug_read_intermediate.argtypes = [vp, vp, vp]
    lib.mlp_chain_debug_read_intermediate.restype = ci
    lib.mlp_chain_run_noalloc.argtypes = [i64, i64, i64, ci, ci, ci, vp, vp, vp, vp, vp, vp]
    lib.mlp_chain_run_noalloc.restype = ci
    sz = ctypes.c_size_t
    lib.mlp_chain_debug_litmus.argtypes = [vp, sz, vp, sz, vp, ci, ci, ci, u32, vp]
    lib.mlp_chain_debug_litmus.restype = ci
    lib.mlp_chain_debug_set_epoch.argtypes = [vp, u32]
    lib.mlp_chain_debug_set_epoch.restype = ci
    lib.mlp_chain_set_weight_ld.argtypes = [vp, i64, i64]
    lib.mlp_chain_set_weight_ld.restype = ci
    lib.mlp_chain_weight_ld.argtypes = [i64, i64, ci, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.mlp_chain_weight_ld.restype = ci
    lib.mlp_chain_create_layers.argtypes = [i64, i64, i64, ci, ci, ci, ci]
    lib.mlp_chain_create_layers.restype = vp
    lib.mlp_chain_run_layers.argtypes = [vp, vp, ctypes.POINTER(vp), ctypes.POINTER(vp), vp, vp]
    lib.mlp_chain_run_layers.restype = ci
    return lib


# ---- the C ABI, name for name -------------------------------------------------

def mlp_chain_last_error() -> str:
    return load_library().mlp_chain_last_error().decode()


def _check(rc: int) -> int:
    if rc != MLP_OK:
        raise MlpChainError(rc, mlp_chain_last_error())
    return rc


def mlp_chain_create(M: int, H: int, I: int, act: int, dtype: int, policy: int) -> int:
    """Returns the opaque handle (an integer address); raises on failure."""
    h = load_library().mlp_chain_create(int(M), int(H), int(I), int(act), int(dtype), int(policy))
    if not h:
        raise MlpChainError(MLP_EINVAL, mlp_chain_last_error())
    return h


def mlp_chain_set_weight_ld(h: int, ldw1: int, ldw2: int) -> int:
    return _check(load_library().mlp_chain_set_weight_ld(h, int(ldw1), int(ldw2)))


def mlp_chain_weight_ld(H: int, I: int, act: int) -> tuple[int, int]:
    a, b = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(load_library().mlp_chain_weight_ld(int(H), int(I), int(act), ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def mlp_chain_create_layers(M: int, H: int, I: int, act: int, dtype: int, policy: int, layers: int) -> int:
    """A chain of `layers` MLP layers; returns the opaque handle, raises on failure."""
    h = load_library().mlp_chain_create_layers(int(M), int(H), int(I), int(act), int(dtype), int(policy),
                                               int(layers))
    if not h:
        raise MlpChainError(MLP_EINVAL, mlp_chain_last_error())
    return h


def mlp_chain_run_layers(h: int, x: int, w1s, w2s, out: int, hip_stream: int | None) -> int:
    """`w1s` / `w2s`: sequences of the layers' device pointers."""
    arr1 = (ctypes.c_void_p * len(w1s))(*w1s)
    arr2 = (ctypes.c_void_p * len(w2s))(*w2s)
    return _check(load_library().mlp_chain_run_layers(h, x, arr1, arr2, out, hip_stream or None))


def mlp_chain_run(h: int, x: int, w1: int, w2: int, out: int, hip_stream: int | None) -> int:
    return _check(load_library().mlp_chain_run(h, x, w1, w2, out, hip_stream or None))


def mlp_chain_run_phase(h: int, phase: int, x: int | None, w1: int | None, w2: int | None,
                        out: int | None, hip_stream: int | None) -> int:
    return _check(load_library().mlp_chain_run_phase(h, int(phase), x, w1, w2, out, hip_stream or None))


def mlp_chain_destroy(h: int | None) -> int:
    return _check(load_library().mlp_chain_destroy(h))


def mlp_chain_status(h: int) -> int:
    """Returns MLP_OK or MLP_ETIMEOUT (the sticky watchdog status); raises on
    other errors."""
    rc = load_library().mlp_chain_status(h)
    if rc not in (MLP_OK, MLP_ETIMEOUT):
        raise MlpChainError(rc, mlp_chain_last_error())
    return rc


def mlp_chain_info(h: int) -> dict:
    arr = (ctypes.c_int64 * len(INFO_FIELDS))()
    _check(load_library().mlp_chain_info(h, arr, len(INFO_FIELDS)))
    return dict(zip(INFO_FIELDS, (int(v) for v in arr)))


PLAN_FIELDS = ("config", "S1", "S2", "BM", "BN1", "BN2", "Mt", "N1t", "N2t", "T1", "T2", "ksp1", "ksp2", "tuned")


def mlp_chain_plan(M: int, H: int, I: int, act: int, policy: int, cus: int) -> dict:
    """The plan mlp_chain_create would make on a GPU with `cus` CUs (host
    only); a negative `cus` gives the rules' plan for -cus CUs."""
    arr = (ctypes.c_int64 * len(PLAN_FIELDS))()
    _check(load_library().mlp_chain_plan(int(M), int(H), int(I), int(act), int(policy), int(cus), arr,
                                         len(PLAN_FIELDS)))
    return dict(zip(PLAN_FIELDS, (int(v) for v in arr)))


def mlp_chain_debug_set_spin_limit(h: int, limit: int) -> int:
    return _check(load_library().mlp_chain_debug_set_spin_limit(h, int(limit)))


def mlp_chain_debug_skip_producer(h: int, tile: int) -> int:
    return _check(load_library().mlp_chain_debug_skip_producer(h, int(tile)))


def mlp_chain_debug_set_config(h: int, config_id: int) -> int:
    return _check(load_library().mlp_chain_debug_set_config(h, int(config_id)))


def mlp_chain_debug_set_split(h: int, s1: int, s2: int) -> int:
    return _check(load_library().mlp_chain_debug_set_split(h, int(s1), int(s2)))


def mlp_chain_debug_set_grid(h: int, grid: int) -> int:
    return _check(load_library().mlp_chain_debug_set_grid(h, int(grid)))


def mlp_chain_debug_set_order(h: int, order: int) -> int:
    return _check(load_library().mlp_chain_debug_set_order(h, int(order)))


def mlp_chain_debug_set_epoch(h: int, epoch: int) -> int:
    return _check(load_library().mlp_chain_debug_set_epoch(h, int(epoch) & 0xFFFFFFFF))


def mlp_chain_debug_set_trace(h: int, buffer: int | None) -> int:
    return _check(load_library().mlp_chain_debug_set_trace(h, buffer))


def mlp_chain_debug_litmus(data: int, data_bytes: int, flags: int, flag_bytes: int, result: int, rounds: int,
                           half_lines: bool, agent: bool, spin_limit: int, hip_stream: int | None) -> int:
    return _check(load_library().mlp_chain_debug_litmus(data, int(data_bytes), flags, int(flag_bytes), result,
                                                        int(rounds), int(bool(half_lines)), int(bool(agent)),
                                                        int(spin_limit), hip_stream or None))


def mlp_chain_debug_read_intermediate(h: int, dst: int, hip_stream: int | None) -> int:
    return _check(load_library().mlp_chain_debug_read_intermediate(h, dst, hip_stream or None))


def mlp_chain_run_noalloc(M: int, H: int, I: int, act: int, dtype: int, policy: int, x: int, w1: int, w2: int,
                          out: int, status: int | None, hip_stream: int | None) -> int:
    """One chain pass with the workspace in the library's static scratch (no
    handle, no allocation after the first call on a device)."""
    return _check(load_library().mlp_chain_run_noalloc(int(M), int(H), int(I), int(act), int(dtype), int(policy),
                                                       x, w1, w2, out, status, hip_stream or None))


# ---- convenience wrapper over torch tensors -------------------------------------

class MlpChain:
    """Owns one handle.  `run(x, w1, w2, out)` takes torch device tensors of
    dtype float16 / bfloat16 (or int16 / uint16 bit patterns) and enqueues on
    torch's current stream (or `stream`)."""

    def __init__(self, M: int, H: int, I: int, act: str = "gelu_tanh", dtype: str = "f16",
                 policy: str = "tile_sync", layers: int = 1):
        self.M, self.H, self.I = int(M), int(H), int(I)
        self.act, self.dtype, self.policy, self.layers = act, dtype, policy, int(layers)
        if self.layers == 1:
            self.h = mlp_chain_create(M, H, I, ACTS[act], DTYPES[dtype], POLICIES[policy])
        else:
            self.h = mlp_chain_create_layers(M, H, I, ACTS[act], DTYPES[dtype], POLICIES[policy], self.layers)

    def close(self):
        if self.h:
            mlp_chain_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    @staticmethod
    def _stream(stream):
        if stream is not None:
            return int(getattr(stream, "cuda_stream", stream))
        import torch
        return int(torch.cuda.current_stream().cuda_stream)

    def set_weight_ld(self, ldw1: int, ldw2: int):
        """Row strides (elements) of the weights later runs read; weight
        tensors are then 2-D views with those row strides."""
        mlp_chain_set_weight_ld(self.h, ldw1, ldw2)
        self.ld = {"w1": int(ldw1), "w2": int(ldw2)}

    def _shapes(self, x, w1, w2, out):
        g = 2 if self.act == "swiglu" else 1
        want = {"x": (self.M, self.H), "w1": (self.H, g * self.I), "w2": (self.I, self.H),
                "out": (self.M, self.H)}
        ld = getattr(self, "ld", {"w1": g * self.I, "w2": self.H})
        for name, t in (("x", x), ("w1", w1), ("w2", w2), ("out", out)):
            if t is None:
                continue
            if tuple(t.shape) != want[name]:
                raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {want[name]}")
            rows = (ld[name], 1) if name in ld else (want[name][1], 1)
            if not t.is_cuda or tuple(t.stride()) != rows or t.element_size() != 2:
                raise ValueError(f"{name} must be a 2-byte device tensor with row stride {rows[0]}")

    def run(self, x, w1, w2, out, stream=None):
        self._shapes(x, w1, w2, out)
        mlp_chain_run(self.h, x.data_ptr(), w1.data_ptr(), w2.data_ptr(), out.data_ptr(),
                      self._stream(stream))
        return out

    def run_layers(self, x, w1s, w2s, out, stream=None):
        """One pass of a multi-layer chain: `w1s` / `w2s` are sequences of the
        layers' weight tensors."""
        if len(w1s) != self.layers or len(w2s) != self.layers:
            raise ValueError(f"expected {self.layers} weights per GEMM, got {len(w1s)} and {len(w2s)}")
        for w1, w2 in zip(w1s, w2s):
            self._shapes(x, w1, w2, out)
        mlp_chain_run_layers(self.h, x.data_ptr(), [w.data_ptr() for w in w1s], [w.data_ptr() for w in w2s],
                             out.data_ptr(), self._stream(stream))
        return out

    def run_phase(self, phase, x=None, w1=None, w2=None, out=None, stream=None):
        self._shapes(x, w1, w2, out)
        p = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
        mlp_chain_run_phase(self.h, phase, p(x), p(w1), p(w2), p(out), self._stream(stream))

    def status(self) -> int:
        return mlp_chain_status(self.h)

    def info(self) -> dict:
        return mlp_chain_info(self.h)

    def set_config(self, cfg: int):
        mlp_chain_debug_set_config(self.h, cfg)

    def set_split(self, s1: int, s2: int):
        mlp_chain_debug_set_split(self.h, s1, s2)

    def set_grid(self, grid: int):
        mlp_chain_debug_set_grid(self.h, grid)

    def set_order(self, order: int):
        mlp_chain_debug_set_order(self.h, order)

    def set_epoch(self, epoch: int):
        mlp_chain_debug_set_epoch(self.h, epoch)

    def set_spin_limit(self, limit: int):
        mlp_chain_debug_set_spin_limit(self.h, limit)

    def skip_producer(self, tile: int):
        mlp_chain_debug_skip_producer(self.h, tile)

    def trace(self, enable: bool = True):
        """Attach a timeline buffer (a device int64 tensor of 4 words per
        ticket) to the fused runs, or detach it; returns the buffer."""
        import torch
        if not enable:
            mlp_chain_debug_set_trace(self.h, None)
            self._trace = None
            return None
        info = self.info()
        n = (info["T1"] * info["S1"] + info["T2"] * info["S2"]) * info["layers"]
        self._trace = torch.zeros((n, 4), dtype=torch.int64, device="cuda")
        mlp_chain_debug_set_trace(self.h, self._trace.data_ptr())
        return self._trace

    def read_intermediate(self, stream=None):
        """Copy of the intermediate T [M, I] left by the last run (a device tensor)."""
        import torch
        dt = torch.float16 if self.dtype == "f16" else torch.bfloat16
        t = torch.empty((self.M, self.I), dtype=dt, device="cuda")
        mlp_chain_debug_read_intermediate(self.h, t.data_ptr(), self._stream(stream))
        return t
