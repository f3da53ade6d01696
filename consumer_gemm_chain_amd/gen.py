"""Seeded synthetic inputs for the MLP chain (shared by the tests, the smoke
check and the benchmark).

This module only draws random numbers and casts them to the storage dtype
with numpy's / torch's own fp32 -> fp16 / bf16 casts (round to nearest even).
It holds none of the chain's arithmetic.

The workloads stand in for the pages' MLPs: GPT-3 175B (H=12288) and LLaMA
65.2B (H=8192) under 8-way model parallelism in FP16 (CuSync README, paragraph
on the MLP graphs), and GPT-3 175B / Llama-2 70B (FLUX summary card, Key
points: test setup).  No trained weights are used: Gaussian (or uniform)
weights of the same shapes stand in, seeded per workload.

Seeds: workload c uses seed 100*c for X, 100*c+1 for W1 (gate and up drawn
together as one [H, 2I] matrix for SwiGLU) and 100*c+2 for W2.  X is drawn
once at the workload's largest M, and a run at M uses its first M rows, so
rows agree across M.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

ACTS = ("none", "gelu_tanh", "swiglu")
DTYPES = ("f16", "bf16")


@dataclass(frozen=True)
class Workload:
    idx: int
    name: str
    H: int
    I: int
    act: str
    dtype: str
    dist: str           # "normal" or "uniform"
    x_scale: float      # std of X (normal) or half-width of U (uniform)
    w_scale: float      # std of W (normal) or half-width of U (uniform)
    Ms: tuple = field(default_factory=tuple)

    @property
    def g(self) -> int:
        return 2 if self.act == "swiglu" else 1

    @property
    def max_M(self) -> int:
        return max(self.Ms)

    def flops(self, M: int) -> int:
        """GEMM flops of one chain pass: 2*M*H*I*(g+1) (activation not counted)."""
        return 2 * M * self.H * self.I * (self.g + 1)

    def bytes(self, M: int) -> int:
        """Algorithmic HBM bytes of one pass: weights once, X read, Y written,
        the intermediate written and read once (2-byte elements)."""
        return 2 * (self.H * self.I * (self.g + 1) + 2 * M * self.H + 2 * M * self.I)


_U = 1.0 / math.sqrt(8192.0)

WORKLOADS = {
    0: Workload(0, "tiny_gelu_f16", 512, 2048, "gelu_tanh", "f16", "normal", 1.0, 0.02, (64,)),
    1: Workload(1, "gpt3_175b_mlp_tp8_f16", 12288, 6144, "gelu_tanh", "f16", "normal", 1.0, 0.02,
                (1, 16, 64, 256, 512, 1024, 2048)),
    2: Workload(2, "llama65b_swiglu_tp8_f16", 8192, 2752, "swiglu", "f16", "normal", 1.0, 0.02,
                (1, 64, 256, 512, 1024, 2048)),
    3: Workload(3, "llama2_70b_swiglu_tp8_bf16", 8192, 3584, "swiglu", "bf16", "normal", 1.0, 0.015,
                (128, 512, 2048, 4096, 8192)),
    4: Workload(4, "stress_square_chain_bf16", 8192, 8192, "none", "bf16", "uniform", _U, _U, (8192,)),
}


def to_bits(a: np.ndarray, dtype: str) -> np.ndarray:
    """Cast fp32 values to fp16/bf16 (round to nearest even) and return the
    uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "f16":
        return a.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        import torch
        return torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def from_bits(b: np.ndarray, dtype: str) -> np.ndarray:
    """Widen uint16 bit patterns to fp32 with numpy/torch casts."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    if dtype == "f16":
        return b.view(np.float16).astype(np.float32)
    if dtype == "bf16":
        return (b.astype(np.uint32) << 16).view(np.float32)
    raise ValueError(dtype)


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal_bits(shape, seed: int, std: float, dtype: str) -> np.ndarray:
    z = _rng(seed).standard_normal(size=shape, dtype=np.float32)
    z *= np.float32(std)
    return to_bits(z, dtype)


def uniform_bits(shape, seed: int, half_width: float, dtype: str) -> np.ndarray:
    u = _rng(seed).random(size=shape, dtype=np.float32)
    u = u * np.float32(2.0) - np.float32(1.0)          # U[-1, 1)
    u *= np.float32(half_width)
    return to_bits(u, dtype)


def sparse_int_bits(shape, seed: int, density: float, dtype: str, values=(-1.0, 1.0)) -> np.ndarray:
    """Entries drawn from `values` with probability `density`, else 0 (exact
    small integers in either dtype)."""
    r = _rng(seed)
    mask = r.random(size=shape) < density
    v = r.choice(np.asarray(values, np.float32), size=shape)
    return to_bits(np.where(mask, v, np.float32(0.0)), dtype)


def _draw(w: Workload, shape, seed: int, scale: float) -> np.ndarray:
    if w.dist == "normal":
        return normal_bits(shape, seed, scale, w.dtype)
    return uniform_bits(shape, seed, scale, w.dtype)


def workload_inputs(w: Workload | int, M: int | None = None, max_M: int | None = None):
    """Return (x [M,H], w1 [H,g*I], w2 [I,H]) as uint16 bit patterns for a
    workload.  X is drawn at max_M (default: the workload's largest M) and
    sliced to M rows."""
    if isinstance(w, int):
        w = WORKLOADS[w]
    M = w.max_M if M is None else int(M)
    mm = max(M, w.max_M if max_M is None else int(max_M))
    base = 100 * w.idx
    x = _draw(w, (mm, w.H), base + 0, w.x_scale)[:M]
    w1 = _draw(w, (w.H, w.g * w.I), base + 1, w.w_scale)
    w2 = _draw(w, (w.I, w.H), base + 2, w.w_scale)
    return np.ascontiguousarray(x), w1, w2


def weights(w: Workload | int):
    """Only the weights of a workload (w1, w2)."""
    if isinstance(w, int):
        w = WORKLOADS[w]
    base = 100 * w.idx
    return (_draw(w, (w.H, w.g * w.I), base + 1, w.w_scale),
            _draw(w, (w.I, w.H), base + 2, w.w_scale))


def x_rows(w: Workload | int, M: int, max_M: int | None = None) -> np.ndarray:
    if isinstance(w, int):
        w = WORKLOADS[w]
    mm = max(M, w.max_M if max_M is None else int(max_M))
    return np.ascontiguousarray(_draw(w, (mm, w.H), 100 * w.idx, w.x_scale)[:M])


def random_case(M: int, H: int, I: int, act: str, dtype: str, seed: int,
                x_std: float = 1.0, w_std: float = 0.05):
    """A small seeded case of arbitrary shape (normal X and W)."""
    g = 2 if act == "swiglu" else 1
    x = normal_bits((M, H), seed * 3 + 0, x_std, dtype)
    w1 = normal_bits((H, g * I), seed * 3 + 1, w_std, dtype)
    w2 = normal_bits((I, H), seed * 3 + 2, w_std, dtype)
    return x, w1, w2
