"""Device-tensor marshalling of uint16 bit patterns (fp16 / bf16) for the
binding's callers: numpy bits -> torch device tensor and back."""
from __future__ import annotations

import numpy as np


def torch_dtype(dtype: str):
    import torch
    return torch.float16 if dtype == "f16" else torch.bfloat16


def to_dev(bits: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda")
    return t.view(torch_dtype(dtype))


def from_dev(t) -> np.ndarray:
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def empty_dev(shape, dtype: str):
    import torch
    return torch.empty(shape, dtype=torch_dtype(dtype), device="cuda")


def to_dev_rows(bits: np.ndarray, dtype: str, ld: int):
    """A 2-D device tensor of `bits` whose rows lie `ld` elements apart (a
    view into a zero-filled [rows, ld] allocation), for weights with padded
    rows (mlp_chain_set_weight_ld)."""
    import torch
    rows, cols = bits.shape
    if ld == cols:
        return to_dev(bits, dtype)
    base = torch.zeros((rows, ld), dtype=torch_dtype(dtype), device="cuda")
    view = base[:, :cols]
    view.copy_(to_dev(bits, dtype))
    return view
