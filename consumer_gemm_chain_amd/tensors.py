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
