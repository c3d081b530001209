"""Upload a seeded workload to the GPU as torch tensors (storage bits kept:
bf16 arrays arrive as their raw 16-bit patterns and are viewed as bfloat16)."""

from __future__ import annotations

import numpy as np


def to_device(arr: np.ndarray, dtype: str, device="cuda"):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16))
        return t.to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def upload(w, device="cuda") -> dict:
    return {k: to_device(v, w.dtypes[k], device) for k, v in w.arrays.items()}
