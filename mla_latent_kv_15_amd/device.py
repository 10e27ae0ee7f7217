"""Moves seeded host arrays to and from device tensors (storage format only)."""
from __future__ import annotations

import numpy as np
import torch

from . import inputs


def tensor(arr: "inputs.Array | np.ndarray", device="cuda") -> torch.Tensor:
    """bf16 arrays travel as their exact bit patterns; fp32 as is."""
    if isinstance(arr, inputs.Array):
        if arr.dtype == "bf16":
            t = torch.from_numpy(np.ascontiguousarray(arr.bits).view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(np.ascontiguousarray(arr.f32))
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.to(device)


def bits_tensor(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float32).numpy().astype(np.float64)


def weights(ws: dict, device="cuda") -> dict:
    return {k: tensor(v, device) for k, v in ws.items()}


def storage_dtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    # torch's caching allocator returns blocks aligned to at least 512 bytes
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
