"""Device-memory plumbing: numpy arrays -> torch device tensors.

bf16 values travel as uint16 bit patterns (viewed as int16 for torch); the
library reads the raw bytes.
"""
from __future__ import annotations

import numpy as np


def to_device(arr: np.ndarray, device: str = "cuda"):
    import torch
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def empty_like_bytes(n_bytes: int, device: str = "cuda"):
    import torch
    return torch.empty(n_bytes, dtype=torch.uint8, device=device)
