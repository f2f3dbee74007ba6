"""Moves a generated Workload to torch tensors on a device (plumbing only)."""
from __future__ import annotations

import numpy as np
import torch


def _io_tensor(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


def to_torch(w, device="cuda") -> dict:
    out = {
        "q": _io_tensor(w.q, w.dtype, device),
        "k": _io_tensor(w.k, w.dtype, device),
        "v": _io_tensor(w.v, w.dtype, device),
        "g": torch.from_numpy(w.g).to(device),
        "beta": torch.from_numpy(w.beta).to(device),
        "cu_seqlens": torch.from_numpy(w.cu_seqlens.astype(np.int64)).to(device),
        "S0": None if w.S0 is None else torch.from_numpy(w.S0).to(device),
    }
    if w.seg_start is not None:
        out["seg_start"] = torch.from_numpy(w.seg_start.astype(np.int64)).to(device)
    return out


def to_numpy_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def decode_to_torch(b, device="cuda") -> dict:
    return {
        "q": _io_tensor(b.q, b.dtype, device),
        "k": _io_tensor(b.k, b.dtype, device),
        "v": _io_tensor(b.v, b.dtype, device),
        "g": torch.from_numpy(b.g).to(device),
        "beta": torch.from_numpy(b.beta).to(device),
        "pool": torch.from_numpy(b.pool).to(device),
        "read_idx": torch.from_numpy(b.read_idx).to(device),
        "write_idx": torch.from_numpy(b.write_idx).to(device),
    }


def conv_to_torch(c, device="cuda") -> dict:
    return {
        "x": _io_tensor(c.x, c.dtype, device),
        "cu_seqlens": torch.from_numpy(c.cu_seqlens).to(device),
        "weight": torch.from_numpy(c.weight).to(device),
        "bias": torch.from_numpy(c.bias).to(device),
        "windows": _io_tensor(c.windows, c.dtype, device),
        "read_idx": torch.from_numpy(c.read_idx).to(device),
        "write_idx": torch.from_numpy(c.write_idx).to(device),
    }
