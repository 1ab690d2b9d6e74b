"""Device-memory plumbing for libcca callers: host arrays to torch device
tensors in the storage type, workspaces, and back to float64 on the host.
No step of the forward pass is computed here."""

from __future__ import annotations

import numpy as np
import torch


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 arrays are bf16 bit patterns; float32 arrays stay fp32."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    if a.dtype == np.float32:
        return torch.from_numpy(a).to(device)
    raise TypeError(f"unsupported host dtype {a.dtype}")


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 values of a bf16 / fp16 / fp32 device tensor."""
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A byte tensor of at least nbytes (torch's allocations are 256-byte aligned)."""
    t = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
    assert t.data_ptr() % 256 == 0
    return t


def storage_dtype(dtype: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
