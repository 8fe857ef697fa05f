"""Shared helpers for the GPU parity tests (marshalling numpy <-> torch, error metric)."""
import numpy as np


def rel_err(a, b):
    """max |a - b| / max |b| over the whole tensor (all batches, heads, tokens, columns)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if b.size == 0:
        return 0.0
    m = np.max(np.abs(b))
    return float(np.max(np.abs(a - b)) / (m if m > 0 else 1.0))


def to_device(x, device="cuda", bf16=False):
    import torch
    if x is None:
        return None
    if bf16 and x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def to_host(t):
    import torch
    if t is None:
        return None
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.numpy().astype(np.float64)


TOL = {"f32": 1e-5, "bf16": 1e-2}
