"""Shared test helpers (comparison metrics, device conversions)."""
import numpy as np


def np64(x):
    """torch tensor / array -> float64 numpy (bf16 upcast exactly)."""
    if hasattr(x, "detach"):
        import torch
        x = x.detach().to("cpu")
        if x.dtype == torch.bfloat16:
            x = x.to(torch.float32)
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


def max_rel_err(got, ref) -> float:
    """max |got - ref| / max |ref| over the tensor (0 if both are all zero)."""
    got, ref = np64(got), np64(ref)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(got - ref)) if ref.size else 0.0
    if den == 0.0:
        return float(num)
    return float(num / den)


TOL = {"fp32": 1e-4, "bf16": 2e-2}
