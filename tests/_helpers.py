"""Shared test helpers: the parity metric and GPU tensor marshalling."""
import numpy as np

# Parity bar (max relative error, defined below) by input precision.
TOL = {"f32": 1e-5, "bf16": 3e-3}


def max_rel_err(actual, ref):
    """max |actual - ref| / max |ref| over the whole tensor."""
    actual = np.asarray(actual, np.float64)
    ref = np.asarray(ref, np.float64)
    denom = np.abs(ref).max()
    if denom == 0:
        return float(np.abs(actual).max())
    return float(np.abs(actual - ref).max() / denom)


def to_dev(arr, dtype, device="cuda"):
    """float32 numpy array (bf16-exact values for "bf16") -> torch tensor."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(arr)).to(device)
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t


def to_np(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy()
