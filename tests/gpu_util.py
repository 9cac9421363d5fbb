"""Helpers shared by the GPU parity tests."""
import numpy as np
import torch


def rel_err(y, ref):
    """max|y - ref| / max|ref| (the logits tolerance metric)."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.abs(y - ref).max() / max(np.abs(ref).max(), 1e-30))


def ws(nbytes, device):
    w = torch.zeros(nbytes, dtype=torch.uint8, device=device)
    return w


def codes_i32(U, device):
    return torch.tensor(np.asarray(U, dtype=np.int64).astype(np.int32), device=device)


def log(msg):
    print(msg, flush=True)
