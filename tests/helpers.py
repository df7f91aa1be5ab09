"""Comparison helpers for the GPU parity tests (no arithmetic of the method)."""
import numpy as np


def bf16_round(a):
    """Round float values to bfloat16 (nearest-even) and return float64."""
    import torch
    return torch.as_tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def to_dev(a, dtype):
    import torch
    return torch.as_tensor(np.asarray(a, dtype=np.float32)).to(dtype).cuda()


def to_np(t):
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def rel_err(a, ref):
    a = np.asarray(a, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(a - ref) / den) if den > 0 else float(np.linalg.norm(a))


def max_rel(a, ref):
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    m = np.abs(ref).max()
    return float(np.abs(a - ref).max() / m) if m > 0 else float(np.abs(a).max())


def cosine(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 and nb == 0:
        return 1.0
    return float(a @ b / (na * nb))


def case(msg):
    """Name the case on stdout before a GPU step, so a failing run shows it."""
    print(f"\n[case] {msg}", flush=True)
