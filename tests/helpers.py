"""Shared helpers for the GPU tests (conversions and error metrics only)."""
import numpy as np
import torch


def rel_inf(x, ref) -> float:
    """max |x - ref| / max |ref| (infinity-norm relative error of a tensor)."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max() if ref.size else 0.0
    if den == 0:
        return float(np.abs(x).max()) if x.size else 0.0
    return float(np.abs(x - ref).max() / den)


def rel_fro(x, ref) -> float:
    """||x - ref||_2 / ||ref||_2 over all elements (Frobenius-norm relative error)."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = float(np.linalg.norm(ref))
    if den == 0:
        return float(np.linalg.norm(x))
    return float(np.linalg.norm(x - ref) / den)


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def dev(a, dtype, device="cuda"):
    """numpy -> contiguous device tensor of dtype (bf16 via an exact float32 copy
    of values that are already bf16-representable)."""
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device).to(dtype).contiguous()


TOL = {"f32": 1e-4, "bf16": 1e-2, "mxfp8": 3e-2}
