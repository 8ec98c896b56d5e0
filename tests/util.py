"""Shared helpers for the GPU tests (no method arithmetic here)."""
import numpy as np
import torch


def rel_l2(got, ref):
    got = got.detach().cpu().double().numpy() if hasattr(got, "detach") else np.asarray(got, np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def to_dev(d, device="cuda"):
    out = {}
    for key, val in d.items():
        out[key] = val.to(device) if isinstance(val, torch.Tensor) else val
    return out


# tolerances: relative L2 error against the fp64 oracle
TOL = {"f32": 1e-5, "bf16": 2e-3, "f16": 2e-3}
