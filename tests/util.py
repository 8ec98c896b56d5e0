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


def row_errors(got, ref, block=32, floor_frac=0.05):
    """Worst per-row relative error of [rows, d] (each row's error over
    max(its norm, floor_frac x the RMS row norm), so a row that is nearly
    zero is judged against the unit's scale) and worst rel-L2 over blocks of
    `block` consecutive rows: an error confined to one chunk or to a
    sequence's last partial chunk shows here even where the whole-unit
    rel-L2 averages it away."""
    got = got.detach().cpu().double().numpy() if hasattr(got, "detach") else np.asarray(got, np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    got = got.reshape(len(got), -1)
    ref = ref.reshape(len(ref), -1)
    err = np.linalg.norm(got - ref, axis=1)
    nrm = np.linalg.norm(ref, axis=1)
    if len(nrm) == 0:
        return 0.0, 0.0
    floor = max(floor_frac * float(np.sqrt(np.mean(nrm ** 2))), 1e-300)
    row = float(np.max(err / np.maximum(nrm, floor)))
    worst = 0.0
    for s in range(0, len(ref), block):
        worst = max(worst, rel_l2(got[s:s + block], ref[s:s + block]))
    return row, worst


# per-row and per-32-row-block bars for 16-bit outputs: one bf16 rounding is
# at most 2^-8 relative per element (about 1.7e-3 RMS), so a row can reach
# about 4e-3 from the output rounding alone
ROW_TOL_16 = 1e-2
BLOCK_TOL_16 = 4e-3
