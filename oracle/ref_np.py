"""NumPy twin of the C oracle, for tiny shapes (pure-Python token loop).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Written separately from ``gdn_oracle.c`` from the same definitions (page
"NLP——技术报告解读-Qwen3.8-Flash-Next", sections "Gated DeltaNet 核心机制" and
"GDN 参数化细节"), so that the C oracle and this twin pin each other.
"""
from __future__ import annotations

import numpy as np


def _segments(total, N, cu_seqlens):
    if cu_seqlens is not None:
        cu = [int(c) for c in cu_seqlens]
        return [(cu[i], cu[i + 1]) for i in range(len(cu) - 1)]
    T = total // N
    return [(n * T, (n + 1) * T) for n in range(N)]


def gdn_fwd(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None, N=1,
            form="erase_write"):
    """Per head, per token: decay, error against the decayed state, rank-1
    write, read with the new state. Shapes as in ``oracle.gdn_fwd``."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    la = np.asarray(log_alpha, dtype=np.float64)
    b = np.asarray(beta, dtype=np.float64)
    total, H, dk = q.shape
    dv = v.shape[2]
    segs = _segments(total, N, cu_seqlens)
    y = np.zeros((total, H, dv))
    S_T = np.zeros((len(segs), H, dk, dv))
    for n, (s, e) in enumerate(segs):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else np.array(S0[n, h], dtype=np.float64)
            for t in range(s, e):
                alpha = np.exp(la[t, h])
                kt, vt, qt = k[t, h], v[t, h], q[t, h]
                if form == "erase_write":
                    S_dec = alpha * S
                    err = vt - S_dec.T @ kt
                    S = S_dec + b[t, h] * np.outer(kt, err)
                else:
                    P = np.eye(dk) - b[t, h] * np.outer(kt, kt)
                    S = alpha * (P @ S) + b[t, h] * np.outer(kt, vt)
                y[t, h] = S.T @ qt
            S_T[n, h] = S
    return y, S_T


def decode_step(q, k, v, log_alpha, beta, S):
    """One token per (sequence, head): q, k [N, H, dk]; v [N, H, dv]."""
    S = np.array(S, dtype=np.float64)
    N, H, dk = np.shape(q)
    y = np.zeros((N, H, np.shape(v)[2]))
    for n in range(N):
        for h in range(H):
            alpha = np.exp(float(log_alpha[n, h]))
            kt = np.asarray(k[n, h], dtype=np.float64)
            S_dec = alpha * S[n, h]
            err = np.asarray(v[n, h], dtype=np.float64) - S_dec.T @ kt
            S[n, h] = S_dec + float(beta[n, h]) * np.outer(kt, err)
            y[n, h] = S[n, h].T @ np.asarray(q[n, h], dtype=np.float64)
    return y, S


def frontend(x, w, cu_seqlens=None, N=1, l2=True, eps=1e-6):
    """Causal depthwise conv with zero history (kernel length K = w.shape[1],
    the last tap multiplying the current token), SiLU, optional L2Norm."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    total, H, d = x.shape
    K = w.shape[1]
    wh = w.reshape(H, d, K)
    out = np.zeros_like(x)
    for (s, e) in _segments(total, N, cu_seqlens):
        for t in range(s, e):
            u = np.zeros((H, d))
            for j in range(K):
                src = t - (K - 1) + j
                if src >= s:
                    u += wh[:, :, j] * x[src]
            a = u / (1.0 + np.exp(-u))
            if l2:
                a = a / np.sqrt((a * a).sum(axis=-1, keepdims=True) + eps)
            out[t] = a
    return out


def output_gate(y, z, w=None, eps=1e-6):
    y = np.asarray(y, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    d = y.shape[-1]
    gain = 1.0 + (np.zeros(d) if w is None else np.asarray(w, dtype=np.float64))
    rms = np.sqrt((y * y).mean(axis=-1, keepdims=True) + eps)
    return (1.0 / (1.0 + np.exp(-z))) * (y / rms) * gain
