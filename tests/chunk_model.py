"""fp64 NumPy model of the chunk equations the HIP prefill kernel evaluates.

Test-side design aid, not the oracle: it is checked against the oracle's
token recurrence (tests/test_chunk_model.py) so the algebra the kernel relies
on is pinned before any kernel exists. It shares no code with the kernel.

Derivation (from the erase-write rule of the page
"NLP——技术报告解读-Qwen3.8-Flash-Next", section "Gated DeltaNet 核心机制").
Inside a chunk of C tokens starting from state S, with g_r the in-chunk
cumulative sum of log alpha, gamma_r = exp(g_r), G_ri = exp(g_r - g_i) (r >= i)
and the scaled errors E_r = beta_r e_r:

    S_r          = gamma_r S + sum_{i<=r} G_ri k_i E_i^T
    E_r          = beta_r (v_r - gamma_r S^T k_r - sum_{i<r} G_ri (k_r.k_i) E_i)
    (I + A) E    = diag(beta) (V - diag(gamma) K S),
                   A = strictly_lower(diag(beta) (K K^T o G))
    y_r          = S_r^T q_r = gamma_r S^T q_r + sum_{i<=r} G_ri (q_r.k_i) E_i
    S_next       = gamma_C S + sum_i exp(g_C - g_i) k_i E_i^T

so per chunk:  X = K S;  R = diag(beta)(V - gamma o X);  E = (I + A)^{-1} R;
Y = diag(gamma) Q S + tril(Q K^T o G) E;  S <- gamma_C S + Kt^T E with
Kt_r = exp(g_C - g_r) k_r. Only exponents of non-positive numbers appear.
"""
import numpy as np


def unit_lower_inverse_blocked(A, bs=16):
    """(I + A)^{-1} for strictly lower A by blocks: diagonal blocks by forward
    substitution, off-diagonal blocks T_ij = -T_ii sum_{j<=m<i} A_im T_mj."""
    C = A.shape[0]
    nb = (C + bs - 1) // bs
    T = np.zeros_like(A)
    for b in range(nb):
        s, e = b * bs, min(C, (b + 1) * bs)
        Tb = np.eye(e - s)
        for r in range(1, e - s):
            Tb[r, :r] = -A[s + r, s:s + r] @ Tb[:r, :r]
        T[s:e, s:e] = Tb
    for i in range(nb):
        si, ei = i * bs, min(C, (i + 1) * bs)
        for j in range(i - 1, -1, -1):
            sj, ej = j * bs, min(C, (j + 1) * bs)
            acc = np.zeros((ei - si, ej - sj))
            for m in range(j, i):
                sm, em = m * bs, min(C, (m + 1) * bs)
                acc += A[si:ei, sm:em] @ T[sm:em, sj:ej]
            T[si:ei, sj:ej] = -T[si:ei, si:ei] @ acc
    return T


def chunk_fwd(q, k, v, log_alpha, beta, S0, C=64, blocked=True):
    """One head of one sequence: q, k [T, dk]; v [T, dv]; gates [T];
    S0 [dk, dv]. Returns (y [T, dv], S_T)."""
    T = q.shape[0]
    S = np.array(S0, dtype=np.float64)
    y = np.zeros((T, v.shape[1]))
    for c0 in range(0, T, C):
        c1 = min(T, c0 + C)
        Q, K, V = q[c0:c1], k[c0:c1], v[c0:c1]
        b = beta[c0:c1]
        g = np.cumsum(log_alpha[c0:c1])
        gam = np.exp(g)
        diff = g[:, None] - g[None, :]
        G = np.tril(np.exp(np.minimum(diff, 0.0)))  # r >= i only
        A = np.tril(b[:, None] * (K @ K.T) * G, -1)
        Tm = unit_lower_inverse_blocked(A) if blocked else np.linalg.inv(np.eye(len(b)) + A)
        X = K @ S
        R = b[:, None] * (V - gam[:, None] * X)
        E = Tm @ R
        P = np.tril((Q @ K.T) * G)
        y[c0:c1] = gam[:, None] * (Q @ S) + P @ E
        Kt = np.exp(g[-1] - g)[:, None] * K
        S = gam[-1] * S + Kt.T @ E
    return y, S
