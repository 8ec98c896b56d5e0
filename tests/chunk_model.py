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


def chunk_bwd(q, k, v, log_alpha, beta, S0, dy, dST=None, C=64):
    """Gradients of L = <dy, y> + <dST, S_T> for one head of one sequence,
    chunk by chunk in reverse, from the chunk equations above (the algebra a
    chunked backward kernel evaluates). The chunk-start states come from a
    forward sweep. Returns (dq, dk, dv, dlog_alpha, dbeta, dS0).

    Per chunk, with dS' the gradient of the chunk-end state and dY of Y:
        dE   = Kt dS' + P^T dY,            dR = T^T dE,
        dA   = -strictly_lower(dR E^T),    dP = tril(dY E^T),
        dV   = diag(beta) dR,              dX = -diag(beta gamma) dR,
        dQ   = diag(gamma) dY S^T + (dP o G) K,
        dK   = diag(e^(g_C - g)) E dS'^T + (dP o G)^T Q + dX S^T + (N + N^T) K,
               N = diag(beta) (dA o G),
        dS   = gamma_C dS' + (diag(gamma) Q)^T dY + K^T dX   (to the previous chunk),
    and the gradient of the in-chunk log-decay sums g collects every place a
    decay factor appears (gamma, G, Kt, gamma_C); d log alpha is its reverse
    running sum over the chunk.
    """
    T = q.shape[0]
    dk_, dv_ = q.shape[1], v.shape[1]
    starts = list(range(0, T, C))
    states = []
    S = np.array(S0, dtype=np.float64)
    for c0 in starts:
        states.append(S.copy())
        c1 = min(T, c0 + C)
        K, V, b = k[c0:c1], v[c0:c1], beta[c0:c1]
        g = np.cumsum(log_alpha[c0:c1])
        G = np.tril(np.exp(np.minimum(g[:, None] - g[None, :], 0.0)))
        A = np.tril(b[:, None] * (K @ K.T) * G, -1)
        E = np.linalg.solve(np.eye(len(b)) + A, b[:, None] * (V - np.exp(g)[:, None] * (K @ S)))
        S = np.exp(g[-1]) * S + (np.exp(g[-1] - g)[:, None] * K).T @ E
    dS = np.zeros((dk_, dv_)) if dST is None else np.array(dST, dtype=np.float64)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dla, dbeta = np.zeros(T), np.zeros(T)
    for ci in range(len(starts) - 1, -1, -1):
        c0 = starts[ci]
        c1 = min(T, c0 + C)
        S = states[ci]
        Q, K, V, b = q[c0:c1], k[c0:c1], v[c0:c1], beta[c0:c1]
        g = np.cumsum(log_alpha[c0:c1])
        gam = np.exp(g)
        gC = g[-1]
        G = np.tril(np.exp(np.minimum(g[:, None] - g[None, :], 0.0)))
        KK = K @ K.T
        A = np.tril(b[:, None] * KK * G, -1)
        Tm = np.linalg.inv(np.eye(len(b)) + A)
        X = K @ S
        R = b[:, None] * (V - gam[:, None] * X)
        E = Tm @ R
        P = np.tril((Q @ K.T) * G)
        kdec = np.exp(gC - g)
        dY = dy[c0:c1]
        # chunk-end state S' = gamma_C S + Kt^T E
        dS_prev = np.exp(gC) * dS
        dgC = np.exp(gC) * np.sum(S * dS)
        dKt = E @ dS.T
        dE = (kdec[:, None] * K) @ dS
        cr = kdec * np.sum(K * dKt, axis=1)
        dK = kdec[:, None] * dKt
        dg = -cr
        dgC += cr.sum()
        # Y = diag(gamma) Q S + P E
        dQ = gam[:, None] * (dY @ S.T)
        dS_prev += (gam[:, None] * Q).T @ dY
        dg += gam * np.sum((Q @ S) * dY, axis=1)
        dP = np.tril(dY @ E.T)
        dE += P.T @ dY
        dPG = dP * G
        dQ += dPG @ K
        dK += dPG.T @ Q
        w = dP * P
        dg += w.sum(1) - w.sum(0)
        # E = T R, T = (I + A)^-1
        dR = Tm.T @ dE
        dA = -np.tril(dR @ E.T, -1)
        # R = diag(beta)(V - diag(gamma) X), X = K S
        dV = b[:, None] * dR
        db = np.sum(dR * (V - gam[:, None] * X), axis=1)
        dX = -(b * gam)[:, None] * dR
        dg += -(b * gam) * np.sum(dR * X, axis=1)
        dK += dX @ S.T
        dS_prev += K.T @ dX
        # A = strictly_lower(diag(beta)(K K^T o G))
        db += np.sum(dA * KK * G, axis=1)
        Nm = b[:, None] * dA * G
        dK += (Nm + Nm.T) @ K
        w2 = dA * A
        dg += w2.sum(1) - w2.sum(0)
        dg[-1] += dgC
        dla_sum = np.cumsum(dg[::-1])[::-1]
        # the same d log alpha without forming cancelling pairs (the form the
        # kernel uses): local terms' suffix sums, the decay factors' block
        # sums over r >= s > i, the Kt terms' exclusive prefix, gamma_C <S, dS'>
        Wd = np.tril(w + w2, -1)
        local = gam * np.sum((Q @ S) * dY, axis=1) - (b * gam) * np.sum(dR * X, axis=1)
        n_c = len(g)
        blocks = np.array([Wd[s:, :s].sum() for s in range(n_c)])
        excl = np.concatenate([[0.0], np.cumsum(cr)[:-1]])
        dla_direct = (np.cumsum(local[::-1])[::-1] + blocks + excl
                      + np.exp(gC) * np.sum(S * dS))
        assert np.allclose(dla_direct, dla_sum, rtol=1e-9, atol=1e-9 * max(1.0, abs(dla_sum).max()))
        dla[c0:c1] = dla_direct
        dq[c0:c1], dk[c0:c1], dv[c0:c1], dbeta[c0:c1] = dQ, dK, dV, db
        dS = dS_prev
    return dq, dk, dv, dla, dbeta, dS
