"""Pins for the fp64 oracle: properties fixed by the pages and by algebra,
never the oracle's own formula retyped.

The recurrence is the gated delta rule of the page
"NLP——技术报告解读-Qwen3.8-Flash-Next", section "Gated DeltaNet 核心机制"
(erase-write display and its closed-form equivalent).
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
from oracle import ref_np

RNG = np.random.default_rng(1234)


def _rand_case(total, H, dk, dv, rng, unit=True, s0=True, N=1):
    q = rng.standard_normal((total, H, dk))
    k = rng.standard_normal((total, H, dk))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((total, H, dv))
    la = -np.exp(rng.uniform(-4, 0, size=(1, H))) * np.log1p(np.exp(rng.standard_normal((total, H))))
    b = 1 / (1 + np.exp(-rng.standard_normal((total, H))))
    S0 = rng.standard_normal((N, H, dk, dv)) * 0.5 if s0 else None
    return q, k, v, la, b, S0


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# (A1) the erase-write form and the closed form agree --------------------------
@pytest.mark.parametrize("dk,dv,T", [(1, 1, 50), (2, 3, 40), (3, 2, 60), (8, 8, 300),
                                     (16, 5, 120), (64, 64, 200)])
def test_forms_agree(dk, dv, T):
    rng = np.random.default_rng(dk * 100 + dv)
    q, k, v, la, b, S0 = _rand_case(T, 2, dk, dv, rng)
    yA, SA = oracle.gdn_fwd(q, k, v, la, b, S0, form=oracle.FORM_ERASE_WRITE)
    yB, SB = oracle.gdn_fwd(q, k, v, la, b, S0, form=oracle.FORM_CLOSED)
    assert _rel(yA, yB) < 1e-12
    assert _rel(SA, SB) < 1e-12


# (A2) alpha = 1, beta = 0 leaves S unchanged (bit-exact) ----------------------
@pytest.mark.parametrize("form", [oracle.FORM_ERASE_WRITE, oracle.FORM_CLOSED])
def test_identity_gates_leave_state(form):
    rng = np.random.default_rng(7)
    q, k, v, la, b, S0 = _rand_case(77, 3, 8, 6, rng)
    la[:] = 0.0
    b[:] = 0.0
    y, S = oracle.gdn_fwd(q, k, v, la, b, S0, form=form)
    assert np.array_equal(S, S0)
    # reads then see the unchanged state: y_t = S0^T q_t
    expect = np.einsum("hij,thi->thj", S0[0], q)
    assert np.max(np.abs(y - expect)) < 1e-13


# (A3) orthonormal keys, beta = 1, alpha = 1, S0 = 0: reading with q = k_j
# returns exactly v_j (brute force over key orders) -----------------------------
@pytest.mark.parametrize("dk", [1, 2, 3, 4, 8])
def test_orthonormal_keys_retrieve_values(dk):
    rng = np.random.default_rng(dk)
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    dv = 3
    for n in range(1, dk + 1):
        picks = list(range(n))
        orders = itertools.permutations(picks) if n <= 4 else [tuple(rng.permutation(n))]
        for order in orders:
            keys = Qm[:, list(order)].T  # n orthonormal keys
            vals = rng.standard_normal((n, dv))
            k = keys[:, None, :]
            v = vals[:, None, :]
            la = np.zeros((n, 1))
            b = np.ones((n, 1))
            _, S = oracle.gdn_fwd(k, k, v, la, b, None)
            got = S[0, 0].T @ keys.T  # column j = S^T k_j
            assert np.max(np.abs(got - vals.T)) < 1e-13


# with decay the written value fades by the decays applied after its step,
# but not by its own step's decay (decay precedes the write) --------------------
def test_orthonormal_keys_with_decay():
    rng = np.random.default_rng(11)
    dk, dv, n = 6, 4, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm.T[:n]
    vals = rng.standard_normal((n, dv))
    la = -rng.uniform(0.0, 0.7, size=(n, 1))
    b = np.ones((n, 1))
    _, S = oracle.gdn_fwd(keys[:, None], keys[:, None], vals[:, None], la, b, None)
    for j in range(n):
        fade = np.exp(la[j + 1:, 0].sum())
        assert np.max(np.abs(S[0, 0].T @ keys[j] - fade * vals[j])) < 1e-13


# (A4) beta = 1, q = k, |k| = 1 => y_t = v_t for any alpha and S0 -------------
def test_full_write_then_read_same_key():
    rng = np.random.default_rng(5)
    q, k, v, la, b, S0 = _rand_case(150, 2, 16, 16, rng)
    b[:] = 1.0
    y, _ = oracle.gdn_fwd(k, k, v, la, b, S0)
    assert np.max(np.abs(y - v)) < 1e-12


# (A5) beta = 0 => pure decay: S_T = exp(sum log alpha) S0 -----------------------
def test_pure_decay():
    rng = np.random.default_rng(6)
    q, k, v, la, b, S0 = _rand_case(90, 3, 5, 7, rng)
    b[:] = 0.0
    y, S = oracle.gdn_fwd(q, k, v, la, b, S0)
    for h in range(3):
        assert _rel(S[0, h], np.exp(la[:, h].sum()) * S0[0, h]) < 1e-13
        g = np.cumsum(la[:, h])
        expect = np.exp(g)[:, None] * (q[:, h] @ S0[0, h])
        assert _rel(y[:, h], expect) < 1e-13


# (A6) dk = dv = 1: the scalar recurrence unrolled by hand -----------------------
def test_scalar_closed_form():
    rng = np.random.default_rng(8)
    T = 40
    k = rng.uniform(-1, 1, size=(T, 1, 1))
    q = rng.uniform(-1, 1, size=(T, 1, 1))
    v = rng.standard_normal((T, 1, 1))
    la = -rng.uniform(0, 0.5, size=(T, 1))
    b = rng.uniform(0, 1, size=(T, 1))
    s0 = 0.3
    y, S = oracle.gdn_fwd(q, k, v, la, b, np.full((1, 1, 1, 1), s0))
    a = np.exp(la[:, 0]) * (1 - b[:, 0] * k[:, 0, 0] ** 2)  # multiplier of s_{t-1}
    c = b[:, 0] * k[:, 0, 0] * v[:, 0, 0]  # additive part
    for t in range(T):
        # s_t = prod_{u<=t} a_u * s0 + sum_{i<=t} prod_{i<u<=t} a_u * c_i
        st = np.prod(a[:t + 1]) * s0 + sum(np.prod(a[i + 1:t + 1]) * c[i] for i in range(t + 1))
        assert abs(y[t, 0, 0] - st * q[t, 0, 0]) < 1e-13
    assert abs(S[0, 0, 0, 0] - st) < 1e-13


# rotations of key space and of value space act as the algebra says --------------
def test_rotation_equivariance():
    rng = np.random.default_rng(9)
    dk, dv = 6, 4
    q, k, v, la, b, S0 = _rand_case(60, 2, dk, dv, rng)
    R, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    M, _ = np.linalg.qr(rng.standard_normal((dv, dv)))
    y, S = oracle.gdn_fwd(q, k, v, la, b, S0)
    # keys/queries rotated, state rotated on its key side: y unchanged
    y2, S2 = oracle.gdn_fwd(q @ R.T, k @ R.T, v, la, b, np.einsum("ij,nhjk->nhik", R, S0))
    assert _rel(y2, y) < 1e-12
    assert _rel(S2, np.einsum("ij,nhjk->nhik", R, S)) < 1e-12
    # values rotated on the right: y and S rotate the same way
    y3, S3 = oracle.gdn_fwd(q, k, v @ M, la, b, S0 @ M)
    assert _rel(y3, y @ M) < 1e-12
    assert _rel(S3, S @ M) < 1e-12


# (A7) C oracle == NumPy twin ---------------------------------------------------
@pytest.mark.parametrize("form", ["erase_write", "closed"])
def test_c_matches_numpy_twin(form):
    rng = np.random.default_rng(10)
    lengths = [1, 5, 17, 33]
    total = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    q, k, v, la, b, S0 = _rand_case(total, 2, 8, 5, rng, N=len(lengths))
    yc, Sc = oracle.gdn_fwd(q, k, v, la, b, S0, cu_seqlens=cu,
                            form=oracle.FORM_ERASE_WRITE if form == "erase_write" else oracle.FORM_CLOSED)
    yn, Sn = ref_np.gdn_fwd(q, k, v, la, b, S0, cu_seqlens=cu, form=form)
    assert _rel(yc, yn) < 1e-13 and _rel(Sc, Sn) < 1e-13


def test_column_blocks_and_threads_do_not_change_result():
    rng = np.random.default_rng(12)
    q, k, v, la, b, S0 = _rand_case(64, 2, 8, 12, rng, N=2)
    q, k, v, la, b = (np.concatenate([x, x[::-1]]) for x in (q, k, v, la, b))
    base = oracle.gdn_fwd(q, k, v, la, b, S0, N=2, nthreads=1, col_blocks=1)
    for cb, nt in [(3, 2), (12, 4), (5, 8)]:
        other = oracle.gdn_fwd(q, k, v, la, b, S0, N=2, nthreads=nt, col_blocks=cb)
        assert np.array_equal(base[0], other[0]) and np.array_equal(base[1], other[1])


def test_varlen_equals_per_sequence():
    rng = np.random.default_rng(13)
    lengths = [3, 64, 65, 1, 20]
    total = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    q, k, v, la, b, S0 = _rand_case(total, 2, 8, 8, rng, N=len(lengths))
    y, S = oracle.gdn_fwd(q, k, v, la, b, S0, cu_seqlens=cu)
    for n, (s, e) in enumerate(zip(cu[:-1], cu[1:])):
        yn, Sn = oracle.gdn_fwd(q[s:e], k[s:e], v[s:e], la[s:e], b[s:e], S0[n:n + 1])
        assert np.array_equal(y[s:e], yn) and np.array_equal(S[n], Sn[0])


def test_split_resume_equals_one_pass():
    rng = np.random.default_rng(14)
    q, k, v, la, b, S0 = _rand_case(100, 2, 8, 8, rng)
    y, S = oracle.gdn_fwd(q, k, v, la, b, S0)
    for t0 in (0, 1, 37, 99, 100):
        y1, S1 = oracle.gdn_fwd(q[:t0], k[:t0], v[:t0], la[:t0], b[:t0], S0)
        y2, S2 = oracle.gdn_fwd(q[t0:], k[t0:], v[t0:], la[t0:], b[t0:], S1)
        assert _rel(np.concatenate([y1, y2]), y) < 1e-14 and _rel(S2, S) < 1e-14


def test_decode_steps_equal_fwd():
    rng = np.random.default_rng(15)
    T, N, H, dk, dv = 20, 3, 2, 8, 6
    q, k, v, la, b, S0 = _rand_case(T * N, H, dk, dv, rng, N=N)
    # layout [N*T] rows: sequence n occupies rows n*T .. n*T+T-1
    y, S = oracle.gdn_fwd(q, k, v, la, b, S0, N=N)
    St = S0.copy()
    for t in range(T):
        rows = np.arange(N) * T + t
        yt, St = oracle.decode_step(q[rows], k[rows], v[rows], la[rows], b[rows], St)
        assert _rel(yt, y[rows]) < 1e-13
    assert _rel(St, S) < 1e-13


def test_decode_c_matches_numpy():
    rng = np.random.default_rng(16)
    N, H, dk, dv = 4, 3, 8, 5
    q, k, v, la, b, S0 = _rand_case(N, H, dk, dv, rng, N=N)
    yc, Sc = oracle.decode_step(q, k, v, la, b, S0)
    yn, Sn = ref_np.decode_step(q, k, v, la, b, S0)
    assert _rel(yc, yn) < 1e-14 and _rel(Sc, Sn) < 1e-14


def test_empty_sequence_keeps_state():
    rng = np.random.default_rng(17)
    lengths = [0, 4, 0]
    cu = np.array([0, 0, 4, 4], dtype=np.int32)
    q, k, v, la, b, S0 = _rand_case(4, 2, 4, 4, rng, N=3)
    _, S = oracle.gdn_fwd(q, k, v, la, b, S0, cu_seqlens=cu)
    assert np.array_equal(S[0], S0[0]) and np.array_equal(S[2], S0[2])


# front end: ShortConv -> SiLU -> L2Norm -----------------------------------------
def test_conv_matches_torch_conv1d_and_silu():
    rng = np.random.default_rng(20)
    lengths = [1, 3, 9, 30]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    H, d, K = 2, 5, 4
    x = rng.standard_normal((sum(lengths), H, d))
    w = rng.standard_normal((H * d, K)) * 0.5
    out = oracle.frontend(x, w, cu_seqlens=cu, l2=False)
    for s, e in zip(cu[:-1], cu[1:]):
        xs = torch.tensor(x[s:e].reshape(e - s, H * d).T[None], dtype=torch.float64)
        conv = torch.nn.functional.conv1d(xs, torch.tensor(w[:, None, :]), padding=K - 1,
                                          groups=H * d)[0, :, : e - s]
        expect = torch.nn.functional.silu(conv).T.reshape(e - s, H, d).numpy()
        assert np.max(np.abs(out[s:e] - expect)) < 1e-13


def test_conv_impulse_response_tap_order():
    H, d, K, T = 1, 1, 4, 10
    w = np.array([[0.1, 0.2, 0.3, 0.4]])
    x = np.zeros((T, H, d))
    x[2] = 1.0
    out = oracle.frontend(x, w, l2=False)
    silu = lambda u: u / (1 + np.exp(-u))
    # the last tap multiplies the current token, the first tap the one K-1 back
    expect = np.zeros(T)
    expect[2:6] = silu(np.array([0.4, 0.3, 0.2, 0.1]))
    expect[[0, 1, 6, 7, 8, 9]] = 0.0
    assert np.max(np.abs(out[:, 0, 0] - expect)) < 1e-15


def test_l2norm_gives_unit_rows_and_matches_twin():
    rng = np.random.default_rng(21)
    lengths = [7, 12]
    cu = np.array([0, 7, 19], dtype=np.int32)
    x = rng.standard_normal((19, 3, 16))
    w = rng.standard_normal((48, 4)) * 0.5
    out = oracle.frontend(x, w, cu_seqlens=cu, l2=True, eps=0.0)
    assert np.max(np.abs(np.linalg.norm(out, axis=-1) - 1)) < 1e-14
    out_e = oracle.frontend(x, w, cu_seqlens=cu, l2=True, eps=1e-6)
    twin = ref_np.frontend(x, w, cu_seqlens=cu, l2=True, eps=1e-6)
    assert np.max(np.abs(out_e - twin)) < 1e-14


def test_output_gate_against_torch_rms_norm():
    rng = np.random.default_rng(22)
    y = rng.standard_normal((13, 3, 32))
    z = rng.standard_normal((13, 3, 32))
    w = rng.standard_normal(32) * 0.1
    o = oracle.output_gate(y, z, w, eps=1e-6)
    ref = (torch.sigmoid(torch.tensor(z)) *
           torch.nn.functional.rms_norm(torch.tensor(y), (32,), weight=torch.tensor(1 + w), eps=1e-6))
    assert np.max(np.abs(o - ref.numpy())) < 1e-14
    assert np.max(np.abs(o - ref_np.output_gate(y, z, w, eps=1e-6))) < 1e-14
    # w = 0, sigmoid saturated, eps = 0: rows have unit RMS
    o2 = oracle.output_gate(y, np.full_like(z, 50.0), None, eps=0.0)
    assert np.max(np.abs(np.sqrt((o2 ** 2).mean(-1)) - 1)) < 1e-14


# Gates from raw pre-activations -----------------------------------------------
# log alpha = -exp(A) softplus(a + b_alpha), beta = sigmoid(b): page
# "NLP——技术报告解读-Qwen3.8-Flash-Next", section "GDN 参数化细节".
def test_gates_from_raw_against_torch_and_identities():
    rng = np.random.default_rng(23)
    H = 5
    a = rng.standard_normal((40, H)) * 6
    b = rng.standard_normal((40, H)) * 6
    A = rng.uniform(-3, 1, size=H)
    ba = rng.standard_normal(H)
    la, bt = oracle.gates_from_raw(a, b, A, ba)
    ref_la = -torch.exp(torch.tensor(A)) * torch.nn.functional.softplus(
        torch.tensor(a) + torch.tensor(ba))
    assert np.max(np.abs(la - ref_la.numpy())) < 1e-13
    assert np.max(np.abs(bt - torch.sigmoid(torch.tensor(b)).numpy())) < 1e-15
    # softplus(x) - softplus(-x) = x and sigmoid(x) + sigmoid(-x) = 1
    la_m, bt_m = oracle.gates_from_raw(-a, -b, A, None)
    la_p, _ = oracle.gates_from_raw(a, b, A, None)
    assert np.max(np.abs((la_p - la_m) + np.exp(A) * a)) < 1e-12
    _, bt_p = oracle.gates_from_raw(a, b, A, None)
    assert np.max(np.abs(bt_p + bt_m - 1)) < 1e-15
    # the bias is a shift of a
    la_s, _ = oracle.gates_from_raw(a + ba, b, A, None)
    assert np.max(np.abs(la_s - la)) < 1e-13
    # at zero: softplus(0) = ln 2, sigmoid(0) = 1/2
    z = np.zeros((3, H))
    la0, bt0 = oracle.gates_from_raw(z, z, A, None)
    assert np.max(np.abs(la0 + np.exp(A) * np.log(2.0))) < 1e-15
    assert np.all(bt0 == 0.5)
    # decay strictly in (0, 1) away from saturation; asymptotes
    assert np.all(la < 0) and np.all(bt > 0) and np.all(bt < 1)
    big = np.full((1, H), 60.0)
    la_big, bt_big = oracle.gates_from_raw(big, big, np.zeros(H), None)
    assert np.allclose(la_big, -60.0, rtol=0, atol=1e-13) and np.all(bt_big == 1.0)
    la_neg, bt_neg = oracle.gates_from_raw(-big, -big, np.zeros(H), None)
    assert np.allclose(la_neg, -np.exp(-60.0), rtol=1e-12, atol=0)
    assert np.allclose(bt_neg, np.exp(-60.0), rtol=1e-12, atol=0)


# Backward -------------------------------------------------------------------
def _bwd_case(lengths, H, dk, dv, seed):
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    total, N = int(cu[-1]), len(lengths)
    q, k, v, la, b, S0 = _rand_case(total, H, dk, dv, rng, unit=False, N=N)
    dy = rng.standard_normal((total, H, dv))
    dST = rng.standard_normal((N, H, dk, dv))
    return q, k, v, la, b, S0, dy, dST, cu


def test_bwd_matches_finite_differences():
    """Central differences of L = <dy, y> + <dS_T, S_T>, the forward taken in
    the closed form, against the hand-written reverse sweep, for every
    element of every input (varlen batch with an empty sequence)."""
    q, k, v, la, b, S0, dy, dST, cu = _bwd_case([5, 0, 7], 2, 3, 2, seed=31)
    grads = oracle.gdn_bwd(q, k, v, la, b, S0, dy, dST, cu_seqlens=cu)

    def loss(args):
        y, S = oracle.gdn_fwd(*args, cu_seqlens=cu, form=oracle.FORM_CLOSED)
        return float(np.sum(dy * y) + np.sum(dST * S))

    base = [q, k, v, la, b, S0]
    h = 1e-6
    for which, g in enumerate(grads):
        x = base[which]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            args_p = [a.copy() for a in base]
            args_m = [a.copy() for a in base]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            fd[idx] = (loss(args_p) - loss(args_m)) / (2 * h)
        assert np.max(np.abs(fd - g)) < 1e-7 * max(1.0, np.max(np.abs(fd))), which


def test_bwd_against_torch_autograd():
    """A float64 PyTorch loop of the erase-write recurrence, differentiated
    by autograd, gives the same gradients on a larger case."""
    q, k, v, la, b, S0, dy, dST, _ = _bwd_case([40, 40], 2, 8, 6, seed=32)
    grads = oracle.gdn_bwd(q, k, v, la, b, S0, dy, dST, N=2)
    t = [torch.tensor(x, requires_grad=True) for x in (q, k, v, la, b, S0)]
    tq, tk, tv, tla, tb, tS0 = t
    ys, Ss = [], []
    for n in range(2):
        S = tS0[n]
        for r in range(40 * n, 40 * n + 40):
            a = torch.exp(tla[r])[:, None, None]
            St = a * S
            e = tv[r] - torch.einsum("hij,hi->hj", St, tk[r])
            S = St + tb[r][:, None, None] * tk[r][:, :, None] * e[:, None, :]
            ys.append(torch.einsum("hij,hi->hj", S, tq[r]))
        Ss.append(S)
    L = (torch.stack(ys) * torch.tensor(dy)).sum() + (torch.stack(Ss) * torch.tensor(dST)).sum()
    L.backward()
    for g, x in zip(grads, t):
        assert np.max(np.abs(g - x.grad.numpy())) < 1e-10 * max(1.0, np.abs(g).max())


def test_bwd_zero_write_gate():
    """beta = 0 makes the state a pure decay of S0: no gradient reaches k or v,
    dq = S_t dy and dS0 collects the decayed q dy^T terms."""
    q, k, v, la, b, S0, dy, dST, _ = _bwd_case([9], 1, 3, 2, seed=33)
    b = np.zeros_like(b)
    dq, dk, dv, dla, db, dS0 = oracle.gdn_bwd(q, k, v, la, b, S0, dy, None, N=1)
    assert np.all(dk == 0) and np.all(dv == 0)
    g = np.cumsum(la[:, 0])
    want = sum(np.exp(g[t]) * np.outer(q[t, 0], dy[t, 0]) for t in range(9))
    assert np.max(np.abs(dS0[0, 0] - want)) < 1e-12
    for t in range(9):
        assert np.max(np.abs(dq[t, 0] - np.exp(g[t]) * S0[0, 0] @ dy[t, 0])) < 1e-12


def test_gates_from_raw_bwd_matches_finite_differences():
    """Central differences of <dla, log alpha> + <dbeta, beta> through the
    oracle's gate map, for every a, b, A and b_alpha."""
    rng = np.random.default_rng(34)
    H = 3
    a = rng.standard_normal((6, H)) * 3
    b = rng.standard_normal((6, H)) * 3
    A = rng.uniform(-2, 1, H)
    ba = rng.standard_normal(H)
    dla = rng.standard_normal((6, H))
    dbt = rng.standard_normal((6, H))
    da, db, dA, dba = oracle.gates_from_raw_bwd(a, b, A, ba, dla, dbt)

    def loss(x):
        la, bt = oracle.gates_from_raw(*x)
        return float(np.sum(dla * la) + np.sum(dbt * bt))

    base = [a, b, A, ba]
    h = 1e-6
    for which, g in enumerate((da, db, dA, dba)):
        fd = np.zeros_like(base[which])
        for idx in np.ndindex(fd.shape):
            p_ = [x.copy() for x in base]
            m_ = [x.copy() for x in base]
            p_[which][idx] += h
            m_[which][idx] -= h
            fd[idx] = (loss(p_) - loss(m_)) / (2 * h)
        assert np.max(np.abs(fd - g)) < 1e-7 * max(1.0, np.abs(fd).max()), which
