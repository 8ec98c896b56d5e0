"""(A') the chunk equations of the prefill kernel equal the token recurrence."""
import numpy as np
import pytest

import oracle
from tests import chunk_model


def _case(T, dk, dv, seed, s0=True, extreme=None):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, dk)); q /= np.linalg.norm(q, axis=1, keepdims=True)
    k = rng.standard_normal((T, dk)); k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    la = -np.exp(rng.uniform(-4, 0)) * np.log1p(np.exp(rng.standard_normal(T)))
    b = 1 / (1 + np.exp(-rng.standard_normal(T)))
    if extreme == "no_decay":
        la[:] = 0.0
    elif extreme == "strong_decay":
        la[:] = -30.0
    elif extreme == "beta_one":
        b[:] = 1.0
    elif extreme == "repeated_keys":
        k[1::2] = k[0::2][: len(k[1::2])]
    S0 = rng.standard_normal((dk, dv)) * 0.02 if s0 else np.zeros((dk, dv))
    return q, k, v, la, b, S0


@pytest.mark.parametrize("T,C", [(1, 64), (63, 64), (64, 64), (65, 64), (200, 64), (130, 16),
                                 (77, 1), (90, 90), (32, 32), (33, 32), (95, 32), (160, 32)])
@pytest.mark.parametrize("extreme", [None, "no_decay", "strong_decay", "beta_one", "repeated_keys"])
def test_chunk_model_equals_recurrence(T, C, extreme):
    q, k, v, la, b, S0 = _case(T, 16, 12, seed=T * 7 + C, extreme=extreme)
    y, S = chunk_model.chunk_fwd(q, k, v, la, b, S0, C=C)
    yo, So = oracle.gdn_fwd(q[:, None], k[:, None], v[:, None], la[:, None], b[:, None],
                            S0[None, None])
    scale_y = max(np.abs(yo).max(), 1e-3)
    assert np.abs(y - yo[:, 0]).max() / scale_y < 1e-11
    assert np.abs(S - So[0, 0]).max() / max(np.abs(So).max(), 1e-3) < 1e-11


def test_blocked_inverse_equals_dense():
    rng = np.random.default_rng(3)
    for C in (1, 15, 16, 17, 64):
        A = np.tril(rng.uniform(-1, 1, (C, C)), -1)
        T = chunk_model.unit_lower_inverse_blocked(A)
        assert np.abs(T @ (np.eye(C) + A) - np.eye(C)).max() < 1e-9


@pytest.mark.parametrize("T,C", [(1, 64), (37, 64), (64, 16), (70, 32), (130, 64), (45, 1)])
def test_chunk_bwd_model_equals_oracle(T, C):
    import oracle
    rng = np.random.default_rng(T * 7 + C)
    dk, dv = 6, 5
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    la = -np.exp(rng.uniform(-3, 0.5, T))
    b = rng.uniform(0, 1, T)
    S0 = rng.standard_normal((dk, dv))
    dy = rng.standard_normal((T, dv))
    dST = rng.standard_normal((dk, dv))
    got = chunk_model.chunk_bwd(q, k, v, la, b, S0, dy, dST, C=C)
    ref = oracle.gdn_bwd(q[:, None], k[:, None], v[:, None], la[:, None], b[:, None],
                         S0[None, None], dy[:, None], dST[None, None], N=1)
    ref = [ref[0][:, 0], ref[1][:, 0], ref[2][:, 0], ref[3][:, 0], ref[4][:, 0], ref[5][0, 0]]
    for gm, gr in zip(got, ref):
        assert np.max(np.abs(gm - gr)) < 1e-9 * max(1.0, np.abs(gr).max())
