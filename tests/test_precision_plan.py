"""fp64 emulation of the 16-bit prefill kernel's rounding points.

The chunk equations (derived from the page "NLP——技术报告解读-Qwen3.8-Flash-Next",
section "Gated DeltaNet 核心机制", by unrolling the recurrence over a chunk) are
replayed in float64 with values rounded to bf16 or fp16 exactly where the
kernel rounds them: the state is rounded to bf16 as the operand of K S and to
fp16 as the operand of Q S; R, E, T, P and Kt are rounded to fp16; y is
rounded to bf16 on output; the state itself and every sum stay wide. The
prediction is compared with the fp64 token recurrence (the oracle) on the
prefill workload's input distributions.

These tests pin the precision plan without a GPU: the plan the kernel uses must
predict an error inside the 2e-3 bar with margin, and the alternatives the
plan rejects must predict more error than it.
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle


def bf16(x):
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).double().numpy()


def f16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def ident(x):
    return x


def emulate(q, k, v, la, b, C=32, rS=bf16, rSq=f16, rR=f16, rE=f16, rT=f16, rP=f16, rK=f16,
            ry=bf16):
    """One (sequence, head) through the chunk equations with the given
    rounding at each point; returns (y, S_T)."""
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv))
    y = np.zeros((T, dv))
    for c0 in range(0, T, C):
        Q, K, V, bb = q[c0:c0 + C], k[c0:c0 + C], v[c0:c0 + C], b[c0:c0 + C]
        g = np.cumsum(la[c0:c0 + C])
        gam = np.exp(g)
        G = np.tril(np.exp(np.minimum(g[:, None] - g[None, :], 0.0)))
        A = np.tril(bb[:, None] * (K @ K.T) * G, -1)
        Tm = rT(np.linalg.inv(np.eye(len(bb)) + A))
        X = K @ rS(S)
        QS = Q @ rSq(S)
        R = rR(bb[:, None] * (V - gam[:, None] * X))
        E = rE(Tm @ R)
        P = rP(np.tril((Q @ K.T) * G))
        y[c0:c0 + C] = gam[:, None] * QS + P @ E
        Kt = rK(np.exp(g[-1] - g)[:, None] * K)
        S = gam[-1] * S + Kt.T @ E
    return ry(y), S


@pytest.fixture(scope="module")
def heads():
    """Four heads of the prefill workload's distributions (bf16 q, k, v;
    per-head decay rate A ~ U(-4, 0)), 2048 tokens each, with the oracle's
    outputs."""
    inp = gi.prefill_inputs(1, 4, 2048, 128, 128, "bf16", 0.0, seed=1)
    out = []
    for h in range(4):
        q, k, v, la, b = (inp[key][:, h].double().numpy()
                          for key in ("q", "k", "v", "log_alpha", "beta"))
        yo, So = oracle.gdn_fwd(q[:, None], k[:, None], v[:, None], la[:, None], b[:, None],
                                None)
        out.append(((q, k, v, la, b), yo[:, 0], So[0, 0]))
    return out


def _rel(a, r):
    return float(np.linalg.norm(a - r) / np.linalg.norm(r))


def _worst(heads, **kw):
    ey = es = 0.0
    for args, yo, So in heads:
        y, S = emulate(*args, **kw)
        ey, es = max(ey, _rel(y, yo)), max(es, _rel(S, So))
    return ey, es


def test_emulation_without_rounding_is_the_recurrence(heads):
    ey, es = _worst(heads, rS=ident, rSq=ident, rR=ident, rE=ident, rT=ident, rP=ident,
                    rK=ident, ry=ident)
    assert ey < 1e-10 and es < 1e-10


def test_kernel_plan_inside_the_bar(heads):
    ey, es = _worst(heads)
    ey_out, _ = _worst(heads, rS=ident, rSq=ident, rR=ident, rE=ident, rT=ident, rP=ident,
                       rK=ident)
    print("plan: y %.3e (bf16 output rounding alone %.3e), S %.3e" % (ey, ey_out, es))
    assert ey <= 1.85e-3 and es <= 1e-3
    # the arithmetic's own share, with the output rounding taken out in quadrature
    assert (ey ** 2 - ey_out ** 2) ** 0.5 <= 1e-3


def test_rejected_plans_predict_more_error(heads):
    ey, _ = _worst(heads, ry=ident)
    # the state rounded to bf16 for Q S as well (no fp16 copy of Q)
    ey_sq, _ = _worst(heads, rSq=bf16, ry=ident)
    # E rounded to bf16 (a bf16 operand for the state update)
    ey_e, _ = _worst(heads, rE=bf16, ry=ident)
    print("fp32-output errors: plan %.3e, bf16 S for QS %.3e, bf16 E %.3e" % (ey, ey_sq, ey_e))
    assert ey_sq > 1.5 * ey and ey_e > 1.5 * ey
