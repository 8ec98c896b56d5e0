"""fp64 emulation of the bf16 prefill kernel's rounding points (design aid).

Replays the chunk equations in float64 and rounds to bf16 / fp16 exactly where
the kernel rounds, so the error of a precision plan can be predicted without a
GPU. Not collected by pytest; run it directly:

    python tests/precision_emulation.py

It reproduced the measured full-size y error of the plan that kept the state in
bf16 for Q S (1.914e-3) and of the current plan (1.71e-3).
"""
import numpy as np, torch, sys
sys.path.insert(0, __import__('os').path.dirname(__import__('os').path.dirname(__import__('os').path.abspath(__file__))))
import gdn_inputs as gi, oracle

def bf16(x): return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).double().numpy()
def f16(x): return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)
ident = lambda x: x

def run(q, k, v, la, b, C=32, rS=bf16, rSq=None, rR=f16, rE=f16, rT=f16, rP=f16, rK=f16, ry=bf16):
    rSq = rS if rSq is None else rSq
    T, dk = q.shape; dv = v.shape[1]
    S = np.zeros((dk, dv)); y = np.zeros((T, dv))
    for c0 in range(0, T, C):
        Q, K, V = q[c0:c0+C], k[c0:c0+C], v[c0:c0+C]; bb = b[c0:c0+C]
        g = np.cumsum(la[c0:c0+C]); gam = np.exp(g)
        G = np.tril(np.exp(np.minimum(g[:, None] - g[None, :], 0)))
        A = np.tril(bb[:, None] * (K @ K.T) * G, -1)
        Tm = rT(np.linalg.inv(np.eye(len(bb)) + A))
        X = K @ rS(S); QS = Q @ rSq(S)
        R = rR(bb[:, None] * (V - gam[:, None] * X))
        E = rE(Tm @ R)
        P = rP(np.tril((Q @ K.T) * G))
        y[c0:c0+C] = gam[:, None] * QS + P @ E
        Kt = rK(np.exp(g[-1] - g)[:, None] * K)
        S = gam[-1] * S + Kt.T @ E
    return ry(y), S

inp = gi.prefill_inputs(1, 1, 4096, 128, 128, "bf16", 0.0, seed=1)
q = inp["q"][:, 0].double().numpy(); k = inp["k"][:, 0].double().numpy(); v = inp["v"][:, 0].double().numpy()
la = inp["log_alpha"][:, 0].double().numpy(); b = inp["beta"][:, 0].double().numpy()
yo, So = oracle.gdn_fwd(q[:, None], k[:, None], v[:, None], la[:, None], b[:, None], None)
yo = yo[:, 0]; So = So[0, 0]
rel = lambda a, r: np.linalg.norm(a - r) / np.linalg.norm(r)
cases = {
  "exact, bf16 y": dict(rS=ident, rR=ident, rE=ident, rT=ident, rP=ident, rK=ident),
  "exact, fp32 y": dict(rS=ident, rR=ident, rE=ident, rT=ident, rP=ident, rK=ident, ry=ident),
  "v2 plan (S bf16), fp32 y": dict(ry=ident),
  "v2 plan (S bf16), bf16 y": dict(),
  "S f16, fp32 y": dict(rS=f16, ry=ident),
  "S f16, bf16 y": dict(rS=f16),
  "S bf16 only": dict(rR=ident, rE=ident, rT=ident, rP=ident, rK=ident, ry=ident),
  "S bf16 for X only (QS exact)": dict(rSq=ident, rR=ident, rE=ident, rT=ident, rP=ident, rK=ident, ry=ident),
  "S bf16 for QS only": dict(rS=ident, rSq=bf16, rR=ident, rE=ident, rT=ident, rP=ident, rK=ident, ry=ident),
  "R f16 only": dict(rS=ident, rE=ident, rT=ident, rP=ident, rK=ident, ry=ident),
  "E f16 only": dict(rS=ident, rR=ident, rT=ident, rP=ident, rK=ident, ry=ident),
}
for name, kw in cases.items():
    y, S = run(q, k, v, la, b, **kw)
    print("%-32s y %.2e  S %.2e" % (name, rel(y, yo), rel(S, So)))

print("--- all 16 heads of sequence 0, v2 plan with fp16 blocked T")
def tinv_kernel(A):
    # diag blocks exact (fp32-ish), off-diagonal T10 = -T11 (A10 T00) with fp16 operands
    T = np.zeros_like(A); n = A.shape[0]
    for b0 in range(0, n, 16):
        T[b0:b0+16, b0:b0+16] = np.linalg.inv(np.eye(16) + A[b0:b0+16, b0:b0+16])
    M = f16(A[16:32, 0:16]) @ f16(T[0:16, 0:16])
    T[16:32, 0:16] = -(f16(T[16:32, 16:32]) @ f16(M))
    return f16(T)

def run2(q, k, v, la, b, C=32, rS=bf16, ry=bf16, tinv=tinv_kernel):
    T, dk = q.shape; dv = v.shape[1]
    S = np.zeros((dk, dv)); y = np.zeros((T, dv))
    for c0 in range(0, T, C):
        Q, K, V = q[c0:c0+C], k[c0:c0+C], v[c0:c0+C]; bb = b[c0:c0+C]
        g = np.cumsum(la[c0:c0+C]); gam = np.exp(g)
        G = np.tril(np.exp(np.minimum(g[:, None] - g[None, :], 0)))
        A = np.tril(bb[:, None] * (K @ K.T) * G, -1)
        Tm = tinv(A)
        X = K @ rS(S); QS = Q @ rS(S)
        R = f16(bb[:, None] * (V - gam[:, None] * X))
        E = f16(Tm @ R)
        P = f16(np.tril((Q @ K.T) * G))
        y[c0:c0+C] = gam[:, None] * QS + P @ E
        Kt = f16(np.exp(g[-1] - g)[:, None] * K)
        S = gam[-1] * S + Kt.T @ E
    return ry(y), S

inp = gi.prefill_inputs(4, 16, 4096, 128, 128, "bf16", 0.0, seed=1)
ys, yos, ysf = [], [], []
for h in range(16):
    sl = slice(0, 4096)
    q = inp["q"][sl, h].double().numpy(); k = inp["k"][sl, h].double().numpy(); v = inp["v"][sl, h].double().numpy()
    la = inp["log_alpha"][sl, h].double().numpy(); b = inp["beta"][sl, h].double().numpy()
    yo, So = oracle.gdn_fwd(q[:, None], k[:, None], v[:, None], la[:, None], b[:, None], None)
    y, S = run2(q, k, v, la, b)
    yf, _ = run2(q, k, v, la, b, ry=ident)
    ys.append(y); yos.append(yo[:, 0]); ysf.append(yf)
    print("head %2d  A-scale %.3f  y(bf16) %.2e  y(fp32) %.2e  S %.2e" % (h, float(np.exp(np.log(-la).mean())), rel(y, yo[:, 0]), rel(yf, yo[:, 0]), rel(S, So[0, 0])))
print("sequence 0 all heads: bf16 y %.3e  fp32 y %.3e" % (rel(np.stack(ys), np.stack(yos)), rel(np.stack(ysf), np.stack(yos))))

print("--- variants over 16 heads")
def run3(q, k, v, la, b, C=32, rX=bf16, rQS=f16, ry=bf16, tinv=tinv_kernel, rE=f16, rR=f16, rP=f16, rK=f16):
    T, dk = q.shape; dv = v.shape[1]
    S = np.zeros((dk, dv)); y = np.zeros((T, dv))
    for c0 in range(0, T, C):
        Q, K, V = q[c0:c0+C], k[c0:c0+C], v[c0:c0+C]; bb = b[c0:c0+C]
        g = np.cumsum(la[c0:c0+C]); gam = np.exp(g)
        G = np.tril(np.exp(np.minimum(g[:, None] - g[None, :], 0)))
        A = np.tril(bb[:, None] * (K @ K.T) * G, -1)
        Tm = tinv(A)
        X = K @ rX(S); QS = Q @ rQS(S)
        R = rR(bb[:, None] * (V - gam[:, None] * X))
        E = rE(Tm @ R)
        P = rP(np.tril((Q @ K.T) * G))
        y[c0:c0+C] = gam[:, None] * QS + P @ E
        Kt = rK(np.exp(g[-1] - g)[:, None] * K)
        S = gam[-1] * S + Kt.T @ E
    return ry(y), S
variants = {
  "X bf16, QS f16": dict(),
  "X f16, QS f16": dict(rX=f16),
  "X bf16, QS f16, exact T": dict(tinv=lambda A: f16(np.linalg.inv(np.eye(A.shape[0]) + A))),
  "X bf16, QS f16, E/R fp32": dict(rE=ident, rR=ident),
  "X bf16, QS f16, P fp32": dict(rP=ident),
  "X bf16, QS f16, Kt fp32": dict(rK=ident),
}
data = []
for h in range(16):
    q = inp["q"][:, h].double().numpy()[:4096]; k = inp["k"][:4096, h].double().numpy(); v = inp["v"][:4096, h].double().numpy()
    la = inp["log_alpha"][:4096, h].double().numpy(); b = inp["beta"][:4096, h].double().numpy()
    yo, So = oracle.gdn_fwd(q[:, None], k[:, None], v[:, None], la[:, None], b[:, None], None)
    data.append((q, k, v, la, b, yo[:, 0], So[0, 0]))
for name, kw in variants.items():
    ys, yfs, yos, worst = [], [], [], 0
    for (q, k, v, la, b, yo, So) in data:
        y, S = run3(q, k, v, la, b, **kw); yf, _ = run3(q, k, v, la, b, ry=ident, **kw)
        ys.append(y); yfs.append(yf); yos.append(yo); worst = max(worst, rel(y, yo))
    print("%-28s all-heads bf16 y %.3e  fp32 y %.3e  worst head %.3e" % (name, rel(np.stack(ys), np.stack(yos)), rel(np.stack(yfs), np.stack(yos)), worst))
