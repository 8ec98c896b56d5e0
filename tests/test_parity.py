"""GPU parity: the HIP path against the fp64 oracle, element by element,
through the C ABI (via the thin Python binding).

Bar: relative L2 error <= 1e-5 for fp32 inputs and <= 2e-3 for bf16 inputs
(fp32 state) on y and on the final state.
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
from tests.util import TOL, rel_l2, to_dev

gpu = pytest.mark.gpu


def _lib():
    import gated_deltanet_amd as g
    g.load_library()
    return g


def _run_chunk(inp, out_dtype=None):
    g = _lib()
    d = to_dev(inp)
    y, S = g.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"],
                           cu_seqlens=d["cu_seqlens"], out_dtype=out_dtype, N=d["N"])
    torch.cuda.synchronize()
    return y, S


def _oracle_chunk(inp):
    N = inp["N"]
    return oracle.gdn_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["S0"],
                          cu_seqlens=inp["cu_seqlens"], N=N)


def _flat(inp, y):
    return y.reshape(-1, inp["H"], inp["dv"])


def _check(inp, out_dtype=None, tol=None):
    tol = TOL[inp["dtype"]] if tol is None else tol
    y, S = _run_chunk(inp, out_dtype)
    yo, So = _oracle_chunk(inp)
    ey, es = rel_l2(_flat(inp, y), yo), rel_l2(S, So)
    print("rel_l2 y=%.3e S=%.3e" % (ey, es), flush=True)
    assert np.isfinite(ey) and np.isfinite(es)
    assert ey <= tol and es <= tol, (ey, es)
    return ey, es


@gpu
@pytest.mark.parametrize("T", [1, 63, 64, 65, 200, 256])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk_small(T, d, dtype):
    inp = gi.prefill_inputs(2, 3, T, d, d, dtype, s0_std=0.02, seed=T + d)
    _check(inp, out_dtype=torch.float32)


@gpu
@pytest.mark.parametrize("T", [1, 65, 200])
@pytest.mark.parametrize("d", [64, 128])
def test_chunk_small_f16(T, d):
    inp = gi.prefill_inputs(2, 3, T, d, d, "f16", s0_std=0.02, seed=T + d + 5)
    _check(inp, out_dtype=torch.float32)
    _check(inp, out_dtype=torch.float16)


@gpu
@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 64)])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_chunk_rect_heads(dk, dv, dtype):
    inp = gi.prefill_inputs(1, 2, 130, dk, dv, dtype, s0_std=0.02, seed=dk + 3 * dv)
    _check(inp, out_dtype=torch.float32)


@gpu
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk_zero_state_bf16_out(dtype):
    inp = gi.prefill_inputs(2, 2, 300, 128, 128, dtype, s0_std=0.0, seed=9)
    _check(inp)  # y in the input dtype


@gpu
def test_workload_tiny_fwd():
    """B=1, H=2, T=256, dk=dv=64, fp32, S0 = 0 (the oracle-sized workload)."""
    inp = gi.workload_inputs(0)
    _check(inp)


@gpu
@pytest.mark.parametrize("case", ["no_decay", "strong_decay", "beta0", "beta1", "repeated_keys",
                                  "near_parallel", "large_v", "banded_decay"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk_gate_extremes(case, dtype):
    inp = gi.prefill_inputs(1, 2, 150, 128, 128, dtype, s0_std=0.02, seed=21)
    if case == "no_decay":
        inp["log_alpha"].zero_()
    elif case == "strong_decay":
        inp["log_alpha"].fill_(-30.0)
    elif case == "beta0":
        inp["beta"].zero_()
    elif case == "beta1":
        inp["beta"].fill_(1.0)
    elif case == "repeated_keys":
        inp["k"][1::2] = inp["k"][0::2][: inp["k"][1::2].shape[0]]
    elif case == "near_parallel":
        base = inp["k"][:1].float()
        noise = gi.normal(inp["k"].shape, 77, 1) * 1e-2
        kk = base + noise
        inp["k"] = (kk / kk.norm(dim=-1, keepdim=True)).to(inp["k"].dtype)
    elif case == "large_v":
        # |v| ~ 64: y and the state reach the hundreds, well inside fp16
        inp["v"] = (inp["v"].float() * 64.0).to(inp["v"].dtype)
    elif case == "banded_decay":
        # bands of 40 tokens alternate between no decay and log alpha = -12:
        # stretches whose decay spans exceed the fp32 range of a factorised
        # decay sit next to stretches with none
        band = (torch.arange(inp["log_alpha"].shape[0]) // 40) % 2 == 1
        inp["log_alpha"][band] = -12.0
    _check(inp, out_dtype=torch.float32)


@gpu
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_chunk_varlen(dtype):
    lengths = [1, 2, 63, 64, 65, 1000, 0, 130]
    inp = gi.prefill_inputs(0, 2, 0, 128, 128, dtype, s0_std=0.02, seed=31, lengths=lengths)
    _check(inp, out_dtype=torch.float32)


@gpu
@pytest.mark.parametrize("ns", [1, 4, 8])
@pytest.mark.parametrize("case", ["varlen", "equal", "rect", "strong_decay"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_chunk_wide_state_tiles(ns, case, dtype, monkeypatch):
    """The prefill with one, four or eight state waves per workgroup (16, 64
    or 128 columns; chosen by batch size, forced here by GDN_PREFILL_NS)
    gives the two-wave result bit for bit: each column's arithmetic is the
    same, only the columns' grouping into workgroups differs. Checked
    against the oracle as well."""
    if ns == 8 and case == "rect":
        pytest.skip("eight state waves need dv = 128")
    if case == "varlen":
        inp = gi.prefill_inputs(0, 2, 0, 128, 128, dtype, s0_std=0.02, seed=33,
                                lengths=[1, 2, 63, 64, 65, 1000, 0, 130])
    elif case == "rect":
        inp = gi.prefill_inputs(2, 2, 130, 128, 64, dtype, s0_std=0.02, seed=34)
    else:
        inp = gi.prefill_inputs(3, 2, 200, 128, 128, dtype, s0_std=0.02, seed=35)
        if case == "strong_decay":
            inp["log_alpha"][::3] = -30.0
    monkeypatch.setenv("GDN_PREFILL_NS", "2")
    y2, S2 = _run_chunk(inp, torch.float32)
    monkeypatch.setenv("GDN_PREFILL_NS", str(ns))
    y4, S4 = _run_chunk(inp, torch.float32)
    assert torch.equal(y2.cpu(), y4.cpu()) and torch.equal(S2.cpu(), S4.cpu())
    _check(inp, out_dtype=torch.float32)


@gpu
def test_chunk_in_place_state():
    g = _lib()
    inp = to_dev(gi.prefill_inputs(2, 2, 100, 128, 128, "bf16", s0_std=0.02, seed=41))
    y_ref, S_ref = g.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                                   inp["S0"])  # N from S0
    S = inp["S0"].clone()
    y2, S2 = g.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], S,
                             S_T=S)
    torch.cuda.synchronize()
    assert torch.equal(S, S_ref) and torch.equal(y2, y_ref)


@gpu
def test_chunk_deterministic():
    g = _lib()
    inp = to_dev(gi.prefill_inputs(2, 4, 333, 128, 128, "bf16", s0_std=0.02, seed=42))
    outs = [g.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                            inp["S0"]) for _ in range(3)]
    torch.cuda.synchronize()
    for y, S in outs[1:]:
        assert torch.equal(y, outs[0][0]) and torch.equal(S, outs[0][1])


@gpu
def test_chunk_split_resume():
    """prefill(0..t0) -> S -> prefill(t0..T) equals one pass."""
    g = _lib()
    inp = to_dev(gi.prefill_inputs(1, 2, 300, 128, 128, "f32", s0_std=0.02, seed=43))
    y, S = g.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["S0"])
    for t0 in (1, 64, 100):
        sl = lambda x, a, b: x[a:b].contiguous()
        y1, S1 = g.gdn_chunk_fwd(*(sl(inp[n], 0, t0) for n in ("q", "k", "v", "log_alpha", "beta")),
                                 inp["S0"])
        y2, S2 = g.gdn_chunk_fwd(*(sl(inp[n], t0, 300) for n in ("q", "k", "v", "log_alpha", "beta")),
                                 S1)
        torch.cuda.synchronize()
        assert rel_l2(torch.cat([y1, y2]), y.cpu().double().numpy()) < 1e-5
        assert rel_l2(S2, S.cpu().double().numpy()) < 1e-5


@gpu
def test_chunk_nan_isolated():
    """A NaN in one (sequence, head) does not reach any other."""
    g = _lib()
    inp = gi.prefill_inputs(2, 3, 100, 128, 128, "bf16", s0_std=0.02, seed=44)
    inp["v"][130, 1, 5] = float("nan")  # sequence 1, head 1
    d = to_dev(inp)
    y, S = g.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"])
    torch.cuda.synchronize()
    y = y.reshape(2, 100, 3, 128).cpu()
    S = S.cpu()
    for n in range(2):
        for h in range(3):
            bad = (n, h) == (1, 1)
            assert torch.isfinite(S[n, h]).all() != bad
            if not bad:
                assert torch.isfinite(y[n, :, h]).all()


# ---------------------------------------------------------------- decode ----
@gpu
@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_decode_steps(dk, dv, dtype):
    g = _lib()
    inp = gi.decode_inputs(5, 3, dk, dv, steps=4, dtype=dtype, s0_std=0.02, seed=dk + dv)
    S = inp["S0"].clone().cuda()
    S_or = inp["S0"].double().numpy()
    ys, ys_or = [], []
    for t in range(4):
        args = [inp[n][t].contiguous() for n in ("q", "k", "v", "log_alpha", "beta")]
        y = g.gdn_decode_step(*(a.cuda() for a in args), S, out_dtype=torch.float32)
        yo, S_or = oracle.decode_step(*args, S_or)
        ys.append(y.cpu())
        ys_or.append(yo)
    torch.cuda.synchronize()
    ey = rel_l2(torch.stack(ys), np.stack(ys_or))
    es = rel_l2(S, S_or)
    print("rel_l2 y=%.3e S=%.3e" % (ey, es))
    assert ey <= TOL[dtype] and es <= TOL[dtype]


@gpu
def test_decode_matches_prefill():
    """T decode steps equal one prefill of T tokens (two GPU paths)."""
    g = _lib()
    T = 70
    inp = to_dev(gi.prefill_inputs(3, 2, T, 128, 128, "f32", s0_std=0.02, seed=51))
    y, S = g.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["S0"])
    Sd = inp["S0"].clone()  # N = 3 from S0
    yd = []
    for t in range(T):
        rows = torch.arange(3, device="cuda") * T + t
        args = [inp[n][rows].contiguous() for n in ("q", "k", "v", "log_alpha", "beta")]
        yd.append(g.gdn_decode_step(*args, Sd))
    torch.cuda.synchronize()
    yd = torch.stack(yd, 1).reshape(3 * T, 2, 128)
    assert rel_l2(yd, y.cpu().double().numpy()) < 1e-5
    assert rel_l2(Sd, S.cpu().double().numpy()) < 1e-5


# ------------------------------------------------------------ front end -----
@gpu
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_frontend_varlen(d, dtype):
    g = _lib()
    lengths = [1, 2, 3, 4, 5, 63, 64, 65, 300, 0, 17]
    f = gi.frontend_inputs(lengths, 3, d, d, dtype=dtype, seed=61)
    dev = to_dev(f)
    q, k, v = g.gdn_frontend_qkv(dev["q_raw"], dev["k_raw"], dev["v_raw"], dev["conv_w"],
                                 cu_seqlens=dev["cu_seqlens"], l2_eps=1e-6, out_dtype=torch.float32)
    torch.cuda.synchronize()
    cu = f["cu_seqlens"]
    H = 3
    for i, (raw, got, l2) in enumerate(((f["q_raw"], q, True), (f["k_raw"], k, True),
                                        (f["v_raw"], v, False))):
        ref = oracle.frontend(raw, f["conv_w"][i], cu_seqlens=cu, l2=l2, eps=1e-6)
        e = rel_l2(got, ref)
        print("stream %d rel_l2 %.3e" % (i, e))
        assert e <= 1e-5, (i, e)  # fp32 arithmetic on exact inputs
    # bf16 outputs: one rounding on top
    qb, kb, vb = g.gdn_frontend_qkv(dev["q_raw"], dev["k_raw"], dev["v_raw"], dev["conv_w"],
                                    cu_seqlens=dev["cu_seqlens"], out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = oracle.frontend(f["q_raw"], f["conv_w"][0], cu_seqlens=cu, l2=True, eps=1e-6)
    # one round-to-nearest step to p significant bits leaves an error uniform
    # within half an ulp, whose RMS relative to the value is at most
    # 2^-p / sqrt(3) (reached at the bottom of a binade); plus the fp32 work
    assert rel_l2(qb, ref) <= 2.0 ** -8 / 3 ** 0.5 + 1e-5  # bf16: p = 8
    qh, kh, vh = g.gdn_frontend_qkv(dev["q_raw"], dev["k_raw"], dev["v_raw"], dev["conv_w"],
                                    cu_seqlens=dev["cu_seqlens"], out_dtype=torch.float16)
    torch.cuda.synchronize()
    assert rel_l2(qh, ref) <= 2.0 ** -11 / 3 ** 0.5 + 1e-5  # fp16: p = 11


@gpu
def test_frontend_equal_length_batches():
    g = _lib()
    f = gi.frontend_inputs([50, 50, 50], 2, 128, 128, dtype="bf16", seed=62)
    dev = to_dev(f)
    q, k, v = g.gdn_frontend_qkv(dev["q_raw"], dev["k_raw"], dev["v_raw"], dev["conv_w"], N=3,
                                 out_dtype=torch.float32)
    q2, k2, v2 = g.gdn_frontend_qkv(dev["q_raw"], dev["k_raw"], dev["v_raw"], dev["conv_w"],
                                    cu_seqlens=dev["cu_seqlens"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(k, k2) and torch.equal(v, v2)


@gpu
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype,zdtype", [("f32", "f32"), ("bf16", "bf16"), ("f16", "bf16"),
                                          ("f32", "bf16"), ("f16", "f16")])
@pytest.mark.parametrize("with_w", [False, True])
def test_output_gate(d, dtype, zdtype, with_w):
    g = _lib()
    rows = 1000
    y = gi.normal((rows, d), 71, 1).to(gi.torch_dtype(dtype))
    z = gi.normal((rows, d), 71, 2).to(gi.torch_dtype(zdtype))
    w = gi.normal((d,), 71, 3, std=0.1) if with_w else None
    o = g.gdn_output_gate(y.cuda(), z.cuda(), None if w is None else w.cuda(), 1e-6,
                          out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.output_gate(y, z, w, eps=1e-6)
    e = rel_l2(o, ref)
    print("rel_l2 %.3e" % e)
    assert e <= 1e-5


@gpu
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_fused_prefill_small(d, dtype):
    """gdn_chunk_fwd_fused against the oracle chain (front end -> recurrence
    -> gate) on every unit of a small varlen batch with edge lengths, at the
    16-bit bar (2e-3); the entry point takes 16-bit inputs only."""
    g = _lib()
    lengths = [1, 2, 31, 33, 100, 0, 65]
    f = gi.frontend_inputs(lengths, 3, d, d, dtype=dtype, seed=63, norm_w_std=0.1)
    dev = to_dev(f)
    o, S = g.gdn_chunk_fwd_fused(dev["q_raw"], dev["k_raw"], dev["v_raw"], dev["conv_w"],
                                 dev["log_alpha"], dev["beta"], dev["z"], S0=dev["S0"],
                                 norm_w=dev["norm_w"], cu_seqlens=dev["cu_seqlens"],
                                 out_dtype=torch.float32)
    torch.cuda.synchronize()
    cu = f["cu_seqlens"]
    q, k, v = (oracle.frontend(f[key], f["conv_w"][i], cu_seqlens=cu, l2=l2, eps=1e-6)
               for i, (key, l2) in enumerate((("q_raw", True), ("k_raw", True),
                                              ("v_raw", False))))
    y, So = oracle.gdn_fwd(q, k, v, f["log_alpha"], f["beta"], f["S0"], cu_seqlens=cu)
    oo = oracle.output_gate(y.reshape(-1, d), f["z"].reshape(-1, d), f["norm_w"], eps=1e-6)
    eo, es = rel_l2(o.reshape(-1, d), oo), rel_l2(S, So)
    print("rel_l2 o=%.3e S=%.3e" % (eo, es), flush=True)
    assert eo <= 2e-3 and es <= 2e-3, (eo, es)


# ------------------------------------------------- gates from raw inputs -----
def _raw_case(lengths, H, d, dtype, seed):
    inp = gi.prefill_inputs(len(lengths), H, 0, d, d, dtype, s0_std=0.02, seed=seed,
                            lengths=lengths)
    rows = inp["q"].shape[0]
    a, b, A, b_alpha = gi.raw_gates(rows, H, seed + 1)
    return inp, a, b, A, b_alpha


@gpu
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("with_bias", [False, True])
def test_chunk_gated(d, dtype, with_bias):
    g = _lib()
    lengths = [1, 33, 100, 0, 65]
    inp, a, b, A, b_alpha = _raw_case(lengths, 3, d, dtype, seed=60 + d)
    if not with_bias:
        b_alpha = None
    dv_ = to_dev(inp)
    bias_dev = None if b_alpha is None else b_alpha.cuda()
    y, S = g.gdn_chunk_fwd_gated(dv_["q"], dv_["k"], dv_["v"], a.cuda(), b.cuda(), A.cuda(),
                                 bias_dev, dv_["S0"], cu_seqlens=dv_["cu_seqlens"],
                                 out_dtype=torch.float32)
    torch.cuda.synchronize()
    la, bt = oracle.gates_from_raw(a, b, A, b_alpha)
    yo, So = oracle.gdn_fwd(inp["q"], inp["k"], inp["v"], la, bt, inp["S0"],
                            cu_seqlens=inp["cu_seqlens"], N=inp["N"])
    ey, es = rel_l2(_flat(inp, y), yo), rel_l2(S, So)
    print("gated rel_l2 y=%.3e S=%.3e" % (ey, es), flush=True)
    assert ey <= TOL[dtype] and es <= TOL[dtype], (ey, es)


@gpu
@pytest.mark.parametrize("ns", [1, 4, 8])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_chunk_gated_wide_state_tiles(ns, dtype, monkeypatch):
    """The raw-gate prefill with one, four or eight state waves per
    workgroup (forced by GDN_PREFILL_NS) equals the two-wave result bit for
    bit, and the oracle to the bar; varlen with an empty sequence, biases."""
    g = _lib()
    inp, a, b, A, b_alpha = _raw_case([1, 33, 100, 0, 65, 200], 3, 128, dtype, seed=66)
    dv_ = to_dev(inp)

    def run():
        y, S = g.gdn_chunk_fwd_gated(dv_["q"], dv_["k"], dv_["v"], a.cuda(), b.cuda(), A.cuda(),
                                     b_alpha.cuda(), dv_["S0"], cu_seqlens=dv_["cu_seqlens"],
                                     out_dtype=torch.float32)
        torch.cuda.synchronize()
        return y.cpu(), S.cpu()

    monkeypatch.setenv("GDN_PREFILL_NS", "2")
    y2, S2 = run()
    monkeypatch.setenv("GDN_PREFILL_NS", str(ns))
    y, S = run()
    assert torch.equal(y, y2) and torch.equal(S, S2)
    la, bt = oracle.gates_from_raw(a, b, A, b_alpha)
    yo, So = oracle.gdn_fwd(inp["q"], inp["k"], inp["v"], la, bt, inp["S0"],
                            cu_seqlens=inp["cu_seqlens"], N=inp["N"])
    ey, es = rel_l2(_flat(inp, y), yo), rel_l2(S, So)
    assert ey <= TOL[dtype] and es <= TOL[dtype], (ey, es)


@gpu
def test_chunk_gated_matches_precomputed_gates():
    """The in-kernel gate map and gates precomputed in fp32 by torch drive
    the same recurrence: the two outputs agree to fp32 rounding."""
    g = _lib()
    inp, a, b, A, b_alpha = _raw_case([300, 77], 4, 128, "bf16", seed=70)
    d = to_dev(inp)
    la = (-torch.exp(A)[None, :] * torch.nn.functional.softplus(a + b_alpha[None, :])).contiguous()
    bt = torch.sigmoid(b).contiguous()
    y1, S1 = g.gdn_chunk_fwd(d["q"], d["k"], d["v"], la.cuda(), bt.cuda(), d["S0"],
                             cu_seqlens=d["cu_seqlens"], out_dtype=torch.float32)
    y2, S2 = g.gdn_chunk_fwd_gated(d["q"], d["k"], d["v"], a.cuda(), b.cuda(), A.cuda(),
                                   b_alpha.cuda(), d["S0"], cu_seqlens=d["cu_seqlens"],
                                   out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert rel_l2(y2, y1.cpu().double().numpy()) < 1e-4
    assert rel_l2(S2, S1.cpu().double().numpy()) < 1e-4


@gpu
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_gated_state_slots(dtype):
    """Raw gates plus a slot pool: sequences update their own slots, padding
    entries leave the pool alone and get y = 0."""
    g = _lib()
    N, H, d, n_slots = 6, 3, 128, 9
    idx = torch.tensor([4, -1, 0, 8, 9, 2], dtype=torch.int32)  # 9 is out of range
    inp = gi.decode_inputs(N, H, d, d, steps=3, dtype=dtype, s0_std=0.02, seed=81)
    pool = gi.normal((n_slots, H, d, d), 82, 1, std=0.02)
    S = pool.clone().cuda()
    S_or = pool.double().numpy().copy()
    a, b, A, b_alpha = gi.raw_gates(3 * N, H, 83)
    a, b = a.reshape(3, N, H), b.reshape(3, N, H)
    live = [n for n in range(N) if 0 <= int(idx[n]) < n_slots]
    for t in range(3):
        q, k, v = (inp[nm][t].contiguous() for nm in ("q", "k", "v"))
        y = g.gdn_decode_step_gated(q.cuda(), k.cuda(), v.cuda(), a[t].contiguous().cuda(),
                                    b[t].contiguous().cuda(), A.cuda(), S, b_alpha=b_alpha.cuda(),
                                    state_idx=idx.cuda(), out_dtype=torch.float32)
        la, bt = oracle.gates_from_raw(a[t], b[t], A, b_alpha)
        sl = [int(idx[n]) for n in live]
        yo, Sn = oracle.decode_step(q[live], k[live], v[live], la[live], bt[live], S_or[sl])
        S_or[sl] = Sn
        torch.cuda.synchronize()
        yc = y.cpu()
        assert rel_l2(yc[live], yo) <= TOL[dtype]
        for n in range(N):
            if n not in live:
                assert torch.all(yc[n] == 0)
    untouched = [s for s in range(n_slots) if s not in [int(idx[n]) for n in live]]
    assert torch.equal(S.cpu()[untouched], pool[untouched])
    assert rel_l2(S, S_or) <= TOL[dtype]


# ------------------------------------------------- multi-token decode -----
def _multi_inputs(N, H, dk, dv, n_tok, dtype, seed):
    inp = gi.decode_inputs(N, H, dk, dv, steps=n_tok, dtype=dtype, s0_std=0.02, seed=seed)
    tm = {nm: inp[nm].transpose(0, 1).contiguous() for nm in ("q", "k", "v", "log_alpha",
                                                                "beta")}
    return inp, tm  # inp: [n_tok, N, ...] per step; tm: [N, n_tok, ...]


@gpu
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 64), (64, 128), (128, 128)])
@pytest.mark.parametrize("n_tok", [1, 2, 4, 8])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_multi_matches_steps_and_oracle(dk, dv, n_tok, dtype):
    """n_tok tokens in one call equal n_tok single-token calls (bit for bit
    for one token; for more, the call applies them as blocks of 4 in the
    unrolled form, the same sums in another order, so to fp32 rounding) and
    the oracle to the bar."""
    g = _lib()
    N, H = 5, 3
    inp, tm = _multi_inputs(N, H, dk, dv, n_tok, dtype, seed=dk + dv + n_tok)
    S1 = inp["S0"].clone().cuda()
    y1 = g.gdn_decode_multi(*(tm[nm].cuda() for nm in ("q", "k", "v", "log_alpha", "beta")), S1,
                            out_dtype=torch.float32)
    S2 = inp["S0"].clone().cuda()
    y2 = [g.gdn_decode_step(*(inp[nm][t].contiguous().cuda() for nm in
                              ("q", "k", "v", "log_alpha", "beta")), S2, out_dtype=torch.float32)
          for t in range(n_tok)]
    torch.cuda.synchronize()
    if n_tok == 1:
        assert torch.equal(y1, torch.stack(y2, 1))
        assert torch.equal(S1, S2)
    else:
        assert rel_l2(y1, torch.stack(y2, 1).double().cpu().numpy()) <= 1e-5
        assert rel_l2(S1, S2.double().cpu().numpy()) <= 1e-5
    S_or = inp["S0"].double().numpy()
    yo = []
    for t in range(n_tok):
        y_t, S_or = oracle.decode_step(*(inp[nm][t] for nm in ("q", "k", "v", "log_alpha",
                                                                "beta")), S_or)
        yo.append(y_t)
    assert rel_l2(y1, np.stack(yo, 1)) <= TOL[dtype]
    assert rel_l2(S1, S_or) <= TOL[dtype]


@gpu
@pytest.mark.parametrize("raw", [False, True])
def test_decode_multi_slots_and_rollback_states(raw):
    """Slot table [N, 1 + n_tok]: each sequence starts from its slot and
    leaves the state after chosen tokens in chosen slots (for rolling back to
    an accepted prefix); padding entries write nothing and get y = 0."""
    g = _lib()
    N, H, d, n_tok, n_slots = 4, 2, 128, 4, 20
    inp, tm = _multi_inputs(N, H, d, d, n_tok, "bf16", seed=91)
    pool = gi.normal((n_slots, H, d, d), 92, 1, std=0.02)
    table = torch.tensor([[3, 10, 11, 12, 3],     # every intermediate, final back in place
                          [-1, 13, 14, 15, 16],   # padding: nothing written
                          [7, -1, -1, -1, 17],    # only the final state, elsewhere
                          [0, 18, -1, 19, -1]],   # two intermediates, final dropped
                         dtype=torch.int32)
    if raw:
        a, b, A, b_alpha = gi.raw_gates(N * n_tok, H, 93)
        ga, gb = a.reshape(N, n_tok, H), b.reshape(N, n_tok, H)
        la_o, bt_o = oracle.gates_from_raw(a, b, A, b_alpha)
        la_o, bt_o = la_o.reshape(N, n_tok, H), bt_o.reshape(N, n_tok, H)
        kw = dict(A=A.cuda(), b_alpha=b_alpha.cuda())
    else:
        ga, gb = tm["log_alpha"], tm["beta"]
        la_o, bt_o = ga.double().numpy(), gb.double().numpy()
        kw = {}
    S = pool.clone().cuda()
    y = g.gdn_decode_multi(tm["q"].cuda(), tm["k"].cuda(), tm["v"].cuda(), ga.contiguous().cuda(),
                           gb.contiguous().cuda(), S, state_idx=table.cuda(),
                           out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    Sc, yc = S.cpu(), y.cpu()
    expect = pool.double().numpy().copy()
    written = set()
    for n in range(N):
        start = int(table[n, 0])
        if not 0 <= start < n_slots:
            assert torch.all(yc[n] == 0)
            continue
        st = pool[start].double().numpy()[None]
        for t in range(n_tok):
            y_t, st = oracle.decode_step(tm["q"][n, t][None], tm["k"][n, t][None],
                                         tm["v"][n, t][None], la_o[n, t][None], bt_o[n, t][None],
                                         st)
            assert rel_l2(yc[n, t][None], y_t) <= 2e-3
            w = int(table[n, 1 + t])
            if 0 <= w < n_slots:
                expect[w] = st[0]
                written.add(w)
    for sl in range(n_slots):
        if sl in written:
            assert rel_l2(Sc[sl], expect[sl]) <= 2e-3, sl
        else:
            assert torch.equal(Sc[sl], pool[sl]), sl


# ------------------------------------------------------- fused decode -----
def _fused_decode_reference(f, hist, S0, la, bt, l2_eps=1e-6, rms_eps=1e-6):
    """The fp64 oracle chain for one fused decode call: the front end over
    [three history rows, the call's raw rows] of each sequence (the outputs
    of the history rows are dropped), n_tok oracle decode steps, then the
    output gate. hist [N, H, 3, 3, d]; returns (o [N, n_tok, H, d], S)."""
    N, n_tok, H, d = f["q_raw"].shape
    L = 3 + n_tok
    cu = np.arange(N + 1, dtype=np.int32) * L
    proc = []
    for s, nm in enumerate(("q_raw", "k_raw", "v_raw")):
        h_s = np.asarray(hist, dtype=np.float64)[:, :, s].transpose(0, 2, 1, 3)  # [N, 3, H, d]
        x = np.concatenate([h_s, f[nm].double().numpy()], axis=1).reshape(N * L, H, d)
        out = oracle.frontend(x, f["conv_w"][s], cu_seqlens=cu, l2=s < 2, eps=l2_eps)
        proc.append(out.reshape(N, L, H, d)[:, 3:])
    S = np.asarray(S0, dtype=np.float64)
    ys = []
    for t in range(n_tok):
        y_t, S = oracle.decode_step(proc[0][:, t], proc[1][:, t], proc[2][:, t], la[:, t],
                                    bt[:, t], S)
        ys.append(y_t)
    y = np.stack(ys, 1)
    o = oracle.output_gate(y, f["z"], f["norm_w"], eps=rms_eps)
    return o, S


@gpu
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n_tok", [1, 4])
def test_decode_fused(d, dtype, n_tok):
    g = _lib()
    f = gi.decode_fused_inputs(5, n_tok, 3, d, dtype, seed=d + n_tok)
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in f.items()}
    cs = dev["conv_state"].clone()
    S = dev["S0"].clone()
    o = g.gdn_decode_fused(dev["q_raw"], dev["k_raw"], dev["v_raw"], dev["conv_w"], cs,
                           dev["log_alpha"], dev["beta"], S, dev["z"], norm_w=dev["norm_w"],
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, S_ref = _fused_decode_reference(f, f["conv_state"].double().numpy(), f["S0"],
                                           f["log_alpha"].double().numpy(),
                                           f["beta"].double().numpy())
    eo, es = rel_l2(o, o_ref), rel_l2(S, S_ref)
    print("fused decode rel_l2 o=%.3e S=%.3e" % (eo, es), flush=True)
    assert eo <= TOL[dtype] and es <= TOL[dtype], (eo, es)
    # the new convolution history is the last three raw rows, bit for bit
    rows = torch.cat([f["conv_state"].permute(0, 2, 3, 1, 4)[:, :, :, :, :],
                      torch.stack([f["q_raw"], f["k_raw"], f["v_raw"]], 1)], 2)  # [N,3,3+n,H,d]
    want = rows[:, :, -3:].permute(0, 3, 1, 2, 4).contiguous()  # [N, H, 3, 3, d]
    assert torch.equal(cs.cpu(), want)


@gpu
def test_decode_fused_slots_match_unfused_chain():
    """With a slot table, the fused decode leaves the same states in the same
    slots as the oracle chain, the conv cache follows the state, and padding
    entries write nothing."""
    g = _lib()
    N, n_tok, H, d, n_slots = 3, 3, 2, 128, 12
    f = gi.decode_fused_inputs(N, n_tok, H, d, "bf16", seed=77)
    pool_S = gi.normal((n_slots, H, d, d), 78, 1, std=0.02)
    pool_c = gi.normal((n_slots, H, 3, 3, d), 78, 2).to(torch.bfloat16)
    table = torch.tensor([[5, 6, 7, 5], [-1, 8, 9, 10], [2, -1, -1, 11]], dtype=torch.int32)
    a, b, A, b_alpha = gi.raw_gates(N * n_tok, H, 79)
    ga, gb = a.reshape(N, n_tok, H).contiguous(), b.reshape(N, n_tok, H).contiguous()
    S, cs = pool_S.clone().cuda(), pool_c.clone().cuda()
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in f.items()}
    o = g.gdn_decode_fused(dev["q_raw"], dev["k_raw"], dev["v_raw"], dev["conv_w"], cs,
                           ga.cuda(), gb.cuda(), S, dev["z"], A=A.cuda(), b_alpha=b_alpha.cuda(),
                           state_idx=table.cuda(), norm_w=dev["norm_w"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    la, bt = oracle.gates_from_raw(a, b, A, b_alpha)
    la, bt = la.reshape(N, n_tok, H), bt.reshape(N, n_tok, H)
    Sc, cc, oc = S.cpu(), cs.cpu(), o.cpu()
    touched = set()
    for n in range(N):
        start = int(table[n, 0])
        if start < 0:
            assert torch.all(oc[n] == 0)
            continue
        fn = {k: (v[n:n + 1] if isinstance(v, torch.Tensor) and k in
                  ("q_raw", "k_raw", "v_raw", "z") else v) for k, v in f.items()}
        raw_rows = torch.stack([f["q_raw"][n], f["k_raw"][n], f["v_raw"][n]], 0)  # [3,n_tok,H,d]
        for t in range(n_tok):
            w = int(table[n, 1 + t])
            if w < 0:
                continue
            sub = {k: (v[:, :t + 1].contiguous() if k in ("q_raw", "k_raw", "v_raw", "z") else v)
                   for k, v in fn.items()}
            o_ref, S_ref = _fused_decode_reference(sub, pool_c[start:start + 1].double().numpy(),
                                                   pool_S[start:start + 1], la[n:n + 1, :t + 1],
                                                   bt[n:n + 1, :t + 1])
            assert rel_l2(Sc[w:w + 1], S_ref) <= 2e-3
            assert rel_l2(oc[n:n + 1, :t + 1], o_ref) <= 2e-3
            hist = torch.cat([pool_c[start].permute(1, 2, 0, 3), raw_rows[:, :t + 1]], 1)
            assert torch.equal(cc[w], hist[:, -3:].permute(2, 0, 1, 3))
            touched.add(w)
    for sl in range(n_slots):
        if sl not in touched:
            assert torch.equal(Sc[sl], pool_S[sl]) and torch.equal(cc[sl], pool_c[sl]), sl


# ------------------------------------------------------------- backward -----
def _bwd_inputs(lengths, H, dk, dv, dtype, seed, s0=True, dst=True):
    inp = gi.prefill_inputs(len(lengths), H, 0, dk, dv, dtype, s0_std=0.02 if s0 else 0.0,
                            seed=seed, lengths=lengths)
    rows = inp["q"].shape[0]
    dy = gi.normal((rows, H, dv), seed, 40)
    dST = gi.normal((len(lengths), H, dk, dv), seed, 41) if dst else None
    return inp, dy, dST


def _check_bwd(inp, dy, dST, grad_dtype=torch.float32, tol=None):
    g = _lib()
    d = to_dev(inp)
    dyd = dy.to(grad_dtype).cuda()
    grads = g.gdn_chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], dyd, S0=d["S0"],
                            dS_T=None if dST is None else dST.cuda(),
                            cu_seqlens=d["cu_seqlens"], N=d["N"], grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    ref = oracle.gdn_bwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["S0"],
                         dyd.cpu(), dST, cu_seqlens=inp["cu_seqlens"], N=inp["N"])
    tol = TOL[inp["dtype"]] if tol is None else tol
    names = ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dS0")
    errs = {}
    for nm, got, want in zip(names, grads, ref):
        errs[nm] = rel_l2(got, want)
    print("bwd rel_l2 " + " ".join("%s=%.2e" % kv for kv in errs.items()), flush=True)
    for nm, e in errs.items():
        assert np.isfinite(e) and e <= tol, (nm, e)
    return grads


@gpu
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk_bwd_varlen(d, dtype):
    # fp32 inputs: every product in fp32 (1e-5); 16-bit inputs: fp16 operands (2e-3)
    inp, dy, dST = _bwd_inputs([1, 31, 32, 33, 100, 0, 65], 2, d, d, dtype, seed=100 + d)
    _check_bwd(inp, dy, dST, tol=TOL[dtype])


@gpu
@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 64)])
def test_chunk_bwd_rect_heads_no_state(dk, dv):
    inp, dy, _ = _bwd_inputs([70, 9], 3, dk, dv, "f32", seed=dk + 2 * dv, s0=False, dst=False)
    _check_bwd(inp, dy, None, tol=1e-5)


@gpu
@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 64)])
def test_chunk_bwd_rect_heads_bf16(dk, dv):
    # 16-bit inputs: the chunk-start states come from the prefill kernel
    inp, dy, dST = _bwd_inputs([70, 9, 33], 3, dk, dv, "bf16", seed=dk + 3 * dv)
    _check_bwd(inp, dy, dST, tol=TOL["bf16"])


@gpu
@pytest.mark.parametrize("case", ["no_decay", "strong_decay", "beta0", "beta1", "repeated_keys",
                                  "near_parallel", "large_v", "banded_decay"])
def test_chunk_bwd_gate_extremes_bf16(case):
    # 16-bit inputs (fp16 operands); strong and banded decay also take the
    # prefill kernel's per-element decay path for the chunk-start states
    inp, dy, dST = _bwd_inputs([90, 40], 2, 128, 128, "bf16", seed=125)
    rows = inp["q"].shape[0]
    if case == "no_decay":
        inp["log_alpha"] = torch.zeros(rows, 2)
    elif case == "strong_decay":
        inp["log_alpha"] = torch.full((rows, 2), -30.0)
    elif case == "beta0":
        inp["beta"] = torch.zeros(rows, 2)
    elif case == "beta1":
        inp["beta"] = torch.ones(rows, 2)
    elif case == "repeated_keys":
        inp["k"][1::2] = inp["k"][0::2][: inp["k"][1::2].shape[0]]
    elif case == "near_parallel":
        base = inp["k"][:1].float()
        kk = base + gi.normal(inp["k"].shape, 78, 1) * 1e-2
        inp["k"] = (kk / kk.norm(dim=-1, keepdim=True)).to(inp["k"].dtype)
    elif case == "large_v":
        inp["v"] = (inp["v"].float() * 64.0).to(inp["v"].dtype)
    else:  # banded decay: 40-token bands alternate between none and log alpha = -12
        band = (torch.arange(rows) // 40) % 2 == 1
        inp["log_alpha"][band] = -12.0
    _check_bwd(inp, dy, dST, tol=TOL["bf16"])


@gpu
def test_chunk_bwd_equal_length_bf16_grads_and_deterministic():
    g = _lib()
    inp = gi.prefill_inputs(2, 4, 200, 128, 128, "bf16", s0_std=0.02, seed=110)
    dy = gi.normal((400, 4, 128), 110, 40)
    inp2 = dict(inp)
    grads = _check_bwd(inp2, dy, None, grad_dtype=torch.bfloat16, tol=2e-3)
    d = to_dev(inp)
    again = g.gdn_chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                            dy.to(torch.bfloat16).cuda(), S0=d["S0"], N=2,
                            grad_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for a_, b_ in zip(grads, again):
        assert torch.equal(a_, b_)


@gpu
@pytest.mark.parametrize("case", ["no_decay", "strong_decay", "beta0", "beta1"])
def test_chunk_bwd_gate_extremes(case):
    inp, dy, dST = _bwd_inputs([90, 40], 2, 64, 64, "f32", seed=120)
    rows = inp["q"].shape[0]
    if case == "no_decay":
        inp["log_alpha"] = torch.zeros(rows, 2)
    elif case == "strong_decay":
        inp["log_alpha"] = torch.full((rows, 2), -30.0)
    elif case == "beta0":
        inp["beta"] = torch.zeros(rows, 2)
    else:
        inp["beta"] = torch.ones(rows, 2)
    _check_bwd(inp, dy, dST, tol=1e-5)


@gpu
@pytest.mark.parametrize("with_bias", [False, True])
def test_chunk_bwd_gated(with_bias):
    """Backward through the in-kernel gate map against the oracle chain:
    backward recurrence, then the gate map's chain rule."""
    g = _lib()
    inp, dy, dST = _bwd_inputs([70, 33, 1], 2, 64, 64, "bf16", seed=130)
    rows = inp["q"].shape[0]
    a, b, A, b_alpha = gi.raw_gates(rows, 2, 131)
    if not with_bias:
        b_alpha = None
    d = to_dev(inp)
    out = g.gdn_chunk_bwd_gated(d["q"], d["k"], d["v"], a.cuda(), b.cuda(), A.cuda(), dy.cuda(),
                                b_alpha=None if b_alpha is None else b_alpha.cuda(), S0=d["S0"],
                                dS_T=dST.cuda(), cu_seqlens=d["cu_seqlens"])
    torch.cuda.synchronize()
    la, bt = oracle.gates_from_raw(a, b, A, b_alpha)
    dq, dk, dv, dla, dbt, dS0 = oracle.gdn_bwd(inp["q"], inp["k"], inp["v"], la, bt, inp["S0"],
                                               dy, dST, cu_seqlens=inp["cu_seqlens"],
                                               N=inp["N"])
    da, db, dA, dba = oracle.gates_from_raw_bwd(a, b, A, b_alpha, dla, dbt)
    want = (dq, dk, dv, da, db, dA, dba, dS0)
    names = ("dq", "dk", "dv", "da", "db", "dA", "db_alpha", "dS0")
    for nm, got, w in zip(names, out, want):
        e = rel_l2(got, w)
        print(nm, "%.2e" % e, flush=True)
        assert e <= TOL["bf16"], (nm, e)


@gpu
@pytest.mark.parametrize("ns,dv", [(1, 64), (1, 128), (4, 64), (4, 128), (8, 128)])
def test_chunk_bwd_states_from_wide_state_tiles(ns, dv, monkeypatch):
    """The backward's chunk-start states written by the prefill with one,
    four or eight state waves (16-, 64- or 128-column workgroups, stored as
    the backward's 32-column tiles) give the two-wave gradients bit for
    bit."""
    g = _lib()
    inp, dy, dST = _bwd_inputs([1, 31, 32, 33, 100, 0, 65, 200], 2, 128, dv, "bf16", seed=152)
    d = to_dev(inp)

    def run():
        out = g.gdn_chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], dy.cuda(),
                              S0=d["S0"], dS_T=dST.cuda(), cu_seqlens=d["cu_seqlens"],
                              N=d["N"])
        torch.cuda.synchronize()
        return [t.cpu() for t in out]

    monkeypatch.setenv("GDN_PREFILL_NS", "2")
    two = run()
    monkeypatch.setenv("GDN_PREFILL_NS", str(ns))
    four = run()
    for nm, a, b in zip(("dq", "dk", "dv", "dlog_alpha", "dbeta", "dS0"), two, four):
        assert torch.equal(a, b), nm


_RUN_HOOKS = ("GDN_BWD_RUNS", "GDN_BWD_SEGMENT_ROWS")


def _one_run_vs_split(monkeypatch, run, hook, value):
    """run() once as a single run and once split by the hook."""
    for h in _RUN_HOOKS:
        monkeypatch.delenv(h, raising=False)
    one = run()
    monkeypatch.setenv(hook, str(value))
    split = run()
    monkeypatch.delenv(hook)
    return one, split


@gpu
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("hook,value", [("GDN_BWD_RUNS", 3), ("GDN_BWD_RUNS", 9),
                                        ("GDN_BWD_SEGMENT_ROWS", 32),
                                        ("GDN_BWD_SEGMENT_ROWS", 96)])
@pytest.mark.parametrize("varlen", [True, False])
def test_chunk_bwd_runs_equal_one_run(dtype, hook, value, varlen, monkeypatch):
    """A backward split into runs (forced small by the hooks; long problems
    are split to bound the workspace) gives the one-run gradients bit for
    bit: proportional runs (every sequence in every run, sequences with
    fewer chunks than runs leaving some runs empty) and runs of consecutive
    rows (sequences straddling runs), a sequence without rows included, and
    the oracle's to the bar."""
    g = _lib()
    if varlen:
        inp, dy, dST = _bwd_inputs([1, 31, 32, 33, 100, 0, 65, 200], 2, 64, 64, dtype, seed=150)
    else:  # equal lengths with a ragged last chunk
        inp = gi.prefill_inputs(3, 2, 200, 64, 64, dtype, s0_std=0.02, seed=151)
        dy = gi.normal((600, 2, 64), 151, 40)
        dST = gi.normal((3, 2, 64, 64), 151, 41)
    d = to_dev(inp)

    def run():
        out = g.gdn_chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], dy.cuda(),
                              S0=d["S0"], dS_T=dST.cuda(), cu_seqlens=d["cu_seqlens"],
                              N=d["N"])
        torch.cuda.synchronize()
        return [t.cpu() for t in out]

    one, split = _one_run_vs_split(monkeypatch, run, hook, value)
    for nm, a, b in zip(("dq", "dk", "dv", "dlog_alpha", "dbeta", "dS0"), one, split):
        assert torch.equal(a, b), nm
    _check_bwd(inp, dy, dST, tol=TOL[dtype])


@gpu
@pytest.mark.parametrize("hook,value", [("GDN_BWD_RUNS", 4), ("GDN_BWD_SEGMENT_ROWS", 64)])
def test_chunk_bwd_gated_runs(hook, value, monkeypatch):
    """The raw-gate backward split into runs: per-row gradients as one run
    bit for bit, the per-head sums dA and db_alpha (added run by run) to
    fp32 rounding."""
    g = _lib()
    inp, dy, dST = _bwd_inputs([70, 33, 1, 130], 2, 64, 64, "bf16", seed=160)
    rows = inp["q"].shape[0]
    a, b, A, b_alpha = gi.raw_gates(rows, 2, 161)
    d = to_dev(inp)

    def run():
        out = g.gdn_chunk_bwd_gated(d["q"], d["k"], d["v"], a.cuda(), b.cuda(), A.cuda(),
                                    dy.cuda(), b_alpha=b_alpha.cuda(), S0=d["S0"],
                                    dS_T=dST.cuda(), cu_seqlens=d["cu_seqlens"])
        torch.cuda.synchronize()
        return [t.cpu() for t in out]

    one, split = _one_run_vs_split(monkeypatch, run, hook, value)
    names = ("dq", "dk", "dv", "da", "db", "dA", "db_alpha", "dS0")
    for nm, x, y in zip(names, one, split):
        if nm in ("dA", "db_alpha"):
            assert rel_l2(y, x.double().numpy()) <= 1e-5, nm
        else:
            assert torch.equal(x, y), nm


# ---------------------------------------------- prefill -> decode handoff -----
@gpu
def test_conv_state_from_prefill_is_the_last_raw_rows():
    g = _lib()
    lengths = [5, 1, 0, 2, 40]
    f = gi.frontend_inputs(lengths, 2, 64, 64, "bf16", seed=140)
    cu = f["cu_seqlens"]
    slots = torch.tensor([3, 0, 5, -1, 1], dtype=torch.int32)
    cs = torch.full((6, 2, 3, 3, 64), 7.0, dtype=torch.bfloat16).cuda()
    g.gdn_conv_state_from_prefill(f["q_raw"].cuda(), f["k_raw"].cuda(), f["v_raw"].cuda(),
                                  cu_seqlens=cu.cuda(), slot_idx=slots.cuda(), conv_state=cs)
    torch.cuda.synchronize()
    cs = cs.cpu()
    for n, L in enumerate(lengths):
        sl = int(slots[n])
        if sl < 0:
            continue
        want = torch.zeros(2, 3, 3, 64, dtype=torch.bfloat16)
        for s, nm in enumerate(("q_raw", "k_raw", "v_raw")):
            rows = f[nm][int(cu[n]):int(cu[n + 1])]
            for r in range(3):
                t = L - 3 + r
                if t >= 0:
                    want[:, s, r] = rows[t]
        assert torch.equal(cs[sl], want), n
    assert torch.all(cs[2] == 7.0) and torch.all(cs[4] == 7.0)  # untouched slots


@gpu
def test_prefill_then_fused_decode_equals_one_sequence():
    """Serving path: fused prefill of a varlen batch, conv cache and states
    seeded into slots, then 3 fused decode tokens; the decode outputs and
    final states equal the oracle chain run over each whole sequence."""
    g = _lib()
    lengths, n_dec, H, d = [50, 3, 1, 97], 3, 2, 64
    N = len(lengths)
    total = [L + n_dec for L in lengths]
    f = gi.frontend_inputs(total, H, d, d, "bf16", seed=141, norm_w_std=0.1)
    cu_all = f["cu_seqlens"]
    pre_rows = torch.cat([torch.arange(int(cu_all[n]), int(cu_all[n]) + lengths[n])
                          for n in range(N)])
    dec_rows = torch.stack([torch.arange(int(cu_all[n]) + lengths[n], int(cu_all[n + 1]))
                            for n in range(N)])  # [N, n_dec]
    cu_pre = gi.cu_from_lengths(lengths)
    take = lambda x, r: x[r].contiguous()
    dev = lambda x: x.cuda()
    # prefill
    o_pre, S_T = g.gdn_chunk_fwd_fused(*(dev(take(f[nm], pre_rows)) for nm in
                                         ("q_raw", "k_raw", "v_raw")), dev(f["conv_w"]),
                                       dev(take(f["log_alpha"], pre_rows)),
                                       dev(take(f["beta"], pre_rows)), dev(take(f["z"], pre_rows)),
                                       S0=dev(f["S0"]), norm_w=dev(f["norm_w"]),
                                       cu_seqlens=dev(cu_pre), out_dtype=torch.float32)
    # hand-off into a pool of slots
    n_slots = 8
    slots = torch.tensor([6, 2, 0, 5], dtype=torch.int32)
    pool = torch.zeros((n_slots, H, d, d), dtype=torch.float32).cuda()
    pool[slots.long().cuda()] = S_T
    cs = g.gdn_conv_state_from_prefill(*(dev(take(f[nm], pre_rows)) for nm in
                                         ("q_raw", "k_raw", "v_raw")), cu_seqlens=dev(cu_pre),
                                       slot_idx=dev(slots), n_slots=n_slots)
    table = torch.cat([slots[:, None], torch.full((N, n_dec - 1), -1, dtype=torch.int32),
                       slots[:, None]], 1)
    decin = {nm: dev(f[nm][dec_rows]) for nm in ("q_raw", "k_raw", "v_raw", "z", "log_alpha",
                                                 "beta")}
    o_dec = g.gdn_decode_fused(decin["q_raw"], decin["k_raw"], decin["v_raw"], dev(f["conv_w"]),
                               cs, decin["log_alpha"], decin["beta"], pool, decin["z"],
                               state_idx=dev(table), norm_w=dev(f["norm_w"]),
                               out_dtype=torch.float32)
    torch.cuda.synchronize()
    # the oracle over each whole sequence
    qkv = [oracle.frontend(f[nm], f["conv_w"][s], cu_seqlens=cu_all, l2=s < 2, eps=1e-6)
           for s, nm in enumerate(("q_raw", "k_raw", "v_raw"))]
    y, S_ref = oracle.gdn_fwd(qkv[0], qkv[1], qkv[2], f["log_alpha"], f["beta"], f["S0"],
                              cu_seqlens=cu_all)
    o_ref = oracle.output_gate(y, f["z"], f["norm_w"], eps=1e-6)
    e_o = rel_l2(o_dec.cpu().reshape(-1, H, d), o_ref[dec_rows.reshape(-1).numpy()])
    e_s = rel_l2(pool.cpu()[slots.long()], S_ref)
    e_p = rel_l2(o_pre.cpu(), o_ref[pre_rows.numpy()])
    print("handoff rel_l2 prefill o=%.2e decode o=%.2e S=%.2e" % (e_p, e_o, e_s), flush=True)
    assert e_p <= 2e-3 and e_o <= 2e-3 and e_s <= 2e-3


@gpu
def test_chunk_bwd_f16_inputs():
    inp, dy, dST = _bwd_inputs([45, 70], 2, 128, 128, "f16", seed=150)
    _check_bwd(inp, dy, dST, tol=TOL["f16"])


@gpu
@pytest.mark.parametrize("d", [64, 128])
def test_decode_fused_f16_and_raw_gates(d):
    g = _lib()
    f = gi.decode_fused_inputs(4, 3, 2, d, "f16", seed=151)
    a, b, A, b_alpha = gi.raw_gates(12, 2, 152)
    ga, gb = a.reshape(4, 3, 2).contiguous(), b.reshape(4, 3, 2).contiguous()
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in f.items()}
    cs, S = dev["conv_state"].clone(), dev["S0"].clone()
    o = g.gdn_decode_fused(dev["q_raw"], dev["k_raw"], dev["v_raw"], dev["conv_w"], cs, ga.cuda(),
                           gb.cuda(), S, dev["z"], A=A.cuda(), b_alpha=b_alpha.cuda(),
                           norm_w=dev["norm_w"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    la, bt = oracle.gates_from_raw(a, b, A, b_alpha)
    o_ref, S_ref = _fused_decode_reference(f, f["conv_state"].double().numpy(), f["S0"],
                                           la.reshape(4, 3, 2), bt.reshape(4, 3, 2))
    assert rel_l2(o, o_ref) <= 2e-3 and rel_l2(S, S_ref) <= 2e-3


@gpu
@pytest.mark.parametrize("case", ["no_decay", "strong_decay", "beta0", "beta1"])
def test_decode_multi_gate_extremes(case):
    g = _lib()
    N, H, d, n_tok = 3, 2, 64, 4
    inp, tm = _multi_inputs(N, H, d, d, n_tok, "f32", seed=153)
    if case == "no_decay":
        tm["log_alpha"] = torch.zeros_like(tm["log_alpha"])
    elif case == "strong_decay":
        tm["log_alpha"] = torch.full_like(tm["log_alpha"], -30.0)
    elif case == "beta0":
        tm["beta"] = torch.zeros_like(tm["beta"])
    else:
        tm["beta"] = torch.ones_like(tm["beta"])
    S = inp["S0"].clone().cuda()
    y = g.gdn_decode_multi(*(tm[nm].cuda() for nm in ("q", "k", "v", "log_alpha", "beta")), S,
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    S_or = inp["S0"].double().numpy()
    for t in range(n_tok):
        yo, S_or = oracle.decode_step(tm["q"][:, t], tm["k"][:, t], tm["v"][:, t],
                                      tm["log_alpha"][:, t], tm["beta"][:, t], S_or)
        assert rel_l2(y[:, t], yo) <= 1e-5
    assert rel_l2(S, S_or) <= 1e-5


def _check_segmented(inp, segments, out_dtype=None, tol=None):
    tol = TOL[inp["dtype"]] if tol is None else tol
    g = _lib()
    d = to_dev(inp)
    y, S = g.gdn_chunk_fwd_segmented(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], segments,
                                     d["S0"], cu_seqlens=d["cu_seqlens"], out_dtype=out_dtype,
                                     N=d["N"])
    torch.cuda.synchronize()
    yo, So = _oracle_chunk(inp)
    ey, es = rel_l2(_flat(inp, y), yo), rel_l2(S, So)
    print("segments=%d rel_l2 y=%.3e S=%.3e" % (segments, ey, es), flush=True)
    assert np.isfinite(ey) and np.isfinite(es)
    assert ey <= tol and es <= tol, (ey, es)


@gpu
@pytest.mark.parametrize("ns", [1, 4, 8])
@pytest.mark.parametrize("varlen", [False, True])
def test_chunk_segmented_tile_widths(ns, varlen, monkeypatch):
    """The segmented prefill's runs with one, four or eight state waves per
    workgroup (each launch picks its width; forced here by GDN_PREFILL_NS)
    give the two-wave result bit for bit: equal lengths and varlen with an
    empty sequence, 4 segments, bf16."""
    g = _lib()
    if varlen:
        inp = gi.prefill_inputs(0, 2, 0, 128, 128, "bf16", s0_std=0.02, seed=44,
                                lengths=[700, 0, 65, 1000, 33])
    else:
        inp = gi.prefill_inputs(3, 2, 640, 128, 128, "bf16", s0_std=0.02, seed=45)
    d = to_dev(inp)

    def run():
        y, S = g.gdn_chunk_fwd_segmented(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], 4,
                                         d["S0"], cu_seqlens=d["cu_seqlens"],
                                         out_dtype=torch.float32, N=d["N"])
        torch.cuda.synchronize()
        return y.cpu(), S.cpu()

    monkeypatch.setenv("GDN_PREFILL_NS", "2")
    y2, S2 = run()
    monkeypatch.setenv("GDN_PREFILL_NS", str(ns))
    y, S = run()
    assert torch.equal(y, y2) and torch.equal(S, S2)
    yo, So = _oracle_chunk(inp)
    assert rel_l2(_flat(inp, y), yo) <= TOL["bf16"] and rel_l2(S, So) <= TOL["bf16"]


@gpu
@pytest.mark.parametrize("segments", [2, 3, 5])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk_segmented_equal_length(segments, dtype):
    # two sequences of 700 tokens; segments are whole 32-token chunks (352 + 348
    # for two, 256 + 256 + 188 for three)
    inp = gi.prefill_inputs(2, 3, 700, 128, 128, dtype, s0_std=0.02, seed=40 + segments)
    _check_segmented(inp, segments, out_dtype=torch.float32)


@gpu
@pytest.mark.parametrize("segments", [2, 4])
@pytest.mark.parametrize("d", [64, 128])
def test_chunk_segmented_varlen(segments, d):
    # sequences shorter than one segment's chunk leave later segments empty
    lengths = [1, 40, 0, 300, 97, 129]
    inp = gi.prefill_inputs(0, 2, 0, d, d, "bf16", s0_std=0.02, seed=50 + d, lengths=lengths)
    _check_segmented(inp, segments, out_dtype=torch.float32)


@gpu
@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 64)])
def test_chunk_segmented_rect_heads(dk, dv):
    # the transition runs use dv = dk whatever the value width
    inp = gi.prefill_inputs(1, 2, 400, dk, dv, "f32", s0_std=0.02, seed=dk + 5 * dv)
    _check_segmented(inp, 3, out_dtype=torch.float32)


@gpu
def test_chunk_segmented_matches_serial_bf16_out():
    """Same outputs as the serial prefill up to rounding, y in bf16."""
    g = _lib()
    inp = gi.prefill_inputs(1, 4, 1000, 128, 128, "bf16", s0_std=0.02, seed=60)
    d = to_dev(inp)
    y1, S1 = g.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"], N=1)
    y2, S2 = g.gdn_chunk_fwd_segmented(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], 4,
                                       d["S0"], N=1)
    torch.cuda.synchronize()
    assert rel_l2(y2.float().cpu(), y1.float().cpu()) <= 2e-3
    assert rel_l2(S2.cpu(), S1.cpu()) <= 2e-3
    _check_segmented(inp, 4)
