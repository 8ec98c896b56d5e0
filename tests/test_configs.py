"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times, on (sequence, head) units the oracle recomputes one by one.

Bar: relative L2 error <= 2e-3 on y / o and on the final states (bf16 inputs,
fp32 state), per sampled unit; and, so that an error confined to one chunk or
one tail cannot hide in a long unit's average, <= 1e-2 per output row (a row
of dv values, against max(its norm, 5% of the unit's RMS row norm)) and
<= 4e-3 per block of 32 rows.
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
from tests.util import BLOCK_TOL_16, ROW_TOL_16, rel_l2, row_errors

gpu = pytest.mark.gpu
TOL = 2e-3


def _lib():
    import gated_deltanet_amd as g
    g.load_library()
    return g


def _rows_ok(got, ref, what):
    row, block = row_errors(got, ref)
    print("%s: worst row %.3e, worst 32-row block %.3e" % (what, row, block), flush=True)
    assert row <= ROW_TOL_16 and block <= BLOCK_TOL_16, (what, row, block)


def _unit(inp, n, h, T):
    rows = slice(n * T, (n + 1) * T)
    return [inp[key][rows, h:h + 1].contiguous() for key in ("q", "k", "v", "log_alpha", "beta")]


@gpu
def test_prefill_B4_H16_T4096_sampled():
    g = _lib()
    inp = gi.workload_inputs(1)
    dev = {k: v.cuda() for k, v in inp.items() if isinstance(v, torch.Tensor)}
    y, S = g.gdn_chunk_fwd(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], None,
                           N=4)  # bf16 y, as timed
    torch.cuda.synchronize()
    y, S = y.cpu(), S.cpu()
    T = 4096
    for n, h in [(0, 0), (1, 7), (2, 12), (3, 15)]:
        q, k, v, la, b = _unit(inp, n, h, T)
        yo, So = oracle.gdn_fwd(q, k, v, la, b, None, col_blocks=8)
        ey = rel_l2(y[n * T:(n + 1) * T, h], yo[:, 0])
        es = rel_l2(S[n, h], So[0, 0])
        print("unit (%d, %d): y %.3e S %.3e" % (n, h, ey, es), flush=True)
        assert ey <= TOL and es <= TOL
        _rows_ok(y[n * T:(n + 1) * T, h], yo[:, 0], "unit (%d, %d) y" % (n, h))


@gpu
def test_prefill_B1_H32_T65536_sampled():
    g = _lib()
    inp = gi.workload_inputs(2)
    dev = {k: v.cuda() for k, v in inp.items() if isinstance(v, torch.Tensor)}
    y, S = g.gdn_chunk_fwd(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], dev["S0"])
    torch.cuda.synchronize()
    y, S = y.cpu(), S.cpu()
    T = 65536
    for h in (0, 31):
        q, k, v, la, b = _unit(inp, 0, h, T)
        yo, So = oracle.gdn_fwd(q, k, v, la, b, inp["S0"][:, h:h + 1], col_blocks=16)
        ey = rel_l2(y[:, h], yo[:, 0])
        es = rel_l2(S[0, h], So[0, 0])
        print("head %d: y %.3e S %.3e" % (h, ey, es), flush=True)
        assert ey <= TOL and es <= TOL
        _rows_ok(y[:, h], yo[:, 0], "head %d y" % h)


@gpu
@pytest.mark.parametrize("segments", [4, 9])
def test_prefill_B1_H32_T65536_segmented_sampled(segments):
    """The long-context workload through the segment-parallel form (4 or 9
    segments of 16 384 or 7 296 tokens, the last shorter; the runs take their
    own column-tile width), on two heads the oracle recomputes."""
    g = _lib()
    inp = gi.workload_inputs(2)
    dev = {k: v.cuda() for k, v in inp.items() if isinstance(v, torch.Tensor)}
    y, S = g.gdn_chunk_fwd_segmented(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"],
                                     segments, dev["S0"])
    torch.cuda.synchronize()
    y, S = y.cpu(), S.cpu()
    T = 65536
    for h in (3, 20):
        q, k, v, la, b = _unit(inp, 0, h, T)
        yo, So = oracle.gdn_fwd(q, k, v, la, b, inp["S0"][:, h:h + 1], col_blocks=16)
        ey = rel_l2(y[:, h], yo[:, 0])
        es = rel_l2(S[0, h], So[0, 0])
        print("head %d: y %.3e S %.3e" % (h, ey, es), flush=True)
        assert ey <= TOL and es <= TOL
        _rows_ok(y[:, h], yo[:, 0], "head %d y" % h)


@gpu
def test_decode_N256_H32_sampled():
    """All 128 steps of the decode workload (256 sequences x 32 heads, as the
    benchmark times them), sampled units including the first and the last."""
    g = _lib()
    steps = 128
    inp = gi.workload_inputs(3, steps=steps)
    S = inp["S0"].cuda()
    dq, dk_, dv_ = inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda()
    dla, db = inp["log_alpha"].cuda(), inp["beta"].cuda()
    units = [(0, 0), (17, 5), (128, 31), (255, 16), (200, 2), (255, 31)]
    ys = {u: [] for u in units}
    for t in range(steps):
        yt = g.gdn_decode_step(dq[t], dk_[t], dv_[t], dla[t], db[t], S)
        for u in units:
            ys[u].append(yt[u[0], u[1]])
    torch.cuda.synchronize()
    ys = {u: torch.stack(v).cpu() for u, v in ys.items()}
    Sc = S.cpu()
    for n, h in units:
        Su = inp["S0"][n:n + 1, h:h + 1].double().numpy()
        yo = []
        for t in range(steps):
            args = [inp[key][t, n:n + 1, h:h + 1] for key in ("q", "k", "v", "log_alpha", "beta")]
            yt, Su = oracle.decode_step(*args, Su)
            yo.append(yt[0, 0])
        ey = rel_l2(ys[(n, h)], np.stack(yo))
        es = rel_l2(Sc[n, h], Su[0, 0])
        print("unit (%d, %d): y %.3e S %.3e" % (n, h, ey, es), flush=True)
        assert ey <= TOL and es <= TOL
        _rows_ok(ys[(n, h)], np.stack(yo), "unit (%d, %d) y" % (n, h))


def run_frontend_chain(g, dev, out_dtype=torch.bfloat16):
    """Front end (fp16 q/k/v) -> chunked prefill (fp16 y) -> output gate."""
    q, k, v = g.gdn_frontend_qkv(dev["q_raw"], dev["k_raw"], dev["v_raw"], dev["conv_w"],
                                 cu_seqlens=dev["cu_seqlens"], l2_eps=1e-6,
                                 out_dtype=torch.float16)
    y, S = g.gdn_chunk_fwd(q, k, v, dev["log_alpha"], dev["beta"], dev["S0"],
                           cu_seqlens=dev["cu_seqlens"], out_dtype=torch.float16)
    o = g.gdn_output_gate(y, dev["z"], dev["norm_w"], 1e-6, out_dtype=out_dtype)
    return o, S


def oracle_frontend_chain(f, n, h):
    cu = f["cu_seqlens"]
    s, e = int(cu[n]), int(cu[n + 1])
    w = f["conv_w"]
    H = f["H"]
    d = f["dk"]
    sl = lambda x: x[s:e, h:h + 1]
    wsl = lambda i: w[i].reshape(H, d, -1)[h]
    q = oracle.frontend(sl(f["q_raw"]), wsl(0), l2=True, eps=1e-6)
    k = oracle.frontend(sl(f["k_raw"]), wsl(1), l2=True, eps=1e-6)
    v = oracle.frontend(sl(f["v_raw"]), wsl(2), l2=False)
    y, S = oracle.gdn_fwd(q, k, v, sl(f["log_alpha"]), sl(f["beta"]), f["S0"][n:n + 1, h:h + 1],
                          col_blocks=8)
    o = oracle.output_gate(y, sl(f["z"]), f["norm_w"], eps=1e-6)
    return o[:, 0], S[0, 0]


@gpu
@pytest.mark.parametrize("norm_w_std", [0.0, 0.1])
def test_varlen_frontend_chain_sampled(norm_w_std):
    """Front-end workload distributions on 12 sequences (lengths from the
    workload's U[512, 8192] draw plus edge lengths), all heads on the GPU,
    sampled (sequence, head) units against the oracle chain."""
    g = _lib()
    lengths = gi.seq_lengths(64, 512, 8192, seed=4)[:8].tolist() + [1, 31, 33, 515]
    f = gi.frontend_inputs(lengths, 16, 128, 128, dtype="bf16", seed=4, norm_w_std=norm_w_std)
    dev = {k: v.cuda() for k, v in f.items() if isinstance(v, torch.Tensor)}
    o, S = run_frontend_chain(g, dev)
    torch.cuda.synchronize()
    o, S = o.cpu(), S.cpu()
    cu = f["cu_seqlens"]
    for n, h in [(0, 0), (3, 9), (7, 15), (8, 4), (10, 1), (11, 13)]:
        oo, So = oracle_frontend_chain(f, n, h)
        s, e = int(cu[n]), int(cu[n + 1])
        eo = rel_l2(o[s:e, h], oo)
        es = rel_l2(S[n, h], So)
        print("unit (%d, %d) len %d: o %.3e S %.3e" % (n, h, e - s, eo, es), flush=True)
        assert eo <= TOL and es <= TOL
        _rows_ok(o[s:e, h], oo, "unit (%d, %d) o" % (n, h))


@gpu
def test_varlen_fused_timed_batch_sampled():
    """The varlen front-end workload exactly as the benchmark times it: all 64
    sequences (254 539 tokens at seed 4), 16 heads, through gdn_chunk_fwd_fused
    with bf16 o; eight (sequence, head) units against the oracle chain,
    including the longest and the shortest sequence."""
    g = _lib()
    f = gi.workload_inputs(4)
    dev = {k: v.cuda() for k, v in f.items() if isinstance(v, torch.Tensor)}
    o, S = g.gdn_chunk_fwd_fused(dev["q_raw"], dev["k_raw"], dev["v_raw"], dev["conv_w"],
                                 dev["log_alpha"], dev["beta"], dev["z"], S0=dev["S0"],
                                 norm_w=dev["norm_w"], cu_seqlens=dev["cu_seqlens"],
                                 out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    cu = f["cu_seqlens"]
    assert int(cu[-1]) == 254539
    lens = (cu[1:] - cu[:-1]).tolist()
    order = sorted(range(len(lens)), key=lambda n: lens[n])
    picks = [order[-1], order[0], order[1], order[-2], order[32], 5, 40, 63]
    for i, n in enumerate(picks):
        h = (7 * i + 2) % 16
        s0, e0 = int(cu[n]), int(cu[n + 1])
        oo, So = oracle_frontend_chain(f, n, h)
        got = o[s0:e0, h].cpu()
        eo = rel_l2(got, oo)
        es = rel_l2(S[n, h].cpu(), So)
        print("unit (%d, %d) len %d: o %.3e S %.3e" % (n, h, e0 - s0, eo, es), flush=True)
        assert eo <= TOL and es <= TOL
        _rows_ok(got, oo, "unit (%d, %d) o" % (n, h))


@gpu
def test_fused_prefill_matches_chain_and_oracle():
    """gdn_chunk_fwd_fused equals the three separate calls bit for bit (same
    kernels, same intermediate dtypes) and the oracle chain to the bar."""
    g = _lib()
    lengths = gi.seq_lengths(64, 512, 8192, seed=5)[:6].tolist() + [1, 2, 33, 517]
    f = gi.frontend_inputs(lengths, 16, 128, 128, dtype="bf16", seed=5, norm_w_std=0.1)
    dev = {k: v.cuda() for k, v in f.items() if isinstance(v, torch.Tensor)}
    o_chain, S_chain = run_frontend_chain(g, dev)
    o, S = g.gdn_chunk_fwd_fused(dev["q_raw"], dev["k_raw"], dev["v_raw"], dev["conv_w"],
                                 dev["log_alpha"], dev["beta"], dev["z"], S0=dev["S0"],
                                 norm_w=dev["norm_w"], l2_eps=1e-6, rms_eps=1e-6,
                                 cu_seqlens=dev["cu_seqlens"], out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o, o_chain) and torch.equal(S, S_chain)
    o, S = o.cpu(), S.cpu()
    cu = f["cu_seqlens"]
    for n, h in [(0, 3), (5, 11), (6, 0), (7, 15), (8, 8), (9, 2)]:
        oo, So = oracle_frontend_chain(f, n, h)
        s, e = int(cu[n]), int(cu[n + 1])
        eo = rel_l2(o[s:e, h], oo)
        es = rel_l2(S[n, h], So)
        print("unit (%d, %d) len %d: o %.3e S %.3e" % (n, h, e - s, eo, es), flush=True)
        assert eo <= TOL and es <= TOL
        _rows_ok(o[s:e, h], oo, "unit (%d, %d) o" % (n, h))


@gpu
def test_backward_B4_H16_T4096_sampled():
    """gdn_chunk_bwd at the prefill workload's size (bf16 inputs, bf16 dy and
    gradients, as the benchmark times it), two units checked against the
    oracle's backward on that unit alone."""
    g = _lib()
    inp = gi.workload_inputs(1)
    dev = {k: v.cuda() for k, v in inp.items() if isinstance(v, torch.Tensor)}
    T, H = 4096, 16
    dy = gi.normal((4 * T, H, 128), 13, 40).to(torch.bfloat16)
    grads = g.gdn_chunk_bwd(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"],
                            dy.cuda(), N=4, want_dS0=True)
    torch.cuda.synchronize()
    grads = [x.cpu() for x in grads]
    for n, h in [(0, 3), (3, 14)]:
        q, k, v, la, b = _unit(inp, n, h, T)
        dyu = dy[n * T:(n + 1) * T, h:h + 1]
        ref = oracle.gdn_bwd(q, k, v, la, b, None, dyu, None, N=1)
        rows = slice(n * T, (n + 1) * T)
        got = [grads[0][rows, h:h + 1], grads[1][rows, h:h + 1], grads[2][rows, h:h + 1],
               grads[3][rows, h:h + 1], grads[4][rows, h:h + 1], grads[5][n:n + 1, h:h + 1]]
        for nm, gg, rr in zip(("dq", "dk", "dv", "dla", "dbeta", "dS0"), got, ref):
            e = rel_l2(gg, rr)
            print("unit", n, h, nm, "%.2e" % e, flush=True)
            assert e <= TOL, (n, h, nm, e)


@gpu
def test_backward_many_short_sequences_sampled():
    """gdn_chunk_bwd on a packed batch of 512 sequences of 1-256 tokens (about
    65 000 rows, H = 16, d = 128, bf16) as the library plans it by itself:
    the partial sums of all rows exceed the workspace bound, so the sweep
    runs over consecutive rows in many runs, and sequences that straddle a
    run boundary carry their state gradient from run to run. Sampled
    sequences (the shortest, the longest, and those holding rows at run
    boundaries) against the oracle's backward of that sequence alone."""
    g = _lib()
    H, d = 16, 128
    lengths = gi.seq_lengths(512, 1, 256, seed=17).tolist()
    inp = gi.prefill_inputs(0, H, 0, d, d, "bf16", s0_std=0.02, seed=17, lengths=lengths)
    rows = inp["q"].shape[0]
    per_row = (d // 32) * H * (2 * d + 2) * 4
    ws = g.gdn_chunk_bwd_workspace_size(rows, 512, H, d, d, torch.bfloat16)
    assert ws < rows * per_row  # the partial sums are kept for one run at a time
    dy = gi.normal((rows, H, d), 17, 40).to(torch.bfloat16)
    dST = gi.normal((512, H, d, d), 17, 41)
    dev = {k: v.cuda() for k, v in inp.items() if isinstance(v, torch.Tensor)}
    grads = g.gdn_chunk_bwd(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"],
                            dy.cuda(), S0=dev["S0"], dS_T=dST.cuda(),
                            cu_seqlens=dev["cu_seqlens"], N=512)
    torch.cuda.synchronize()
    grads = [x.cpu() for x in grads]
    cu = inp["cu_seqlens"].tolist()
    order = sorted(range(512), key=lambda n: lengths[n])

    def holding(row):  # the sequence that holds a row
        return max(n for n in range(512) if cu[n] <= row and cu[n + 1] > row)

    picks = {order[0], order[-1]} | {holding(r) for r in (3008, 6016, 30080, 60160)}
    for i, n in enumerate(sorted(picks)):
        h = (5 * i + 1) % H
        s0, e0 = cu[n], cu[n + 1]
        unit = [inp[key][s0:e0, h:h + 1].contiguous()
                for key in ("q", "k", "v", "log_alpha", "beta")]
        ref = oracle.gdn_bwd(*unit, inp["S0"][n:n + 1, h:h + 1], dy[s0:e0, h:h + 1],
                             dST[n:n + 1, h:h + 1], N=1)
        got = [grads[0][s0:e0, h:h + 1], grads[1][s0:e0, h:h + 1], grads[2][s0:e0, h:h + 1],
               grads[3][s0:e0, h:h + 1], grads[4][s0:e0, h:h + 1], grads[5][n:n + 1, h:h + 1]]
        for nm, gg, rr in zip(("dq", "dk", "dv", "dla", "dbeta", "dS0"), got, ref):
            e = rel_l2(gg, rr)
            print("sequence", n, "len", e0 - s0, "head", h, nm, "%.2e" % e, flush=True)
            assert e <= TOL, (n, h, nm, e)


@gpu
def test_prefill_and_backward_B16_H16_T2048_sampled():
    """A large equal-length batch (B = 16, H = 16, T = 2048, bf16): the
    prefill takes whole-head workgroups (eight state waves, 128 columns) and
    the backward's chunk-start states come from the same kernel, while the
    backward sweep runs in proportional runs. Sampled units of y, S_T and of
    every gradient against the oracle on that unit alone."""
    g = _lib()
    B, H, T, d = 16, 16, 2048, 128
    assert g.gdn_prefill_state_columns(B, H, d, d, torch.bfloat16) == 128
    inp = gi.prefill_inputs(B, H, T, d, d, "bf16", s0_std=0.02, seed=23)
    dev = {k: v.cuda() for k, v in inp.items() if isinstance(v, torch.Tensor)}
    y, S = g.gdn_chunk_fwd(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"],
                           dev["S0"], N=B)
    dy = gi.normal((B * T, H, d), 23, 40).to(torch.bfloat16)
    grads = g.gdn_chunk_bwd(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"],
                            dy.cuda(), S0=dev["S0"], N=B)
    torch.cuda.synchronize()
    y, S = y.cpu(), S.cpu()
    grads = [x.cpu() for x in grads]
    for n, h in [(0, 0), (7, 9), (15, 15)]:
        q, k, v, la, b = _unit(inp, n, h, T)
        S0u = inp["S0"][n:n + 1, h:h + 1]
        rows = slice(n * T, (n + 1) * T)
        yo, So = oracle.gdn_fwd(q, k, v, la, b, S0u, col_blocks=8)
        ey, es = rel_l2(y[rows, h], yo[:, 0]), rel_l2(S[n, h], So[0, 0])
        print("unit (%d, %d): y %.3e S %.3e" % (n, h, ey, es), flush=True)
        assert ey <= TOL and es <= TOL
        _rows_ok(y[rows, h], yo[:, 0], "unit (%d, %d) y" % (n, h))
        ref = oracle.gdn_bwd(q, k, v, la, b, S0u, dy[rows, h:h + 1], None, N=1)
        got = [grads[0][rows, h:h + 1], grads[1][rows, h:h + 1], grads[2][rows, h:h + 1],
               grads[3][rows, h:h + 1], grads[4][rows, h:h + 1], grads[5][n:n + 1, h:h + 1]]
        for nm, gg, rr in zip(("dq", "dk", "dv", "dla", "dbeta", "dS0"), got, ref):
            e = rel_l2(gg, rr)
            print("unit", n, h, nm, "%.2e" % e, flush=True)
            assert e <= TOL, (n, h, nm, e)


@gpu
def test_decode_multi_N256_H32_sampled():
    """gdn_decode_multi at the decode workload's size with 4 tokens per call
    (next_n = 4), sampled units against 4 oracle decode steps."""
    g = _lib()
    w = gi.WORKLOADS[3]
    inp = gi.workload_inputs(3, steps=4)
    tm = {nm: inp[nm].transpose(0, 1).contiguous() for nm in ("q", "k", "v", "log_alpha", "beta")}
    S = inp["S0"].cuda()
    y = g.gdn_decode_multi(*(tm[nm].cuda() for nm in ("q", "k", "v", "log_alpha", "beta")), S)
    torch.cuda.synchronize()
    y, S = y.cpu(), S.cpu()
    for n, h in [(0, 0), (77, 31), (255, 9)]:
        S_or = inp["S0"][n:n + 1, h:h + 1].double().numpy()
        for t in range(4):
            yo, S_or = oracle.decode_step(*(inp[nm][t][n:n + 1, h:h + 1] for nm in
                                            ("q", "k", "v", "log_alpha", "beta")), S_or)
            assert rel_l2(y[n, t, h:h + 1], yo[0]) <= TOL
        assert rel_l2(S[n:n + 1, h:h + 1], S_or) <= TOL
