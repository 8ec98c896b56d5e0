#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one gdn_chunk_fwd call (in-chunk gate cumsum, UT inverse, state
scan and intra-chunk products) over the chunked-prefill workload
B=4, H=16, T=4096, dk=dv=128, bf16 q/k/v, fp32 gates and state, S0 = 0,
32-token chunks. `value` is prefill tokens/s (B*T per step). The same line
also carries the decode-step workload (256 sequences x 32 heads x 128x128
fp32 states, 128 consecutive steps) as state GB/s against the HBM peak,
the roofline of the prefill kernel, and the fp64 CPU oracle timed on the
host cores on the same prefill batch.

Inputs are synthetic (seeded, generated on the CPU, resident in HBM before
timing starts). Timing uses HIP events on the stream the kernels run on.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import gdn_inputs as gi  # noqa: E402

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 matrix peak, AMD's published figure
ALG_CHUNK = 64  # chunk size the algorithmic flop count is defined at, whatever the kernel uses
KERNEL_CHUNK = 32  # tokens per chunk inside the 16-bit prefill kernel


def prefill_flops_per_token_head(dk, dv, C=ALG_CHUNK):
    """Algorithmic work of chunked prefill per token per head (triangles
    halved): 6 dk dv + C (3 dk + 2 dv) + C^2 / 3, counted at C = 64 so the
    figure does not depend on the kernel's own chunk size (140 629 at
    dk = dv = 128)."""
    return 6 * dk * dv + C * (3 * dk + 2 * dv) + C * C / 3.0


def prefill_bytes(tokens, H, dk, dv, N, in_b=2, out_b=2, s0=False):
    """Algorithmic HBM bytes: q, k, v read, y written, gates read, state
    written (and read when S0 is given)."""
    per_tok_head = (2 * dk + dv) * in_b + dv * out_b + 8
    state = N * H * dk * dv * 4
    return tokens * H * per_tok_head + state * (2 if s0 else 1)


def decode_bytes_per_step(N, H, dk, dv, in_b=2, out_b=2):
    return N * H * (2 * dk * dv * 4 + (2 * dk + dv) * in_b + dv * out_b + 8)


def measured_traffic(key, source):
    """HBM bytes per dispatch measured with rocprofv3 counters (profiles/),
    or None when the kernel source changed since they were taken."""
    import hashlib
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", "traffic_per_dispatch.json")))[key]
        src = open(os.path.join(ROOT, "gated_deltanet_amd", "csrc", source), "rb").read()
    except (OSError, KeyError, ValueError):
        return None
    if hashlib.sha256(src).hexdigest()[:16] != rec.get("source_sha256_16"):
        return None
    return rec["bytes"]


def measured_mfma(key, source):
    """MFMA counters per dispatch from rocprofv3 (profiles/): busy fraction
    and issued flops, or None when the kernel source changed since."""
    import hashlib
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", "mfma_per_dispatch.json")))[key]
        src = open(os.path.join(ROOT, "gated_deltanet_amd", "csrc", source), "rb").read()
    except (OSError, KeyError, ValueError):
        return None
    if hashlib.sha256(src).hexdigest()[:16] != rec.get("source_sha256_16"):
        return None
    return dict(mfma_busy=rec["mfma_busy"], issued_flops=rec["issued_flops"])


def fused_traffic():
    """HBM bytes of the varlen fused call: its three kernels' counters, or
    None unless all three are current."""
    parts = [measured_traffic("frontend_kernel_varlen64_H16_d128", "frontend.hip"),
             measured_traffic("chunk_fwd_bf16_kernel_varlen64_H16_d128", "chunk_fwd.hip"),
             measured_traffic("output_gate_kernel_varlen64_H16_d128", "frontend.hip")]
    return None if any(x is None for x in parts) else sum(parts)


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def row_errors(got, ref, block=32, floor_frac=0.05):
    """Worst per-row relative error over the rows of [rows, d] (each row's
    error over max(its norm, floor_frac x the RMS row norm), so near-zero rows
    do not divide by ~0) and worst rel-L2 over blocks of `block` rows."""
    got = np.asarray(got, dtype=np.float64).reshape(len(got), -1)
    ref = np.asarray(ref, dtype=np.float64).reshape(len(ref), -1)
    err = np.linalg.norm(got - ref, axis=1)
    nrm = np.linalg.norm(ref, axis=1)
    floor = floor_frac * float(np.sqrt(np.mean(nrm ** 2))) if len(nrm) else 0.0
    row = float(np.max(err / np.maximum(nrm, max(floor, 1e-300)))) if len(nrm) else 0.0
    worst = 0.0
    for s0 in range(0, len(ref), block):
        worst = max(worst, rel_l2(got[s0:s0 + block], ref[s0:s0 + block]))
    return row, worst


def _roofline(kernel, nbytes, flops, ms, traffic=None):
    """HBM roofline record of one call from its algorithmic bytes and flops;
    traffic: HBM bytes per call from rocprofv3 counters, or None."""
    gbs = nbytes / (ms * 1e-3) / 1e9
    tf = flops / (ms * 1e-3) / 1e12
    return dict(kernel=kernel, bound="hbm", achieved=gbs, peak=HBM_PEAK_GBS, unit="GB/s",
                frac=gbs / HBM_PEAK_GBS, traffic=traffic, alg_bytes_per_launch=nbytes,
                alg_flops_per_launch=flops, mfma_tflops=tf, mfma_frac_bf16_peak=tf / BF16_PEAK_TFLOPS)


WARM_SECONDS = 0.5


def time_launches(fn, steps, warmup, stream):
    """Events around `steps` back-to-back calls of fn on `stream`, after
    `warmup` untimed calls and, beyond those, untimed calls until the GPU
    has been busy for WARM_SECONDS (its clocks ramp up over the first few
    hundred milliseconds of load)."""
    t0 = time.perf_counter()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < WARM_SECONDS:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end)  # ms


def prefill_kernel_name(g, N, H, dk, dv):
    """The prefill kernel instance the library launches for this bf16 shape
    (its state waves per workgroup = columns / 16)."""
    ns = g.gdn_prefill_state_columns(N, H, dk, dv, torch.bfloat16) // 16
    return "chunk_fwd_bf16_kernel<%d,%d,bf16,bf16>" % (dk, ns)


def bench_prefill(g, steps, warmup, copies=3):
    w = gi.WORKLOADS[1]
    inp = gi.workload_inputs(1)
    N, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    tokens = N * T
    dev = torch.device("cuda", 0)
    # several copies of the inputs so consecutive steps do not hit the
    # 256 MB last-level cache with the previous step's data
    sets = []
    for _ in range(copies):
        sets.append({k: inp[k].to(dev) for k in ("q", "k", "v", "log_alpha", "beta")})
    y = torch.empty((tokens, H, dv), dtype=torch.bfloat16, device=dev)
    S_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    it = [0]

    def step():
        d = sets[it[0] % copies]
        it[0] += 1
        g.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], None, y=y, S_T=S_T, N=N)

    ms = time_launches(step, steps, warmup, stream)
    ms_step = ms / steps
    # one extra call on the first copy for the parity check
    d = sets[0]
    g.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], None, y=y, S_T=S_T, N=N)
    torch.cuda.synchronize()
    return dict(inp=inp, ms_step=ms_step, tokens=tokens, N=N, H=H, T=T, dk=dk, dv=dv,
                y=y.float().cpu(), S_T=S_T.cpu())


def bench_prefill_gated(g, steps, warmup, copies=3):
    """The prefill workload through gdn_chunk_fwd_gated: raw gate
    pre-activations (a, b, A, b_alpha) turned into gates inside the kernel."""
    w = gi.WORKLOADS[1]
    inp = gi.workload_inputs(1)
    N, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    tokens = N * T
    dev = torch.device("cuda", 0)
    a, b, A, b_alpha = gi.raw_gates(tokens, H, seed=11)
    sets = []
    for _ in range(copies):
        d = {k: inp[k].to(dev) for k in ("q", "k", "v")}
        d.update(a=a.to(dev), b=b.to(dev))
        sets.append(d)
    A, b_alpha = A.to(dev), b_alpha.to(dev)
    y = torch.empty((tokens, H, dv), dtype=torch.bfloat16, device=dev)
    S_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    it = [0]

    def step():
        d = sets[it[0] % copies]
        it[0] += 1
        g.gdn_chunk_fwd_gated(d["q"], d["k"], d["v"], d["a"], d["b"], A, b_alpha, None, y=y,
                              S_T=S_T, N=N)

    ms = time_launches(step, steps, warmup, stream) / steps
    return dict(workload=w.name, entry_point="gdn_chunk_fwd_gated", ms_per_call=ms,
                tokens_per_s=tokens / (ms * 1e-3))


def bench_backward(g, steps=5, warmup=1):
    """gdn_chunk_bwd on the prefill workload (B=4 H=16 T=4096 d=128, bf16
    q/k/v, bf16 dy and gradients, no S0, no dS_T): one call runs the prefill
    kernel for the chunk-start states, the reverse sweep and the tile
    reduction."""
    w = gi.WORKLOADS[1]
    inp = gi.workload_inputs(1)
    N, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    tokens = N * T
    dev = torch.device("cuda", 0)
    d = {k: inp[k].to(dev) for k in ("q", "k", "v", "log_alpha", "beta")}
    dy = gi.normal((tokens, H, dv), 13, 40).to(torch.bfloat16).to(dev)
    ws = torch.empty(g.gdn_chunk_bwd_workspace_size(tokens, N, H, dk, dv, torch.bfloat16),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        g.gdn_chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], dy, N=N, workspace=ws,
                        want_dS0=False)

    ms = time_launches(step, steps, warmup, stream) / steps
    return dict(workload=w.name, entry_point="gdn_chunk_bwd", ms_per_call=ms,
                tokens_per_s=tokens / (ms * 1e-3), workspace_MB=ws.numel() / 1e6)


def bench_decode(g, n_steps=128, reps=2):
    w = gi.WORKLOADS[3]
    N, H, dk, dv = w.B, w.H, w.dk, w.dv
    dev = torch.device("cuda", 0)
    inp = gi.workload_inputs(3, steps=n_steps)
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    la, b = inp["log_alpha"].to(dev), inp["beta"].to(dev)
    S = inp["S0"].to(dev)
    y = torch.empty((n_steps, N, H, dv), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def one_pass():
        for t in range(n_steps):
            g.gdn_decode_step(q[t], k[t], v[t], la[t], b[t], S, y=y[t])

    one_pass()  # warm-up (advances the state; the timing does not depend on values)
    torch.cuda.synchronize()
    ms = time_launches(one_pass, reps, 0, stream)
    us_step = ms * 1e3 / (reps * n_steps)
    bytes_step = decode_bytes_per_step(N, H, dk, dv)
    gbs = bytes_step / (us_step * 1e-6) / 1e9
    # one more pass from the initial states, whose outputs the oracle checks
    # on sampled (sequence, head) units over all n_steps steps
    S.copy_(inp["S0"].to(dev))
    one_pass()
    torch.cuda.synchronize()
    units = [(0, 0), (255, 31), (17, 5), (128, 16), (200, 2)]
    check = dict(inp=inp, units=units, y={u: y[:, u[0], u[1]].float().cpu() for u in units},
                 S={u: S[u[0], u[1]].cpu() for u in units})
    return dict(_check=check, workload=w.name, us_per_step=us_step, GBps=gbs,
                frac_hbm=gbs / HBM_PEAK_GBS,
                tokens_per_s=N / (us_step * 1e-6), bytes_per_step=bytes_step, steps=n_steps,
                roofline=dict(kernel="decode_token_kernel<128,128,bf16,bf16,unfused> (n_tok = 1)",
                              bound="hbm", achieved=gbs, peak=HBM_PEAK_GBS, unit="GB/s",
                              frac=gbs / HBM_PEAK_GBS,
                              traffic=measured_traffic("decode_token_kernel_N256_H32_d128",
                                                       "decode.hip")))


def bench_decode_multi(g, n_tok=4, calls=32):
    """The decode workload (256 sequences x 32 heads, 128x128 states) with
    n_tok tokens per sequence in each call (a speculative verify step of
    next_n = 4); the state is read and written once per call."""
    w = gi.WORKLOADS[3]
    N, H, dk, dv = w.B, w.H, w.dk, w.dv
    dev = torch.device("cuda", 0)
    inp = gi.workload_inputs(3, steps=n_tok)
    tm = {nm: inp[nm].transpose(0, 1).contiguous().to(dev)
          for nm in ("q", "k", "v", "log_alpha", "beta")}
    S = inp["S0"].to(dev)
    y = torch.empty((N, n_tok, H, dv), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def call():
        g.gdn_decode_multi(tm["q"], tm["k"], tm["v"], tm["log_alpha"], tm["beta"], S, y=y)

    us = time_launches(call, calls, 2, stream) * 1e3 / calls
    nbytes = N * H * (2 * dk * dv * 4 + n_tok * ((2 * dk + 2 * dv) * 2 + 8))
    gbs = nbytes / (us * 1e-6) / 1e9
    return dict(workload=w.name, entry_point="gdn_decode_multi", n_tok=n_tok, us_per_call=us,
                tokens_per_s=N * n_tok / (us * 1e-6), GBps=gbs, frac_hbm=gbs / HBM_PEAK_GBS,
                bytes_per_call=nbytes,
                roofline=dict(kernel="decode_block_kernel<128,128,bf16,bf16,unfused> (n_tok = %d)"
                              % n_tok, bound="hbm", achieved=gbs, peak=HBM_PEAK_GBS, unit="GB/s",
                              frac=gbs / HBM_PEAK_GBS,
                              traffic=measured_traffic("decode_block_kernel_N256_H32_d128_ntok4",
                                                       "decode.hip") if n_tok == 4 else None))


def bench_decode_fused(g, n_tok=4, calls=32):
    """The decode workload through gdn_decode_fused: front end with the
    convolution cache, n_tok recurrence steps and the output gate in one
    kernel, from raw projections to o."""
    w = gi.WORKLOADS[3]
    N, H, d = w.B, w.H, w.dk
    dev = torch.device("cuda", 0)
    f = gi.decode_fused_inputs(N, n_tok, H, d, "bf16", seed=12)
    t = {k: v.to(dev) for k, v in f.items() if isinstance(v, torch.Tensor)}
    o = torch.empty((N, n_tok, H, d), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def call():
        g.gdn_decode_fused(t["q_raw"], t["k_raw"], t["v_raw"], t["conv_w"], t["conv_state"],
                           t["log_alpha"], t["beta"], t["S0"], t["z"], norm_w=t["norm_w"], o=o)

    us = time_launches(call, calls, 2, stream) * 1e3 / calls
    nbytes = N * H * (2 * d * d * 4 + 2 * 9 * d * 2 + n_tok * (5 * d * 2 + 8))
    gbs = nbytes / (us * 1e-6) / 1e9
    return dict(workload=w.name, entry_point="gdn_decode_fused", n_tok=n_tok, us_per_call=us,
                tokens_per_s=N * n_tok / (us * 1e-6), GBps=gbs, frac_hbm=gbs / HBM_PEAK_GBS,
                bytes_per_call=nbytes)


def bench_longctx(g, steps=3, warmup=1):
    """B=1, H=32, T=65536 prefill from a nonzero S0 (fp32 state)."""
    w = gi.WORKLOADS[2]
    inp = gi.workload_inputs(2)
    dev = torch.device("cuda", 0)
    d = {k: inp[k].to(dev) for k in ("q", "k", "v", "log_alpha", "beta", "S0")}
    y = torch.empty(d["v"].shape, dtype=torch.bfloat16, device=dev)
    S_T = torch.empty_like(d["S0"])
    stream = torch.cuda.current_stream(dev)

    def step():
        g.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"], y=y, S_T=S_T)

    ms = time_launches(step, steps, warmup, stream) / steps
    tokens = w.B * w.T
    flops = tokens * w.H * prefill_flops_per_token_head(w.dk, w.dv)
    nbytes = prefill_bytes(tokens, w.H, w.dk, w.dv, w.B, s0=True)
    return dict(workload=w.name, ms_per_call=ms, tokens_per_s=tokens / (ms * 1e-3),
                pct_bf16_mfma_peak=100.0 * flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                hbm_GBps=nbytes / (ms * 1e-3) / 1e9,
                roofline=_roofline(prefill_kernel_name(g, w.B, w.H, w.dk, w.dv), nbytes,
                                   flops, ms,
                                   measured_traffic("chunk_fwd_bf16_kernel_B1_H32_T65536_d128",
                                                    "chunk_fwd.hip")))


def bench_longctx_segmented(g, segment_counts=(2, 4, 9), steps=3, warmup=1):
    """The long-context workload through gdn_chunk_fwd_segmented (each
    sequence cut into P pieces whose state summaries are chained), per P."""
    w = gi.WORKLOADS[2]
    inp = gi.workload_inputs(2)
    dev = torch.device("cuda", 0)
    d = {k: inp[k].to(dev) for k in ("q", "k", "v", "log_alpha", "beta", "S0")}
    y = torch.empty(d["v"].shape, dtype=torch.bfloat16, device=dev)
    S_T = torch.empty_like(d["S0"])
    stream = torch.cuda.current_stream(dev)
    rows = w.B * w.T
    out = dict(workload=w.name, entry_point="gdn_chunk_fwd_segmented", ms_per_call={})
    for P in segment_counts:
        ws = torch.empty(g.gdn_chunk_fwd_segmented_workspace_size(rows, w.B, w.H, w.dk, w.dv, P,
                                                                  torch.bfloat16),
                         dtype=torch.uint8, device=dev)

        def step():
            g.gdn_chunk_fwd_segmented(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], P,
                                      d["S0"], y=y, S_T=S_T, workspace=ws)

        out["ms_per_call"][str(P)] = time_launches(step, steps, warmup, stream) / steps
        del ws
    return out


def bench_varlen_frontend(g, steps=3, warmup=1):
    """64 packed sequences (lengths U[512, 8192]), H=16, d=128 through
    gdn_chunk_fwd_fused: front end -> chunked prefill -> output gate (q/k/v
    and y in fp16 between the stages, in a preallocated workspace)."""
    w = gi.WORKLOADS[4]
    f = gi.workload_inputs(4)
    dev = torch.device("cuda", 0)
    d = {k: v.to(dev) for k, v in f.items() if isinstance(v, torch.Tensor)}
    rows = int(f["cu_seqlens"][-1])
    shape = d["q_raw"].shape
    S_T = torch.empty_like(d["S0"])
    o = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(g.gdn_fused_workspace_size(rows, w.H, w.dk), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        g.gdn_chunk_fwd_fused(d["q_raw"], d["k_raw"], d["v_raw"], d["conv_w"], d["log_alpha"],
                              d["beta"], d["z"], S0=d["S0"], norm_w=d["norm_w"],
                              cu_seqlens=d["cu_seqlens"], out_dtype=torch.bfloat16, o=o,
                              S_T=S_T, workspace=ws)

    ms = time_launches(step, steps, warmup, stream) / steps
    flops = rows * w.H * prefill_flops_per_token_head(w.dk, w.dv)
    # raw q, k, v and z read, o written, gates read, S0 read and S_T written
    fused_bytes = rows * w.H * (3 * 128 * 2 + 128 * 2 + 128 * 2 + 8) + 2 * w.n_seqs * w.H * 128 * 128 * 4
    # outputs of the last timed call on sampled units: the longest and the
    # shortest sequence and four more, one head each, for the oracle chain
    cu = f["cu_seqlens"]
    lens = (cu[1:] - cu[:-1]).tolist()
    order = sorted(range(len(lens)), key=lambda n: lens[n])
    picks = [order[-1], order[0], order[len(order) // 2], 7, 31, 50]
    units = [(n, (5 * i + 3) % w.H) for i, n in enumerate(picks)]
    torch.cuda.synchronize()
    check = dict(f=f, units=units,
                 o={u: o[int(cu[u[0]]):int(cu[u[0] + 1]), u[1]].float().cpu() for u in units},
                 S={u: S_T[u[0], u[1]].cpu() for u in units})
    return dict(_check=check, workload=w.name, tokens=rows, ms_per_call=ms,
                tokens_per_s=rows / (ms * 1e-3),
                pct_bf16_mfma_peak=100.0 * flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                hbm_GBps_of_fused_bytes=fused_bytes / (ms * 1e-3) / 1e9,
                roofline=_roofline("gdn_chunk_fwd_fused (whole call)", fused_bytes, flops, ms,
                                   fused_traffic()),
                entry_point="gdn_chunk_fwd_fused")


def cpu_baseline(pf, max_seconds=30.0, min_seconds=10.0):
    """The fp64 oracle on the host cores, on the same prefill batch: every
    head of as many whole sequences as fit the time budget (starting with
    one); when the whole batch takes less than min_seconds, further passes
    over it are timed too, so the rate averages over at least that long.
    Returns the record and the first pass's oracle outputs for the parity
    check."""
    import oracle
    inp = pf["inp"]
    H, T, N = pf["H"], pf["T"], pf["N"]
    threads = len(os.sched_getaffinity(0))
    done = 0  # sequences run, over all passes
    spent = 0.0
    outs = []
    while True:
        n = done % N
        rows = slice(n * T, (n + 1) * T)
        t0 = time.perf_counter()
        y, S = oracle.gdn_fwd(inp["q"][rows], inp["k"][rows], inp["v"][rows],
                              inp["log_alpha"][rows], inp["beta"][rows], None, N=1,
                              nthreads=threads)
        spent += time.perf_counter() - t0
        if done < N:
            outs.append((n, y, S))
        done += 1
        if spent * (done + 1) / done > max_seconds:
            break
        if done >= N and done % N == 0 and spent >= min_seconds:
            break
    tok_s = done * T / spent
    if done <= N:
        what = "%d of %d sequences" % (done, N)
    else:
        what = "all %d sequences, %d passes (%d sequence runs)" % (N, (done + N - 1) // N, done)
    rec = dict(value=tok_s, unit="tokens/s", cores=threads, kind="oracle",
               sample="%s (all %d heads, %d tokens each), fp64 token recurrence, %.1f s"
                      % (what, H, T, spent))
    return rec, outs


def decode_parity(chk):
    """All decode steps of sampled (sequence, head) units against the oracle's
    decode step applied the same number of times from the same state."""
    import oracle
    inp = chk["inp"]
    ey, es, er = [], [], []
    steps = inp["q"].shape[0]
    for n, h in chk["units"]:
        S = inp["S0"][n:n + 1, h:h + 1].double().numpy()
        yo = []
        for t in range(steps):
            args = [inp[key][t, n:n + 1, h:h + 1] for key in ("q", "k", "v", "log_alpha", "beta")]
            yt, S = oracle.decode_step(*args, S)
            yo.append(yt[0, 0])
        yo = np.stack(yo)
        got = chk["y"][(n, h)].numpy()
        ey.append(rel_l2(got, yo))
        er.append(row_errors(got, yo)[0])
        es.append(rel_l2(chk["S"][(n, h)].numpy(), S[0, 0]))
    return dict(units=len(chk["units"]), steps=steps, y_rel_l2=max(ey), S_rel_l2=max(es),
                y_row_rel_max=max(er))


def varlen_parity(chk):
    """Sampled (sequence, head) units of the fused varlen call against the
    oracle chain: front end, token recurrence from S0, output gate."""
    import oracle
    f = chk["f"]
    cu, w, H, d = f["cu_seqlens"], f["conv_w"], f["H"], f["dk"]
    eo, es, er, eb = [], [], [], []
    for n, h in chk["units"]:
        s0, e0 = int(cu[n]), int(cu[n + 1])
        sl = lambda x: x[s0:e0, h:h + 1]
        wsl = lambda i: w[i].reshape(H, d, -1)[h]
        q = oracle.frontend(sl(f["q_raw"]), wsl(0), l2=True, eps=1e-6)
        k = oracle.frontend(sl(f["k_raw"]), wsl(1), l2=True, eps=1e-6)
        v = oracle.frontend(sl(f["v_raw"]), wsl(2), l2=False)
        y, S = oracle.gdn_fwd(q, k, v, sl(f["log_alpha"]), sl(f["beta"]),
                              f["S0"][n:n + 1, h:h + 1], col_blocks=8)
        oo = oracle.output_gate(y, sl(f["z"]), f["norm_w"], eps=1e-6)[:, 0]
        got = chk["o"][(n, h)].numpy()
        eo.append(rel_l2(got, oo))
        r, b = row_errors(got, oo)
        er.append(r)
        eb.append(b)
        es.append(rel_l2(chk["S"][(n, h)].numpy(), S[0, 0]))
    lens = [int(cu[n + 1] - cu[n]) for n, _ in chk["units"]]
    return dict(units=len(chk["units"]), lengths=lens, o_rel_l2=max(eo), S_T_rel_l2=max(es),
                o_row_rel_max=max(er), o_chunk_rel_l2_max=max(eb))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--decode-steps", type=int, default=128)
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the long-context and varlen front-end workloads")
    ap.add_argument("--no-serving", action="store_true",
                    help="skip the multi-token and fused serving decode workloads")
    ap.add_argument("--warm-seconds", type=float, default=0.5,
                    help="untimed GPU load before each timed region, beyond --warmup steps")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run one plain 1 GiB device copy (torch copy_), the known-size "
                         "reference for scaling HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only (--gpus %d given): the GDN mixer shards over "
              "(sequence, head) with no exchange, and a multi-GPU run is not provided." % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    global WARM_SECONDS
    WARM_SECONDS = max(0.0, args.warm_seconds)
    import gated_deltanet_amd as g
    g.load_library()
    torch.cuda.set_device(0)

    if args.calibrate_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1.0)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print("[bench] calibration copy: %d bytes read, %d bytes written" %
              (src.numel() * 4, dst.numel() * 4), file=sys.stderr, flush=True)
        del src, dst

    print("[bench] prefill workload 1: B=4 H=16 T=4096 d=128 bf16", file=sys.stderr, flush=True)
    pf = bench_prefill(g, args.steps, args.warmup)
    ms = pf["ms_step"]
    tokens, H, dk, dv, N = pf["tokens"], pf["H"], pf["dk"], pf["dv"], pf["N"]
    value = tokens / (ms * 1e-3)
    flops = tokens * H * prefill_flops_per_token_head(dk, dv)
    nbytes = prefill_bytes(tokens, H, dk, dv, N)
    achieved_gbs = nbytes / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    traffic = measured_traffic("chunk_fwd_bf16_kernel_B4_H16_T4096_d128", "chunk_fwd.hip")
    mfma = measured_mfma("chunk_fwd_bf16_kernel_B4_H16_T4096_d128", "chunk_fwd.hip")
    roofline = dict(kernel=prefill_kernel_name(g, N, H, dk, dv), bound="hbm",
                    achieved=achieved_gbs, peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=achieved_gbs / HBM_PEAK_GBS, traffic=traffic,
                    alg_bytes_per_launch=nbytes, alg_flops_per_launch=flops,
                    mfma_tflops=tflops, mfma_frac_bf16_peak=tflops / BF16_PEAK_TFLOPS,
                    mfma_busy=None if mfma is None else mfma["mfma_busy"],
                    mfma_issued_flops_per_launch=None if mfma is None else mfma["issued_flops"])

    rec = dict(metric="GDN prefill tokens/s (% bf16 MFMA peak); decode state GB/s (% HBM peak)",
               value=value, unit="tokens/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
               ms_per_step=ms, higher_is_better=True, scaling="weak", vs_baseline=None,
               dtype="bf16", data="synthetic",
               config=dict(workload=gi.WORKLOADS[1].name, B=N, H=H, T=pf["T"], dk=dk, dv=dv,
                           flop_count_chunk=ALG_CHUNK, kernel_chunk=KERNEL_CHUNK, q_k_v="bf16",
                           y="bf16", state="fp32", S0="zeros"),
               pct_bf16_mfma_peak=100.0 * tflops / BF16_PEAK_TFLOPS,
               roofline=roofline)

    if not args.no_decode:
        print("[bench] decode workload 3: 256 x 32 heads, %d steps" % args.decode_steps,
              file=sys.stderr, flush=True)
        rec["decode"] = bench_decode(g, args.decode_steps)
    if not args.no_decode and not args.no_serving:
        print("[bench] decode workload 3 with 4 tokens per call", file=sys.stderr, flush=True)
        rec["decode_multi"] = bench_decode_multi(g)
        print("[bench] fused serving decode, 4 tokens per call", file=sys.stderr, flush=True)
        rec["decode_fused"] = bench_decode_fused(g)

    if not args.no_extra:
        print("[bench] prefill workload 1 with raw gates", file=sys.stderr, flush=True)
        rec["prefill_gated"] = bench_prefill_gated(g, args.steps, args.warmup)
        rec["prefill_gated"]["ms_vs_plain"] = rec["prefill_gated"]["ms_per_call"] / ms
        print("[bench] backward on prefill workload 1", file=sys.stderr, flush=True)
        rec["backward"] = bench_backward(g)
        rec["backward"]["ms_vs_forward"] = rec["backward"]["ms_per_call"] / ms
        print("[bench] long-context prefill workload 2: B=1 H=32 T=65536", file=sys.stderr,
              flush=True)
        rec["longctx"] = bench_longctx(g)
        print("[bench] long-context prefill, segment-parallel form", file=sys.stderr, flush=True)
        rec["longctx_segmented"] = bench_longctx_segmented(g)
        rec["longctx_segmented"]["ms_vs_serial"] = {
            P: t / rec["longctx"]["ms_per_call"]
            for P, t in rec["longctx_segmented"]["ms_per_call"].items()}
        print("[bench] varlen front-end workload 4: 64 sequences, H=16", file=sys.stderr,
              flush=True)
        rec["varlen_frontend"] = bench_varlen_frontend(g)

    checks = {key: rec[key].pop("_check") for key in ("decode", "varlen_frontend")
              if key in rec and "_check" in rec[key]}
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cb, outs = cpu_baseline(pf)
        rec["cpu_baseline"] = cb
        ey, es, er, eb = [], [], [], []
        T = pf["T"]
        for n, yo, So in outs:
            got = pf["y"][n * T:(n + 1) * T].numpy()
            ey.append(rel_l2(got, yo))
            es.append(rel_l2(pf["S_T"][n].numpy(), So[0]))
            for h in range(H):
                r, b = row_errors(got[:, h], yo[:, h])
                er.append(r)
                eb.append(b)
        rec["parity"] = dict(y_rel_l2=max(ey), S_T_rel_l2=max(es), y_row_rel_max=max(er),
                             y_chunk_rel_l2_max=max(eb), sequences=len(outs), tolerance=2e-3,
                             row_tolerance=1e-2)
        print("[bench] parity of the timed decode and varlen workloads", file=sys.stderr,
              flush=True)
        if "decode" in checks:
            rec["parity"]["decode"] = decode_parity(checks["decode"])
        if "varlen_frontend" in checks:
            rec["parity"]["varlen_frontend"] = varlen_parity(checks["varlen_frontend"])
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
