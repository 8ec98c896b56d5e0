"""Seeded synthetic inputs for the Gated DeltaNet token mixer.

This module holds only random-number recipes: it draws the inputs that both
the HIP library and the fp64 oracle consume (the same bits go to both), and
it performs none of the method's arithmetic. Everything is drawn on the CPU
in float32 from ``torch.Generator`` streams, one stream per tensor, seeded
from (seed, tensor id), then cast with round-to-nearest-even where a bf16
tensor is asked for.

Distributions (the five workloads the library is measured on):

* q, k ~ N(0, 1), scaled to unit L2 norm per (token, head) before the cast;
  v ~ N(0, 1);
* per head A_h ~ U(-4, 0); per (token, head) x ~ N(0, 1) and
  log_alpha = -exp(A_h) * softplus(x), beta = sigmoid(N(0, 1)); this is the
  gate parameterisation of the page "NLP——技术报告解读-Qwen3.8-Flash-Next",
  section "GDN 参数化细节", with the projections replaced by random draws;
* raw gate inputs (for the in-kernel gate path): the same a = x and b = n
  draws with the same A_h, plus a per-head bias b_alpha ~ N(0, 0.5);
* states S0 ~ N(0, std) with std the second parameter;
* front-end workload: raw projections ~ N(0, 1) bf16, depthwise conv weights
  ~ N(0, 0.5) float32 [3][H*d][4], z ~ N(0, 1) bf16, sequence lengths drawn
  uniformly from the integers in [512, 8192].
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

# ---------------------------------------------------------------------------
# workload table
# ---------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str  # "prefill" | "decode" | "varlen_fused"
    B: int
    H: int
    T: int
    dk: int
    dv: int
    dtype: str  # "f32" | "bf16" | "f16" for q/k/v
    s0_std: float  # 0.0 => S0 = zeros (passed as NULL)
    steps: int = 0
    n_seqs: int = 0
    len_lo: int = 0
    len_hi: int = 0
    conv_k: int = 4
    conv_std: float = 0.5


WORKLOADS = {
    0: Workload("tiny_fwd_B1_H2_T256_d64_f32", "prefill", 1, 2, 256, 64, 64, "f32", 0.0),
    1: Workload("prefill_B4_H16_T4096_d128_bf16", "prefill", 4, 16, 4096, 128, 128, "bf16", 0.0),
    2: Workload("longctx_prefill_B1_H32_T65536_d128_bf16", "prefill", 1, 32, 65536, 128, 128,
                "bf16", 0.02),
    3: Workload("decode_N256_H32_d128_128steps", "decode", 256, 32, 1, 128, 128, "bf16", 0.02,
                steps=128),
    4: Workload("varlen64_fused_frontend_H16_d128", "varlen_fused", 64, 16, 0, 128, 128, "bf16",
                0.02, n_seqs=64, len_lo=512, len_hi=8192),
}

_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def torch_dtype(name: str) -> torch.dtype:
    return _DT[name]


# ---------------------------------------------------------------------------
# primitive draws
# ---------------------------------------------------------------------------


def _gen(seed: int, tensor_id: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed) * 1000003 + int(tensor_id))
    return g


def normal(shape, seed, tensor_id, std=1.0) -> torch.Tensor:
    x = torch.randn(shape, generator=_gen(seed, tensor_id), dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x


def unit_rows(shape, seed, tensor_id) -> torch.Tensor:
    """N(0,1) draws scaled to unit L2 norm along the last axis."""
    x = normal(shape, seed, tensor_id)
    x.div_(x.norm(dim=-1, keepdim=True))
    return x


def head_log_decay_scale(H, seed, tensor_id=90) -> torch.Tensor:
    """A_h ~ U(-4, 0), one per head."""
    return torch.rand((H,), generator=_gen(seed, tensor_id), dtype=torch.float32) * -4.0


def gates(rows, H, seed, A=None, tid_x=91, tid_b=92):
    """log_alpha = -exp(A_h) softplus(x), beta = sigmoid(n); x, n ~ N(0,1).
    Returns float32 tensors of shape [rows, H]."""
    if A is None:
        A = head_log_decay_scale(H, seed)
    x = normal((rows, H), seed, tid_x)
    log_alpha = -torch.exp(A)[None, :] * torch.nn.functional.softplus(x)
    beta = torch.sigmoid(normal((rows, H), seed, tid_b))
    return log_alpha.contiguous(), beta.contiguous()


def raw_gates(rows, H, seed, bias_std=0.5, tid_x=91, tid_b=92, tid_bias=93):
    """Raw gate pre-activations for the in-kernel gate path: a, b ~ N(0, 1)
    [rows, H] (the same draws as ``gates``), per head A ~ U(-4, 0) and
    b_alpha ~ N(0, bias_std). Returns float32 (a, b, A, b_alpha)."""
    a = normal((rows, H), seed, tid_x)
    b = normal((rows, H), seed, tid_b)
    A = head_log_decay_scale(H, seed)
    b_alpha = normal((H,), seed, tid_bias, std=bias_std)
    return a.contiguous(), b.contiguous(), A, b_alpha


def seq_lengths(n, lo, hi, seed, tensor_id=80) -> torch.Tensor:
    """Integer lengths uniform on [lo, hi]."""
    return torch.randint(lo, hi + 1, (n,), generator=_gen(seed, tensor_id), dtype=torch.int64)


def cu_from_lengths(lengths) -> torch.Tensor:
    lengths = torch.as_tensor(lengths, dtype=torch.int64)
    cu = torch.zeros(lengths.numel() + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(lengths, 0)
    return cu.to(torch.int32)


# ---------------------------------------------------------------------------
# composite workloads
# ---------------------------------------------------------------------------


def prefill_inputs(B, H, T, dk, dv, dtype="bf16", s0_std=0.0, seed=0, lengths=None):
    """Inputs for the chunked prefill.

    Equal-length batch when ``lengths`` is None (total = B*T rows), else a
    packed varlen batch with ``cu_seqlens``. Returns a dict of CPU tensors:
    q, k [tot, H, dk], v [tot, H, dv] in ``dtype``; log_alpha, beta [tot, H]
    float32; S0 [N, H, dk, dv] float32 or None; cu_seqlens int32 or None.
    """
    if lengths is not None:
        cu = cu_from_lengths(lengths)
        N = int(cu.numel() - 1)
        total = int(cu[-1])
    else:
        cu = None
        N = B
        total = B * T
    tdt = _DT[dtype]
    q = unit_rows((total, H, dk), seed, 1).to(tdt)
    k = unit_rows((total, H, dk), seed, 2).to(tdt)
    v = normal((total, H, dv), seed, 3).to(tdt)
    la, b = gates(total, H, seed)
    S0 = normal((N, H, dk, dv), seed, 4, std=s0_std) if s0_std > 0 else None
    return dict(q=q, k=k, v=v, log_alpha=la, beta=b, S0=S0, cu_seqlens=cu, N=N, T=T,
                H=H, dk=dk, dv=dv, dtype=dtype)


def decode_inputs(N, H, dk, dv, steps, dtype="bf16", s0_std=0.02, seed=3):
    """Inputs for ``steps`` consecutive decode steps: q, k [steps, N, H, dk],
    v [steps, N, H, dv] in ``dtype``; log_alpha, beta [steps, N, H] float32
    (A_h fixed across steps); S0 [N, H, dk, dv] float32."""
    tdt = _DT[dtype]
    q = unit_rows((steps, N, H, dk), seed, 11).to(tdt)
    k = unit_rows((steps, N, H, dk), seed, 12).to(tdt)
    v = normal((steps, N, H, dv), seed, 13).to(tdt)
    A = head_log_decay_scale(H, seed)
    la, b = gates(steps * N, H, seed, A=A)
    la = la.reshape(steps, N, H).contiguous()
    b = b.reshape(steps, N, H).contiguous()
    S0 = normal((N, H, dk, dv), seed, 14, std=s0_std)
    return dict(q=q, k=k, v=v, log_alpha=la, beta=b, S0=S0, N=N, H=H, dk=dk, dv=dv,
                steps=steps, dtype=dtype)


def frontend_inputs(lengths, H, dk, dv, dtype="bf16", s0_std=0.02, seed=4, conv_k=4,
                    conv_std=0.5, norm_w_std=0.0):
    """Inputs for the fused front-end prefill on a packed varlen batch: raw
    projections q_raw, k_raw [tot, H, dk], v_raw, z [tot, H, dv] (N(0,1),
    ``dtype``), conv_w float32 [3, H*d, conv_k] (q, k, v weights; requires
    dk == dv), gates float32 [tot, H], S0 float32 [N, H, dk, dv], norm_w
    float32 [dv] (zeros unless norm_w_std > 0)."""
    assert dk == dv, "one conv weight tensor [3][H*d][K] needs dk == dv"
    cu = cu_from_lengths(lengths)
    N = int(cu.numel() - 1)
    total = int(cu[-1])
    tdt = _DT[dtype]
    q_raw = normal((total, H, dk), seed, 21).to(tdt)
    k_raw = normal((total, H, dk), seed, 22).to(tdt)
    v_raw = normal((total, H, dv), seed, 23).to(tdt)
    z = normal((total, H, dv), seed, 24).to(tdt)
    conv_w = normal((3, H * dk, conv_k), seed, 25, std=conv_std)
    la, b = gates(total, H, seed)
    S0 = normal((N, H, dk, dv), seed, 26, std=s0_std) if s0_std > 0 else None
    norm_w = (normal((dv,), seed, 27, std=norm_w_std) if norm_w_std > 0
              else torch.zeros(dv, dtype=torch.float32))
    return dict(q_raw=q_raw, k_raw=k_raw, v_raw=v_raw, z=z, conv_w=conv_w, log_alpha=la,
                beta=b, S0=S0, norm_w=norm_w, cu_seqlens=cu, N=N, H=H, dk=dk, dv=dv,
                dtype=dtype)


def decode_fused_inputs(N, n_tok, H, d, dtype="bf16", s0_std=0.02, seed=5, conv_std=0.5,
                        norm_w_std=0.1):
    """Inputs for the fused serving decode: raw projections q_raw, k_raw,
    v_raw and z [N, n_tok, H, d] (N(0,1), ``dtype``), conv_w float32
    [3, H*d, 4], a convolution cache conv_state [N, H, 3, 3, d] holding three
    earlier raw rows per stream (N(0,1), ``dtype``), gates float32
    [N, n_tok, H], S0 float32 [N, H, d, d] and norm_w float32 [d]."""
    tdt = _DT[dtype]
    q_raw = normal((N, n_tok, H, d), seed, 31).to(tdt)
    k_raw = normal((N, n_tok, H, d), seed, 32).to(tdt)
    v_raw = normal((N, n_tok, H, d), seed, 33).to(tdt)
    z = normal((N, n_tok, H, d), seed, 34).to(tdt)
    conv_w = normal((3, H * d, 4), seed, 35, std=conv_std)
    conv_state = normal((N, H, 3, 3, d), seed, 36).to(tdt)
    la, b = gates(N * n_tok, H, seed)
    S0 = normal((N, H, d, d), seed, 37, std=s0_std)
    norm_w = normal((d,), seed, 38, std=norm_w_std)
    return dict(q_raw=q_raw, k_raw=k_raw, v_raw=v_raw, z=z, conv_w=conv_w,
                conv_state=conv_state, log_alpha=la.reshape(N, n_tok, H).contiguous(),
                beta=b.reshape(N, n_tok, H).contiguous(), S0=S0, norm_w=norm_w, N=N,
                n_tok=n_tok, H=H, d=d, dtype=dtype)


def workload_inputs(wid: int, seed: Optional[int] = None, **kw):
    """Inputs of workload ``wid`` (0..4), seeded by ``seed`` (default: wid)."""
    w = WORKLOADS[wid]
    seed = wid if seed is None else seed
    if w.kind == "prefill":
        return prefill_inputs(w.B, w.H, w.T, w.dk, w.dv, w.dtype, w.s0_std, seed, **kw)
    if w.kind == "decode":
        steps = kw.pop("steps", w.steps)
        N = kw.pop("N", w.B)
        return decode_inputs(N, w.H, w.dk, w.dv, steps, w.dtype, w.s0_std, seed)
    if w.kind == "varlen_fused":
        n = kw.pop("n_seqs", w.n_seqs)
        lengths = kw.pop("lengths", None)
        if lengths is None:
            lengths = seq_lengths(n, w.len_lo, w.len_hi, seed)
        return frontend_inputs(lengths, w.H, w.dk, w.dv, w.dtype, w.s0_std, seed,
                               w.conv_k, w.conv_std, **kw)
    raise ValueError(w.kind)
