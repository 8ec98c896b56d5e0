"""The Python binding rejects mis-shaped arguments before any library call.

The C entry points receive pointers and sizes only, so a tensor shorter than
the sizes say would be read or written past its end on the device. The binding
checks every tensor against the sizes it derives, then the devices. These
tests run on the CPU with ``meta`` tensors (shape and dtype, no storage): a
shape mistake must raise GdnError naming the argument, and a correctly shaped
call must get as far as the device check, which meta tensors fail.
"""
import pytest
import torch

import gated_deltanet_amd as g
from gated_deltanet_amd import GdnError

M = dict(device="meta")
bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32


def _t(shape, dtype=bf):
    return torch.empty(shape, dtype=dtype, **M)


def _raises(fn, word):
    with pytest.raises(GdnError) as e:
        fn()
    assert word in str(e.value), str(e.value)


def _prefill(rows=64, H=2, dk=64, dv=64, N=2):
    return dict(q=_t((rows, H, dk)), k=_t((rows, H, dk)), v=_t((rows, H, dv)),
                log_alpha=_t((rows, H), f32), beta=_t((rows, H), f32), N=N)


def test_prefill_shapes():
    a = _prefill()
    _raises(lambda: g.gdn_chunk_fwd(**a), "device")  # well-formed: stops at the device
    for key, bad in (("k", _t((63, 2, 64))), ("k", _t((64, 2, 32))), ("v", _t((64, 3, 64))),
                     ("log_alpha", _t((64, 2, 1), f32)), ("beta", _t((32, 2), f32))):
        b = dict(a)
        b[key] = bad
        _raises(lambda: g.gdn_chunk_fwd(**b), key)
    _raises(lambda: g.gdn_chunk_fwd(**a, S0=_t((2, 2, 64, 32), f32)), "S0")
    _raises(lambda: g.gdn_chunk_fwd(**a, y=_t((64, 2, 32))), "y")
    _raises(lambda: g.gdn_chunk_fwd(**a, y=_t((64, 2, 64), f32)), "y")
    _raises(lambda: g.gdn_chunk_fwd(**a, S_T=_t((1, 2, 64, 64), f32)), "S_T")
    b = dict(a)
    b["N"] = 3
    _raises(lambda: g.gdn_chunk_fwd(**b), "multiple")
    _raises(lambda: g.gdn_chunk_fwd(**a, cu_seqlens=_t((2, 2), i32)), "cu_seqlens")


def test_gated_prefill_and_backward_shapes():
    a = _prefill()
    q, k, v, la, be = a["q"], a["k"], a["v"], a["log_alpha"], a["beta"]
    A = _t((2,), f32)
    _raises(lambda: g.gdn_chunk_fwd_gated(q, k, v, la, be, A, N=2), "device")
    _raises(lambda: g.gdn_chunk_fwd_gated(q, k, v, la, be, _t((3,), f32), N=2), "A")
    _raises(lambda: g.gdn_chunk_fwd_gated(q, k, v, la[:32], be, A, N=2), "a")
    dy = _t((64, 2, 64))
    _raises(lambda: g.gdn_chunk_bwd(q, k, v, la, be, dy, N=2), "device")
    _raises(lambda: g.gdn_chunk_bwd(q, k, v, la, be, dy[:32], N=2), "dy")
    _raises(lambda: g.gdn_chunk_bwd(q, k, v, la, be, dy, N=2, dS_T=_t((2, 2, 64, 8), f32)),
            "dS_T")
    _raises(lambda: g.gdn_chunk_bwd_gated(q, k, v, la, be, A, dy[:, :1], N=2), "dy")
    _raises(lambda: g.gdn_chunk_fwd_segmented(q, k, v, la, be, 2, N=2, y=_t((64, 2, 8))), "y")
    _raises(lambda: g.gdn_chunk_fwd_segmented(q, k, v, la, be, 2, N=2), "device")


def test_decode_shapes():
    N, H, d = 4, 2, 64
    q, k, v = _t((N, H, d)), _t((N, H, d)), _t((N, H, d))
    la, be, S = _t((N, H), f32), _t((N, H), f32), _t((N, H, d, d), f32)
    _raises(lambda: g.gdn_decode_step(q, k, v, la, be, S), "device")
    _raises(lambda: g.gdn_decode_step(q, k[:2], v, la, be, S), "k")
    _raises(lambda: g.gdn_decode_step(q, k, v, la, be[:, :1], S), "beta")
    _raises(lambda: g.gdn_decode_step(q, k, v, la, be, S[:2]), "S")
    _raises(lambda: g.gdn_decode_step(q, k, v, la, be, S, y=_t((N, H, 8))), "y")
    A = _t((H,), f32)
    _raises(lambda: g.gdn_decode_step_gated(q, k, v, la, be, A, S), "device")
    _raises(lambda: g.gdn_decode_step_gated(q, k, v[:, :1], la, be, A, S), "v")
    n_tok = 3
    qm, km, vm = _t((N, n_tok, H, d)), _t((N, n_tok, H, d)), _t((N, n_tok, H, d))
    ga, gb = _t((N, n_tok, H), f32), _t((N, n_tok, H), f32)
    _raises(lambda: g.gdn_decode_multi(qm, km, vm, ga, gb, S), "device")
    _raises(lambda: g.gdn_decode_multi(qm, km, vm, ga[:, :2], gb, S), "g_a")
    _raises(lambda: g.gdn_decode_multi(qm, km, vm[:, :, :, :32], ga, gb, S), "v")
    _raises(lambda: g.gdn_decode_multi(qm, km, vm, ga, gb, S, y=_t((N, n_tok, H, 8))), "y")
    cw, cs, z = _t((3, H * d, 4), f32), _t((N, H, 3, 3, d)), _t((N, n_tok, H, d))
    _raises(lambda: g.gdn_decode_fused(qm, km, vm, cw, cs, ga, gb, S, z), "device")
    _raises(lambda: g.gdn_decode_fused(qm, km, vm, cw[:, :8], cs, ga, gb, S, z), "conv_w")
    _raises(lambda: g.gdn_decode_fused(qm, km, vm, cw, cs, ga, gb, S, z[:1]), "z")
    _raises(lambda: g.gdn_decode_fused(qm, km, vm, cw, cs, ga, gb, S, z,
                                       norm_w=_t((8,), f32)), "norm_w")


def test_frontend_gate_fused_shapes():
    rows, H, d = 64, 2, 64
    qr, kr, vr = _t((rows, H, d)), _t((rows, H, d)), _t((rows, H, d))
    cw = _t((3, H * d, 4), f32)
    _raises(lambda: g.gdn_frontend_qkv(qr, kr, vr, cw), "device")
    _raises(lambda: g.gdn_frontend_qkv(qr, kr[:8], vr, cw), "k_raw")
    _raises(lambda: g.gdn_frontend_qkv(qr, kr, vr, cw, out=(qr, kr, vr[:8])), "v")
    y, z = _t((rows, H, d)), _t((rows, H, d))
    _raises(lambda: g.gdn_output_gate(y, z), "device")
    _raises(lambda: g.gdn_output_gate(y, z, norm_w=_t((d + 1,), f32)), "norm_w")
    _raises(lambda: g.gdn_output_gate(y, z, o=_t((rows, H, 8))), "o")
    la, be = _t((rows, H), f32), _t((rows, H), f32)
    _raises(lambda: g.gdn_chunk_fwd_fused(qr, kr, vr, cw, la, be, z), "device")
    _raises(lambda: g.gdn_chunk_fwd_fused(qr, kr, vr, cw, la[:8], be, z), "log_alpha")
    _raises(lambda: g.gdn_chunk_fwd_fused(qr, kr, vr, cw, la, be, z[:8]), "z")
    _raises(lambda: g.gdn_chunk_fwd_fused(qr, kr, vr, cw, la, be, z,
                                          S_T=_t((1, H, d, 8), f32)), "S_T")
    _raises(lambda: g.gdn_conv_state_from_prefill(qr, kr, vr, N=2,
                                                  conv_state=_t((2, H, 3, 3, 8))), "conv_state")
    _raises(lambda: g.gdn_conv_state_from_prefill(qr, kr, vr, N=2), "device")
