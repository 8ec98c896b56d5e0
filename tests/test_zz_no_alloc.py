"""gdn_chunk_fwd_segmented_noalloc (the segment-parallel prefill with the
library's fixed per-GPU scratch as its workspace) against
gdn_chunk_fwd_segmented with a caller workspace, called through the C ABI:
two calls in a row on one GPU, the second on a smaller problem, each equal to
the workspace entry point bit for bit (same kernels, same operands), plus the
rejection of a problem too large for the fixed scratch."""
import ctypes

import pytest
import torch

import gdn_inputs as gi

gpu = pytest.mark.gpu


def _lib():
    import gated_deltanet_amd as g
    return g, g.load_library()


def _call_both(g, lib, inp, N, P, S0):
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    q, k, v, la, b = (dev[n] for n in ("q", "k", "v", "log_alpha", "beta"))
    rows, H, dk = q.shape
    dv = v.shape[-1]
    s0 = dev["S0"] if S0 else None
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    y_ref = torch.empty_like(v)
    st_ref = torch.empty((N, H, dk, dv), dtype=torch.float32, device="cuda")
    need = lib.gdn_chunk_fwd_segmented_workspace_size(rows, N, H, dk, dv, P, 1)
    assert 0 < need <= g.NOALLOC_SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    rc = lib.gdn_chunk_fwd_segmented(p(q), p(k), p(v), p(la), p(b), p(s0), p(y_ref), p(st_ref),
                                     None, N, rows // N, H, dk, dv, P, p(ws), need, 1, 1, stream)
    assert rc == 0, lib.gdn_last_error()
    y = torch.full_like(v, float("nan"))
    st = torch.full((N, H, dk, dv), float("nan"), dtype=torch.float32, device="cuda")
    rc = lib.gdn_chunk_fwd_segmented_noalloc(p(q), p(k), p(v), p(la), p(b), p(s0), p(y), p(st),
                                             None, N, rows // N, H, dk, dv, P, 1, 1, stream)
    assert rc == 0, lib.gdn_last_error()
    torch.cuda.synchronize()
    return y, st, y_ref, st_ref


@gpu
def test_noalloc_segmented_equals_workspace_entry_twice():
    g, lib = _lib()
    # first call: 3 sequences x 4 heads, 700 tokens, d = 128, 4 segments, S0
    big = gi.prefill_inputs(3, 4, 700, 128, 128, "bf16", s0_std=0.02, seed=91)
    y, st, y_ref, st_ref = _call_both(g, lib, big, N=3, P=4, S0=True)
    assert torch.equal(y, y_ref) and torch.equal(st, st_ref)
    # second call, smaller: 1 sequence x 2 heads, 200 tokens, d = 64, 2 segments
    small = gi.prefill_inputs(1, 2, 200, 64, 64, "bf16", s0_std=0.0, seed=92)
    y, st, y_ref, st_ref = _call_both(g, lib, small, N=1, P=2, S0=False)
    assert torch.equal(y, y_ref) and torch.equal(st, st_ref)
    assert not torch.isnan(y).any()


@gpu
def test_noalloc_rejects_more_than_its_scratch():
    g, lib = _lib()
    # 16 sequences x 32 heads x 4 segments at d = 128 need 16 * 32 * 8 states of
    # 64 KiB = 256 MiB of workspace, more than the fixed scratch
    assert lib.gdn_chunk_fwd_segmented_workspace_size(16 * 64, 16, 32, 128, 128, 4, 1) > \
        g.NOALLOC_SCRATCH_BYTES
    t = torch.zeros(16 * 64 * 32 * 128, dtype=torch.bfloat16, device="cuda")
    gate = torch.zeros(16 * 64 * 32, dtype=torch.float32, device="cuda")
    y = torch.empty_like(t)
    p = lambda x: ctypes.c_void_p(x.data_ptr())
    rc = lib.gdn_chunk_fwd_segmented_noalloc(p(t), p(t), p(t), p(gate), p(gate), None, p(y), None,
                                             None, 16, 64, 32, 128, 128, 4, 1, 1, None)
    assert rc == -1 and b"scratch" in lib.gdn_last_error()
