"""Python binding of libgdn, the Gated DeltaNet token mixer for MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libgdn.so`` (built in-tree by ``gated_deltanet_amd.build``).
PyTorch supplies device memory and the current stream. There is no fallback:
if the library is missing or the GPU is absent, calls raise.

Functions carry the names of the C entry points declared in include/gdn.h:

* ``gdn_chunk_fwd(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None,
  out_dtype=None, S_T=None, y=None)`` -> (y, S_T)
* ``gdn_decode_step(q, k, v, log_alpha, beta, S, out_dtype=None, y=None)`` -> y
* ``gdn_frontend_qkv(q_raw, k_raw, v_raw, conv_w, cu_seqlens=None, N=None,
  l2_eps=1e-6, out_dtype=None)`` -> (q, k, v)
* ``gdn_output_gate(y, z, norm_w=None, rms_eps=1e-6, out_dtype=None)`` -> o
* ``gdn_chunk_fwd_fused(q_raw, k_raw, v_raw, conv_w, log_alpha, beta, z,
  S0=None, norm_w=None, l2_eps=1e-6, rms_eps=1e-6, cu_seqlens=None, N=None,
  out_dtype=None)`` -> (o, S_T)
* ``gdn_fused_workspace_size(rows, H, d)`` -> bytes
* ``gdn_chunk_fwd_segmented(q, k, v, log_alpha, beta, segments, S0=None,
  cu_seqlens=None, out_dtype=None, ...)`` -> (y, S_T)
* ``gdn_chunk_fwd_segmented_workspace_size(rows, N, H, dk, dv, segments,
  in_dtype)`` -> bytes
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_F32 = 0
GDN_BF16 = 1
GDN_F16 = 2
GDN_OK = 0

_lib = None


class GdnError(RuntimeError):
    pass


def load_library(path: str = LIB_PATH):
    """Load libgdn.so and declare the C signatures. Raises if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise GdnError("libgdn.so not built (%s); run `python -m gated_deltanet_amd.build`" % path)
    lib = ctypes.CDLL(path)
    vp, fp, ip, i32 = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32
    lib.gdn_chunk_fwd.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, ip, i32, i32, i32, i32, i32,
                                  i32, i32, vp]
    lib.gdn_chunk_fwd.restype = ctypes.c_int
    lib.gdn_decode_step.argtypes = [vp, vp, vp, fp, fp, fp, vp, i32, i32, i32, i32, i32, i32,
                                    vp]
    lib.gdn_decode_step.restype = ctypes.c_int
    f32, i64 = ctypes.c_float, ctypes.c_int64
    lib.gdn_frontend_qkv.argtypes = [vp, vp, vp, fp, ip, i32, i32, i32, i32, f32, vp, vp, vp,
                                     i32, i32, vp]
    lib.gdn_frontend_qkv.restype = ctypes.c_int
    lib.gdn_output_gate.argtypes = [vp, vp, fp, f32, vp, i64, i32, i32, i32, i32, vp]
    lib.gdn_output_gate.restype = ctypes.c_int
    sz = ctypes.c_size_t
    lib.gdn_fused_workspace_size.argtypes = [i64, i32, i32]
    lib.gdn_fused_workspace_size.restype = sz
    lib.gdn_chunk_fwd_fused.argtypes = [vp, vp, vp, fp, fp, fp, fp, vp, fp, f32, f32, vp, fp, ip,
                                        i32, i32, i32, i32, i32, i32, i32, vp, sz, vp]
    lib.gdn_chunk_fwd_fused.restype = ctypes.c_int
    lib.gdn_chunk_fwd_gated.argtypes = [vp, vp, vp, fp, fp, fp, fp, fp, vp, fp, ip, i32, i32,
                                        i32, i32, i32, i32, i32, vp]
    lib.gdn_chunk_fwd_gated.restype = ctypes.c_int
    lib.gdn_decode_step_gated.argtypes = [vp, vp, vp, fp, fp, fp, fp, fp, ip, i32, vp, i32, i32,
                                          i32, i32, i32, i32, vp]
    lib.gdn_decode_step_gated.restype = ctypes.c_int
    lib.gdn_decode_multi.argtypes = [vp, vp, vp, fp, fp, fp, fp, fp, ip, i32, vp, i32, i32, i32,
                                     i32, i32, i32, i32, vp]
    lib.gdn_decode_multi.restype = ctypes.c_int
    lib.gdn_decode_fused.argtypes = [vp, vp, vp, fp, vp, fp, fp, fp, fp, fp, ip, i32, vp, fp, f32,
                                     f32, vp, i32, i32, i32, i32, i32, i32, vp]
    lib.gdn_decode_fused.restype = ctypes.c_int
    lib.gdn_chunk_bwd_workspace_size.argtypes = [i64, i32, i32, i32, i32, i32]
    lib.gdn_chunk_bwd_workspace_size.restype = sz
    lib.gdn_chunk_bwd.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, ip, i32, i32, i32, i32, i32,
                                  vp, vp, vp, fp, fp, fp, i32, i32, vp, sz, vp]
    lib.gdn_chunk_bwd.restype = ctypes.c_int
    lib.gdn_chunk_bwd_gated.argtypes = [vp, vp, vp, fp, fp, fp, fp, fp, vp, fp, ip, i32, i32, i32,
                                        i32, i32, vp, vp, vp, fp, fp, fp, fp, fp, i32, i32, vp,
                                        sz, vp]
    lib.gdn_chunk_bwd_gated.restype = ctypes.c_int
    lib.gdn_conv_state_from_prefill.argtypes = [vp, vp, vp, ip, i32, i32, i32, i32, ip, i32, vp,
                                                i32, vp]
    lib.gdn_conv_state_from_prefill.restype = ctypes.c_int
    lib.gdn_chunk_fwd_segmented_workspace_size.argtypes = [i64, i32, i32, i32, i32, i32, i32]
    lib.gdn_chunk_fwd_segmented_workspace_size.restype = sz
    lib.gdn_chunk_fwd_segmented.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, ip, i32, i32, i32,
                                            i32, i32, i32, vp, sz, i32, i32, vp]
    lib.gdn_chunk_fwd_segmented.restype = ctypes.c_int
    lib.gdn_chunk_fwd_segmented_noalloc.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, ip, i32, i32,
                                                    i32, i32, i32, i32, i32, i32, vp]
    lib.gdn_chunk_fwd_segmented_noalloc.restype = ctypes.c_int
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_last_error.argtypes = []
    lib.gdn_last_error.restype = ctypes.c_char_p
    lib.gdn_version.argtypes = []
    lib.gdn_version.restype = ctypes.c_int
    lib.gdn_prefill_state_columns.argtypes = [i32] * 5
    lib.gdn_prefill_state_columns.restype = ctypes.c_int32
    _lib = lib
    return lib


def _dt(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return GDN_BF16
    if t == torch.float32:
        return GDN_F32
    if t == torch.float16:
        return GDN_F16
    raise GdnError("unsupported dtype %s (fp32, bf16 or fp16)" % t)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(rc, lib, name):
    if rc != GDN_OK:
        raise GdnError("%s: %s (%s)" % (name, lib.gdn_status_string(rc).decode(),
                                        lib.gdn_last_error().decode()))


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t, name, dtype=None):
    """Layout and dtype of a tensor argument. The device is checked last, by
    _devices, after every shape: a short or mis-shaped tensor is rejected
    here, before the library sees a pointer it would read or write past."""
    if not isinstance(t, torch.Tensor):
        raise GdnError("%s must be a tensor" % name)
    if not t.is_contiguous():
        raise GdnError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise GdnError("%s must be %s" % (name, dtype))


def _shape(t, name, shape):
    """t (if given) has exactly this shape."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise GdnError("%s must have shape %s, not %s" % (name, tuple(shape), tuple(t.shape)))


def _devices(*named):
    """Every given (tensor, name) lives on one GPU device; returns it."""
    dev = None
    for t, name in named:
        if t is None:
            continue
        if not t.is_cuda:
            raise GdnError("%s must be a device tensor" % name)
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise GdnError("%s is on %s, the other arguments on %s" % (name, t.device, dev))
    return dev


def _rows_layout(q, name="q"):
    """(rows, H, d) of a token-major tensor [rows, H, d] or [N, T, H, d]."""
    if q.dim() not in (3, 4):
        raise GdnError("%s must be [rows, H, d] or [N, T, H, d]" % name)
    H, d = q.shape[-2], q.shape[-1]
    if H <= 0 or d <= 0:
        raise GdnError("%s has an empty head dimension" % name)
    return q.numel() // (H * d), H, d


def _prefill_shape(q, v, S0, cu_seqlens, N):
    """(N, T, H, dk, dv) of a prefill call; T is the per-sequence length, or
    the total row count when cu_seqlens is given."""
    rows, H, dk = _rows_layout(q)
    dv = v.shape[-1]
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32)
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
            raise GdnError("cu_seqlens must be [N + 1]")
        N = cu_seqlens.numel() - 1
        T = rows
    elif q.dim() == 4:
        N, T = q.shape[0], q.shape[1]
    else:
        if N is None:
            N = S0.shape[0] if S0 is not None else 1
        if N <= 0 or rows % N:
            raise GdnError("rows (%d) must be a multiple of N (%d)" % (rows, N))
        T = rows // N
    if S0 is not None:
        _need(S0, "S0", torch.float32)
        _shape(S0, "S0", (N, H, dk, dv))
    return N, T, H, dk, dv


def _prefill_checked(q, k, v, g1, g2, names):
    """dtypes and shapes of the token inputs of a prefill call: k like q,
    v like q with its own last size, the two per-token gates [.., H]."""
    in_dtype = q.dtype
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, in_dtype)
    _need(g1, names[0], torch.float32)
    _need(g2, names[1], torch.float32)
    _rows_layout(q)
    _shape(k, "k", q.shape)
    if v.dim() != q.dim() or tuple(v.shape[:-1]) != tuple(q.shape[:-1]):
        raise GdnError("v must be %s + [dv], not %s" % (list(q.shape[:-1]), list(v.shape)))
    _shape(g1, names[0], q.shape[:-1])
    _shape(g2, names[1], q.shape[:-1])
    return in_dtype


def _outputs(y, y_shape, y_dtype, S_T, s_shape):
    """Caller-supplied outputs have the shapes and dtypes the call writes."""
    if y is not None:
        _need(y, "y", y_dtype)
        _shape(y, "y", y_shape)
    if S_T is not None:
        _need(S_T, "S_T", torch.float32)
        _shape(S_T, "S_T", s_shape)


def gdn_chunk_fwd(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None, out_dtype=None,
                  S_T=None, y=None, want_state=True, N=None):
    """Chunked prefill. q, k [rows, H, dk]; v [rows, H, dv] (bf16 or fp32);
    log_alpha, beta fp32 [rows, H]; S0 fp32 [N, H, dk, dv] or None; cu_seqlens
    int32 [N+1] (device) or None. Without cu_seqlens the rows hold N
    equal-length sequences back to back: N is taken from a 4-D q [N, T, H, dk],
    else from the argument N, else from S0, else 1. Returns (y, S_T) with y
    shaped like v."""
    lib = load_library()
    in_dtype = _prefill_checked(q, k, v, log_alpha, beta, ("log_alpha", "beta"))
    out_dtype = in_dtype if out_dtype is None else out_dtype
    N, T, H, dk, dv = _prefill_shape(q, v, S0, cu_seqlens, N)
    _dt(out_dtype)
    _outputs(y, v.shape, out_dtype, S_T, (N, H, dk, dv))
    _devices((q, "q"), (k, "k"), (v, "v"), (log_alpha, "log_alpha"), (beta, "beta"), (S0, "S0"),
             (cu_seqlens, "cu_seqlens"), (y, "y"), (S_T, "S_T"))
    if y is None:
        y = torch.empty(v.shape, dtype=out_dtype, device=v.device)
    if S_T is None and want_state:
        S_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=v.device)
    rc = lib.gdn_chunk_fwd(_p(q), _p(k), _p(v), _p(log_alpha), _p(beta), _p(S0), _p(y), _p(S_T),
                           _p(cu_seqlens), N, T, H, dk, dv, _dt(in_dtype), _dt(out_dtype),
                           _stream(v.device))
    _check(rc, lib, "gdn_chunk_fwd")
    return y, S_T


def gdn_chunk_fwd_segmented_workspace_size(rows: int, N: int, H: int, dk: int, dv: int,
                                           segments: int, in_dtype: torch.dtype) -> int:
    return int(load_library().gdn_chunk_fwd_segmented_workspace_size(
        rows, N, H, dk, dv, segments, _dt(in_dtype)))


def gdn_chunk_fwd_segmented(q, k, v, log_alpha, beta, segments, S0=None, cu_seqlens=None,
                            out_dtype=None, S_T=None, y=None, want_state=True, N=None,
                            workspace=None):
    """Segment-parallel prefill: each sequence cut into `segments` pieces whose
    state summaries are computed independently and chained. Arguments and
    results as gdn_chunk_fwd; `workspace` (uint8 device tensor) is allocated
    when not given."""
    lib = load_library()
    in_dtype = _prefill_checked(q, k, v, log_alpha, beta, ("log_alpha", "beta"))
    out_dtype = in_dtype if out_dtype is None else out_dtype
    N, T, H, dk, dv = _prefill_shape(q, v, S0, cu_seqlens, N)
    rows = T if cu_seqlens is not None else N * T
    _dt(out_dtype)
    _outputs(y, v.shape, out_dtype, S_T, (N, H, dk, dv))
    if workspace is not None:
        _need(workspace, "workspace")
    _devices((q, "q"), (k, "k"), (v, "v"), (log_alpha, "log_alpha"), (beta, "beta"), (S0, "S0"),
             (cu_seqlens, "cu_seqlens"), (y, "y"), (S_T, "S_T"), (workspace, "workspace"))
    if y is None:
        y = torch.empty(v.shape, dtype=out_dtype, device=v.device)
    if S_T is None and want_state:
        S_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=v.device)
    nbytes = lib.gdn_chunk_fwd_segmented_workspace_size(rows, N, H, dk, dv, segments,
                                                        _dt(in_dtype))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=v.device)
    rc = lib.gdn_chunk_fwd_segmented(_p(q), _p(k), _p(v), _p(log_alpha), _p(beta), _p(S0), _p(y),
                                     _p(S_T), _p(cu_seqlens), N, T, H, dk, dv, segments,
                                     _p(workspace), workspace.numel() * workspace.element_size(),
                                     _dt(in_dtype),
                                     _dt(out_dtype), _stream(v.device))
    _check(rc, lib, "gdn_chunk_fwd_segmented")
    return y, S_T


NOALLOC_SCRATCH_BYTES = 64 << 20  # GDN_NOALLOC_SCRATCH_BYTES


def gdn_chunk_fwd_segmented_noalloc(q, k, v, log_alpha, beta, segments, S0=None,
                                    cu_seqlens=None, out_dtype=None, S_T=None, y=None,
                                    want_state=True, N=None):
    """gdn_chunk_fwd_segmented with the library's fixed per-GPU scratch as its
    workspace (nothing allocated by the library; calls on one GPU must not
    overlap). y and S_T are allocated here unless given."""
    lib = load_library()
    in_dtype = _prefill_checked(q, k, v, log_alpha, beta, ("log_alpha", "beta"))
    out_dtype = in_dtype if out_dtype is None else out_dtype
    N, T, H, dk, dv = _prefill_shape(q, v, S0, cu_seqlens, N)
    _dt(out_dtype)
    _outputs(y, v.shape, out_dtype, S_T, (N, H, dk, dv))
    _devices((q, "q"), (k, "k"), (v, "v"), (log_alpha, "log_alpha"), (beta, "beta"), (S0, "S0"),
             (cu_seqlens, "cu_seqlens"), (y, "y"), (S_T, "S_T"))
    if y is None:
        y = torch.empty(v.shape, dtype=out_dtype, device=v.device)
    if S_T is None and want_state:
        S_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=v.device)
    rc = lib.gdn_chunk_fwd_segmented_noalloc(_p(q), _p(k), _p(v), _p(log_alpha), _p(beta), _p(S0),
                                             _p(y), _p(S_T), _p(cu_seqlens), N, T, H, dk, dv,
                                             segments, _dt(in_dtype), _dt(out_dtype),
                                             _stream(v.device))
    _check(rc, lib, "gdn_chunk_fwd_segmented_noalloc")
    return y, S_T


def gdn_prefill_state_columns(N: int, H: int, dk: int, dv: int, in_dtype=torch.bfloat16) -> int:
    """State columns per workgroup that gdn_chunk_fwd uses for this shape
    (16, 32, 64 or 128; a query, nothing is launched)."""
    return int(load_library().gdn_prefill_state_columns(N, H, dk, dv, _dt(in_dtype)))


def gdn_chunk_bwd_workspace_size(rows: int, N: int, H: int, dk: int, dv: int,
                                 in_dtype=torch.bfloat16) -> int:
    """Workspace bytes of gdn_chunk_bwd / gdn_chunk_bwd_gated for inputs of
    in_dtype (fp32 inputs keep fp32 chunk-start states, 16-bit ones fp16)."""
    return int(load_library().gdn_chunk_bwd_workspace_size(rows, N, H, dk, dv, _dt(in_dtype)))


def gdn_chunk_bwd(q, k, v, log_alpha, beta, dy, S0=None, dS_T=None, cu_seqlens=None, N=None,
                  grad_dtype=None, workspace=None, want_dS0=True):
    """Gradients of <dy, y> + <dS_T, S_T> of gdn_chunk_fwd with respect to
    (q, k, v, log_alpha, beta, S0). Shapes as gdn_chunk_fwd; dy like v in
    grad_dtype (default: dy's dtype). Returns (dq, dk, dv, dlog_alpha, dbeta,
    dS0) with dS0 None unless want_dS0."""
    lib = load_library()
    in_dtype = _prefill_checked(q, k, v, log_alpha, beta, ("log_alpha", "beta"))
    grad_dtype = dy.dtype if grad_dtype is None else grad_dtype
    _need(dy, "dy", grad_dtype)
    N, T, H, dk, dv = _prefill_shape(q, v, S0, cu_seqlens, N)
    _shape(dy, "dy", v.shape)
    if dS_T is not None:
        _need(dS_T, "dS_T", torch.float32)
        _shape(dS_T, "dS_T", (N, H, dk, dv))
    if workspace is not None:
        _need(workspace, "workspace")
    dev = _devices((q, "q"), (k, "k"), (v, "v"), (log_alpha, "log_alpha"), (beta, "beta"),
                   (S0, "S0"), (dy, "dy"), (dS_T, "dS_T"), (cu_seqlens, "cu_seqlens"),
                   (workspace, "workspace"))
    rows = q.numel() // (H * dk)
    need = gdn_chunk_bwd_workspace_size(rows, N, H, dk, dv, in_dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    dq = torch.empty(q.shape, dtype=grad_dtype, device=dev)
    dk_ = torch.empty(k.shape, dtype=grad_dtype, device=dev)
    dv_ = torch.empty(v.shape, dtype=grad_dtype, device=dev)
    dla = torch.empty(log_alpha.shape, dtype=torch.float32, device=dev)
    db = torch.empty(beta.shape, dtype=torch.float32, device=dev)
    dS0 = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev) if want_dS0 else None
    rc = lib.gdn_chunk_bwd(_p(q), _p(k), _p(v), _p(log_alpha), _p(beta), _p(S0), _p(dy), _p(dS_T),
                           _p(cu_seqlens), N, T, H, dk, dv, _p(dq), _p(dk_), _p(dv_), _p(dla),
                           _p(db), _p(dS0), _dt(in_dtype), _dt(grad_dtype), _p(workspace),
                           workspace.numel() * workspace.element_size(), _stream(dev))
    _check(rc, lib, "gdn_chunk_bwd")
    return dq, dk_, dv_, dla, db, dS0


def gdn_chunk_bwd_gated(q, k, v, a, b, A, dy, b_alpha=None, S0=None, dS_T=None,
                        cu_seqlens=None, N=None, grad_dtype=None, workspace=None, want_dS0=True):
    """gdn_chunk_bwd for the raw-gate prefill (gdn_chunk_fwd_gated): returns
    (dq, dk, dv, da, db, dA, db_alpha, dS0)."""
    lib = load_library()
    in_dtype = _prefill_checked(q, k, v, a, b, ("a", "b"))
    grad_dtype = dy.dtype if grad_dtype is None else grad_dtype
    _need(dy, "dy", grad_dtype)
    N, T, H, dk, dv = _prefill_shape(q, v, S0, cu_seqlens, N)
    _shape(dy, "dy", v.shape)
    _head_params(A, b_alpha, H)
    if dS_T is not None:
        _need(dS_T, "dS_T", torch.float32)
        _shape(dS_T, "dS_T", (N, H, dk, dv))
    if workspace is not None:
        _need(workspace, "workspace")
    dev = _devices((q, "q"), (k, "k"), (v, "v"), (a, "a"), (b, "b"), (A, "A"),
                   (b_alpha, "b_alpha"), (S0, "S0"), (dy, "dy"), (dS_T, "dS_T"),
                   (cu_seqlens, "cu_seqlens"), (workspace, "workspace"))
    rows = q.numel() // (H * dk)
    need = gdn_chunk_bwd_workspace_size(rows, N, H, dk, dv, in_dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    dq = torch.empty(q.shape, dtype=grad_dtype, device=dev)
    dk_ = torch.empty(k.shape, dtype=grad_dtype, device=dev)
    dv_ = torch.empty(v.shape, dtype=grad_dtype, device=dev)
    da = torch.empty(a.shape, dtype=torch.float32, device=dev)
    db = torch.empty(b.shape, dtype=torch.float32, device=dev)
    dA = torch.empty(H, dtype=torch.float32, device=dev)
    dba = torch.empty(H, dtype=torch.float32, device=dev)
    dS0 = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev) if want_dS0 else None
    rc = lib.gdn_chunk_bwd_gated(_p(q), _p(k), _p(v), _p(a), _p(b), _p(A), _p(b_alpha), _p(S0),
                                 _p(dy), _p(dS_T), _p(cu_seqlens), N, T, H, dk, dv, _p(dq),
                                 _p(dk_), _p(dv_), _p(da), _p(db), _p(dA), _p(dba), _p(dS0),
                                 _dt(in_dtype), _dt(grad_dtype), _p(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(dev))
    _check(rc, lib, "gdn_chunk_bwd_gated")
    return dq, dk_, dv_, da, db, dA, dba, dS0


def gdn_conv_state_from_prefill(q_raw, k_raw, v_raw, cu_seqlens=None, N=None, slot_idx=None,
                                conv_state=None, n_slots=None):
    """Convolution cache [slots, H, 3, 3, d] for gdn_decode_fused from a
    prefill batch's raw projections [rows, H, d]: the last three raw rows of
    each sequence, oldest first, zero-padded. Written into conv_state (or a
    new tensor of N slots, or n_slots with slot_idx) and returned."""
    lib = load_library()
    dt = q_raw.dtype
    for t, nm in ((q_raw, "q_raw"), (k_raw, "k_raw"), (v_raw, "v_raw")):
        _need(t, nm, dt)
    rows, H, d = _rows_layout(q_raw, "q_raw")
    _shape(k_raw, "k_raw", q_raw.shape)
    _shape(v_raw, "v_raw", q_raw.shape)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32)
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
            raise GdnError("cu_seqlens must be [N + 1]")
        N = cu_seqlens.numel() - 1
        T = rows
    else:
        N = 1 if N is None else int(N)
        if N <= 0 or rows % N:
            raise GdnError("rows must be a multiple of N")
        T = rows // N
    if slot_idx is not None:
        _need(slot_idx, "slot_idx", torch.int32)
        _shape(slot_idx, "slot_idx", (N,))
    if conv_state is not None:
        _need(conv_state, "conv_state", dt)
        if conv_state.dim() != 5 or tuple(conv_state.shape[1:]) != (H, 3, 3, d):
            raise GdnError("conv_state must be [slots, H, 3, 3, d]")
        if slot_idx is None and conv_state.shape[0] != N:
            raise GdnError("conv_state must hold one slot per sequence without slot_idx")
    dev = _devices((q_raw, "q_raw"), (k_raw, "k_raw"), (v_raw, "v_raw"),
                   (cu_seqlens, "cu_seqlens"), (slot_idx, "slot_idx"), (conv_state, "conv_state"))
    if conv_state is None:
        slots = N if slot_idx is None else int(n_slots)
        conv_state = torch.zeros((slots, H, 3, 3, d), dtype=dt, device=dev)
    slots = conv_state.shape[0]
    rc = lib.gdn_conv_state_from_prefill(_p(q_raw), _p(k_raw), _p(v_raw), _p(cu_seqlens), N, T,
                                         H, d, _p(slot_idx), slots, _p(conv_state), _dt(dt),
                                         _stream(q_raw.device))
    _check(rc, lib, "gdn_conv_state_from_prefill")
    return conv_state


def _head_params(A, b_alpha, H):
    _need(A, "A", torch.float32)
    if A.numel() != H:
        raise GdnError("A must hold one value per head (%d)" % H)
    if b_alpha is not None:
        _need(b_alpha, "b_alpha", torch.float32)
        if b_alpha.numel() != H:
            raise GdnError("b_alpha must hold one value per head (%d)" % H)


def gdn_chunk_fwd_gated(q, k, v, a, b, A, b_alpha=None, S0=None, cu_seqlens=None,
                        out_dtype=None, S_T=None, y=None, want_state=True, N=None):
    """Chunked prefill with the gates computed in-kernel from raw fp32
    pre-activations a, b [rows, H] and per-head A, b_alpha [H]:
    log alpha = -exp(A) softplus(a + b_alpha), beta = sigmoid(b). Otherwise
    as gdn_chunk_fwd."""
    lib = load_library()
    in_dtype = _prefill_checked(q, k, v, a, b, ("a", "b"))
    out_dtype = in_dtype if out_dtype is None else out_dtype
    N, T, H, dk, dv = _prefill_shape(q, v, S0, cu_seqlens, N)
    _head_params(A, b_alpha, H)
    _dt(out_dtype)
    _outputs(y, v.shape, out_dtype, S_T, (N, H, dk, dv))
    _devices((q, "q"), (k, "k"), (v, "v"), (a, "a"), (b, "b"), (A, "A"), (b_alpha, "b_alpha"),
             (S0, "S0"), (cu_seqlens, "cu_seqlens"), (y, "y"), (S_T, "S_T"))
    if y is None:
        y = torch.empty(v.shape, dtype=out_dtype, device=v.device)
    if S_T is None and want_state:
        S_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=v.device)
    rc = lib.gdn_chunk_fwd_gated(_p(q), _p(k), _p(v), _p(a), _p(b), _p(A), _p(b_alpha), _p(S0),
                                 _p(y), _p(S_T), _p(cu_seqlens), N, T, H, dk, dv, _dt(in_dtype),
                                 _dt(out_dtype), _stream(v.device))
    _check(rc, lib, "gdn_chunk_fwd_gated")
    return y, S_T


def gdn_decode_step(q, k, v, log_alpha, beta, S, out_dtype=None, y=None):
    """One decode token per (sequence, head), updating S in place.
    q, k [N, H, dk]; v [N, H, dv]; gates fp32 [N, H]; S fp32 [N, H, dk, dv]."""
    lib = load_library()
    in_dtype = q.dtype
    out_dtype = in_dtype if out_dtype is None else out_dtype
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, in_dtype)
    _need(log_alpha, "log_alpha", torch.float32)
    _need(beta, "beta", torch.float32)
    _need(S, "S", torch.float32)
    if q.dim() != 3:
        raise GdnError("q must be [N, H, dk]")
    N, H, dk = q.shape
    dv = v.shape[-1]
    _shape(k, "k", q.shape)
    _shape(v, "v", (N, H, dv))
    _shape(log_alpha, "log_alpha", (N, H))
    _shape(beta, "beta", (N, H))
    _shape(S, "S", (N, H, dk, dv))
    _dt(out_dtype)
    if y is not None:
        _need(y, "y", out_dtype)
        _shape(y, "y", (N, H, dv))
    _devices((q, "q"), (k, "k"), (v, "v"), (log_alpha, "log_alpha"), (beta, "beta"), (S, "S"),
             (y, "y"))
    if y is None:
        y = torch.empty((N, H, dv), dtype=out_dtype, device=v.device)
    rc = lib.gdn_decode_step(_p(q), _p(k), _p(v), _p(log_alpha), _p(beta), _p(S), _p(y), N, H,
                             dk, dv, _dt(in_dtype), _dt(out_dtype), _stream(v.device))
    _check(rc, lib, "gdn_decode_step")
    return y


def gdn_decode_step_gated(q, k, v, a, b, A, S, b_alpha=None, state_idx=None, out_dtype=None,
                          y=None):
    """One decode token per (sequence, head) with the gates computed in-kernel
    from raw fp32 pre-activations a, b [N, H] and per-head A, b_alpha [H].
    S is [N, H, dk, dv], or with state_idx (int32 [N]) a pool
    [n_slots, H, dk, dv] of which sequence n updates slot state_idx[n]; an
    out-of-range slot leaves the pool untouched and gives y = 0."""
    lib = load_library()
    in_dtype = q.dtype
    out_dtype = in_dtype if out_dtype is None else out_dtype
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, in_dtype)
    _need(a, "a", torch.float32)
    _need(b, "b", torch.float32)
    _need(S, "S", torch.float32)
    if q.dim() != 3:
        raise GdnError("q must be [N, H, dk]")
    N, H, dk = q.shape
    dv = v.shape[-1]
    _shape(k, "k", q.shape)
    _shape(v, "v", (N, H, dv))
    _shape(a, "a", (N, H))
    _shape(b, "b", (N, H))
    _head_params(A, b_alpha, H)
    n_slots = 0
    if state_idx is not None:
        _need(state_idx, "state_idx", torch.int32)
        if state_idx.numel() != N:
            raise GdnError("state_idx must hold one slot per sequence (%d)" % N)
        n_slots = S.shape[0]
    elif S.shape[0] != N:
        raise GdnError("S must be [N, H, dk, dv]")
    if tuple(S.shape[1:]) != (H, dk, dv):
        raise GdnError("S must be [slots, H, dk, dv] with H, dk, dv = %s" % ((H, dk, dv),))
    _dt(out_dtype)
    if y is not None:
        _need(y, "y", out_dtype)
        _shape(y, "y", (N, H, dv))
    _devices((q, "q"), (k, "k"), (v, "v"), (a, "a"), (b, "b"), (A, "A"), (b_alpha, "b_alpha"),
             (S, "S"), (state_idx, "state_idx"), (y, "y"))
    if y is None:
        y = torch.empty((N, H, dv), dtype=out_dtype, device=v.device)
    rc = lib.gdn_decode_step_gated(_p(q), _p(k), _p(v), _p(a), _p(b), _p(A), _p(b_alpha), _p(S),
                                   _p(state_idx), n_slots, _p(y), N, H, dk, dv, _dt(in_dtype),
                                   _dt(out_dtype), _stream(v.device))
    _check(rc, lib, "gdn_decode_step_gated")
    return y


def gdn_decode_multi(q, k, v, g_a, g_b, S, A=None, b_alpha=None, state_idx=None,
                     out_dtype=None, y=None):
    """n_tok decode tokens per sequence in one pass over the state.
    q, k [N, n_tok, H, dk]; v [N, n_tok, H, dv]; g_a, g_b fp32 [N, n_tok, H]
    (log_alpha and beta, or raw a and b when A [H] is given). S is
    [N, H, dk, dv] (updated in place), or with state_idx (int32
    [N, 1 + n_tok]: start slot, then the slot receiving the state after each
    token) a pool [n_slots, H, dk, dv]. Returns y [N, n_tok, H, dv]."""
    lib = load_library()
    in_dtype = q.dtype
    out_dtype = in_dtype if out_dtype is None else out_dtype
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, in_dtype)
    _need(g_a, "g_a", torch.float32)
    _need(g_b, "g_b", torch.float32)
    _need(S, "S", torch.float32)
    if q.dim() != 4:
        raise GdnError("q must be [N, n_tok, H, dk]")
    N, n_tok, H, dk = q.shape
    dv = v.shape[-1]
    _shape(k, "k", q.shape)
    _shape(v, "v", (N, n_tok, H, dv))
    _shape(g_a, "g_a", (N, n_tok, H))
    _shape(g_b, "g_b", (N, n_tok, H))
    if A is not None:
        _head_params(A, b_alpha, H)
    elif b_alpha is not None:
        raise GdnError("b_alpha needs A")
    n_slots = 0
    if state_idx is not None:
        _need(state_idx, "state_idx", torch.int32)
        if tuple(state_idx.shape) != (N, 1 + n_tok):
            raise GdnError("state_idx must be [N, 1 + n_tok]")
        n_slots = S.shape[0]
    elif S.shape[0] != N:
        raise GdnError("S must be [N, H, dk, dv]")
    if S.dim() != 4 or tuple(S.shape[1:]) != (H, dk, dv):
        raise GdnError("S must be [slots, H, dk, dv] with H, dk, dv = %s" % ((H, dk, dv),))
    _dt(out_dtype)
    if y is not None:
        _need(y, "y", out_dtype)
        _shape(y, "y", (N, n_tok, H, dv))
    _devices((q, "q"), (k, "k"), (v, "v"), (g_a, "g_a"), (g_b, "g_b"), (A, "A"),
             (b_alpha, "b_alpha"), (S, "S"), (state_idx, "state_idx"), (y, "y"))
    if y is None:
        y = torch.empty((N, n_tok, H, dv), dtype=out_dtype, device=v.device)
    rc = lib.gdn_decode_multi(_p(q), _p(k), _p(v), _p(g_a), _p(g_b), _p(A), _p(b_alpha), _p(S),
                              _p(state_idx), n_slots, _p(y), N, n_tok, H, dk, dv, _dt(in_dtype),
                              _dt(out_dtype), _stream(v.device))
    _check(rc, lib, "gdn_decode_multi")
    return y


def gdn_decode_fused(q_raw, k_raw, v_raw, conv_w, conv_state, g_a, g_b, S, z, A=None,
                     b_alpha=None, state_idx=None, norm_w=None, l2_eps=1e-6, rms_eps=1e-6,
                     out_dtype=None, o=None):
    """Serving decode of the whole mixer: front end with a convolution cache,
    n_tok recurrence steps and the output gate in one kernel.
    q_raw, k_raw, v_raw, z [N, n_tok, H, d]; conv_w fp32 [3, H*d, 4];
    conv_state [slots, H, 3, 3, d] in the input dtype (the three previous raw
    rows of q, k, v, oldest first) and S fp32 [slots, H, d, d], both updated
    in place (slots = N without state_idx); g_a, g_b fp32 [N, n_tok, H] (log
    alpha and beta, or raw a and b when A is given); state_idx int32
    [N, 1 + n_tok] as for gdn_decode_multi. Returns o [N, n_tok, H, d]."""
    lib = load_library()
    in_dtype = q_raw.dtype
    out_dtype = in_dtype if out_dtype is None else out_dtype
    for t, nm in ((q_raw, "q_raw"), (k_raw, "k_raw"), (v_raw, "v_raw"), (z, "z"),
                  (conv_state, "conv_state")):
        _need(t, nm, in_dtype)
    _need(conv_w, "conv_w", torch.float32)
    _need(g_a, "g_a", torch.float32)
    _need(g_b, "g_b", torch.float32)
    _need(S, "S", torch.float32)
    if q_raw.dim() != 4:
        raise GdnError("q_raw must be [N, n_tok, H, d]")
    N, n_tok, H, d = q_raw.shape
    for t, nm in ((k_raw, "k_raw"), (v_raw, "v_raw"), (z, "z")):
        _shape(t, nm, q_raw.shape)
    _shape(g_a, "g_a", (N, n_tok, H))
    _shape(g_b, "g_b", (N, n_tok, H))
    _shape(conv_w, "conv_w", (3, H * d, 4))
    if A is not None:
        _head_params(A, b_alpha, H)
    elif b_alpha is not None:
        raise GdnError("b_alpha needs A")
    if norm_w is not None:
        _need(norm_w, "norm_w", torch.float32)
        _shape(norm_w, "norm_w", (d,))
    n_slots = 0
    if state_idx is not None:
        _need(state_idx, "state_idx", torch.int32)
        if tuple(state_idx.shape) != (N, 1 + n_tok):
            raise GdnError("state_idx must be [N, 1 + n_tok]")
        n_slots = S.shape[0]
    elif S.shape[0] != N:
        raise GdnError("S must be [N, H, d, d]")
    if tuple(S.shape[1:]) != (H, d, d) or tuple(conv_state.shape) != (S.shape[0], H, 3, 3, d):
        raise GdnError("S must be [slots, H, d, d] and conv_state [slots, H, 3, 3, d]")
    _dt(out_dtype)
    if o is not None:
        _need(o, "o", out_dtype)
        _shape(o, "o", q_raw.shape)
    _devices((q_raw, "q_raw"), (k_raw, "k_raw"), (v_raw, "v_raw"), (conv_w, "conv_w"),
             (conv_state, "conv_state"), (g_a, "g_a"), (g_b, "g_b"), (A, "A"),
             (b_alpha, "b_alpha"), (S, "S"), (state_idx, "state_idx"), (z, "z"),
             (norm_w, "norm_w"), (o, "o"))
    if o is None:
        o = torch.empty((N, n_tok, H, d), dtype=out_dtype, device=q_raw.device)
    rc = lib.gdn_decode_fused(_p(q_raw), _p(k_raw), _p(v_raw), _p(conv_w), _p(conv_state),
                              _p(g_a), _p(g_b), _p(A), _p(b_alpha), _p(S), _p(state_idx), n_slots,
                              _p(z), _p(norm_w), float(l2_eps), float(rms_eps), _p(o), N, n_tok,
                              H, d, _dt(in_dtype), _dt(out_dtype), _stream(q_raw.device))
    _check(rc, lib, "gdn_decode_fused")
    return o


def gdn_frontend_qkv(q_raw, k_raw, v_raw, conv_w, cu_seqlens=None, N=None, l2_eps=1e-6,
                     out_dtype=None, out=None):
    """ShortConv -> SiLU -> L2Norm (q, k) / ShortConv -> SiLU (v) on raw
    projections [rows, H, d]; conv_w fp32 [3, H*d, 4]. Sequence boundaries as
    in gdn_chunk_fwd (cu_seqlens, or N equal-length sequences; default 1).
    Returns (q, k, v)."""
    lib = load_library()
    in_dtype = q_raw.dtype
    out_dtype = in_dtype if out_dtype is None else out_dtype
    for t, nm in ((q_raw, "q_raw"), (k_raw, "k_raw"), (v_raw, "v_raw")):
        _need(t, nm, in_dtype)
    _need(conv_w, "conv_w", torch.float32)
    rows, H, d = _rows_layout(q_raw, "q_raw")
    _shape(k_raw, "k_raw", q_raw.shape)
    _shape(v_raw, "v_raw", q_raw.shape)
    if tuple(conv_w.shape) != (3, H * d, 4):
        raise GdnError("conv_w must be [3, H*d, 4]")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32)
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
            raise GdnError("cu_seqlens must be [N + 1]")
        N, T = cu_seqlens.numel() - 1, rows
    else:
        N = 1 if N is None else N
        if N <= 0 or rows % N:
            raise GdnError("rows (%d) must be a multiple of N (%d)" % (rows, N))
        T = rows // N
    _dt(out_dtype)
    if out is not None:
        if len(out) != 3:
            raise GdnError("out must be a (q, k, v) triple")
        for t, nm in zip(out, ("q", "k", "v")):
            _need(t, nm, out_dtype)
            _shape(t, nm, q_raw.shape)
    outs = () if out is None else tuple(zip(out, ("q", "k", "v")))
    _devices((q_raw, "q_raw"), (k_raw, "k_raw"), (v_raw, "v_raw"), (conv_w, "conv_w"),
             (cu_seqlens, "cu_seqlens"), *outs)
    if out is None:
        out = tuple(torch.empty(q_raw.shape, dtype=out_dtype, device=q_raw.device)
                    for _ in range(3))
    q, k, v = out
    rc = lib.gdn_frontend_qkv(_p(q_raw), _p(k_raw), _p(v_raw), _p(conv_w), _p(cu_seqlens), N, T,
                              H, d, float(l2_eps), _p(q), _p(k), _p(v), _dt(in_dtype),
                              _dt(out_dtype), _stream(q_raw.device))
    _check(rc, lib, "gdn_frontend_qkv")
    return q, k, v


def gdn_output_gate(y, z, norm_w=None, rms_eps=1e-6, out_dtype=None, o=None):
    """o = sigmoid(z) * y / sqrt(mean(y^2) + eps) * (1 + norm_w) over the last
    dimension (d in {64, 128}); y and z may have different dtypes."""
    lib = load_library()
    in_dtype = y.dtype
    out_dtype = in_dtype if out_dtype is None else out_dtype
    _need(y, "y", in_dtype)
    _need(z, "z", z.dtype)
    if z.shape != y.shape:
        raise GdnError("z must have the shape of y")
    if y.dim() < 1:
        raise GdnError("y must have a feature dimension")
    d = y.shape[-1]
    if norm_w is not None:
        _need(norm_w, "norm_w", torch.float32)
        _shape(norm_w, "norm_w", (d,))
    rows = y.numel() // d if d > 0 else 0
    _dt(out_dtype)
    if o is not None:
        _need(o, "o", out_dtype)
        _shape(o, "o", y.shape)
    _devices((y, "y"), (z, "z"), (norm_w, "norm_w"), (o, "o"))
    if o is None:
        o = torch.empty(y.shape, dtype=out_dtype, device=y.device)
    rc = lib.gdn_output_gate(_p(y), _p(z), _p(norm_w), float(rms_eps), _p(o), rows, d,
                             _dt(in_dtype), _dt(z.dtype), _dt(out_dtype), _stream(y.device))
    _check(rc, lib, "gdn_output_gate")
    return o


def gdn_fused_workspace_size(rows: int, H: int, d: int) -> int:
    """Workspace bytes gdn_chunk_fwd_fused needs (0 for invalid sizes)."""
    return int(load_library().gdn_fused_workspace_size(int(rows), int(H), int(d)))


def gdn_chunk_fwd_fused(q_raw, k_raw, v_raw, conv_w, log_alpha, beta, z, S0=None, norm_w=None,
                        l2_eps=1e-6, rms_eps=1e-6, cu_seqlens=None, N=None, out_dtype=None,
                        o=None, S_T=None, want_state=True, workspace=None):
    """Front end -> chunked prefill -> output gate in one library call.
    q_raw, k_raw, v_raw, z [rows, H, d] (one dtype); conv_w fp32 [3, H*d, 4];
    gates fp32 [rows, H]; S0 fp32 [N, H, d, d] or None; norm_w fp32 [d] or
    None. Sequence boundaries as in gdn_chunk_fwd. The workspace (fp16 q, k, v
    and y) is allocated here unless given. Returns (o, S_T)."""
    lib = load_library()
    in_dtype = q_raw.dtype
    out_dtype = in_dtype if out_dtype is None else out_dtype
    for t, nm in ((q_raw, "q_raw"), (k_raw, "k_raw"), (v_raw, "v_raw"), (z, "z")):
        _need(t, nm, in_dtype)
    _need(conv_w, "conv_w", torch.float32)
    _need(log_alpha, "log_alpha", torch.float32)
    _need(beta, "beta", torch.float32)
    rows, H, d = _rows_layout(q_raw, "q_raw")
    for t, nm in ((k_raw, "k_raw"), (v_raw, "v_raw"), (z, "z")):
        _shape(t, nm, q_raw.shape)
    _shape(log_alpha, "log_alpha", q_raw.shape[:-1])
    _shape(beta, "beta", q_raw.shape[:-1])
    if tuple(conv_w.shape) != (3, H * d, 4):
        raise GdnError("conv_w must be [3, H*d, 4]")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32)
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
            raise GdnError("cu_seqlens must be [N + 1]")
        N, T = cu_seqlens.numel() - 1, rows
    else:
        if N is None:
            N = S0.shape[0] if S0 is not None else 1
        if N <= 0 or rows % N:
            raise GdnError("rows (%d) must be a multiple of N (%d)" % (rows, N))
        T = rows // N
    if S0 is not None:
        _need(S0, "S0", torch.float32)
        if tuple(S0.shape) != (N, H, d, d):
            raise GdnError("S0 must be [N, H, d, d] = %s" % ((N, H, d, d),))
    if norm_w is not None:
        _need(norm_w, "norm_w", torch.float32)
        _shape(norm_w, "norm_w", (d,))
    _dt(out_dtype)
    if o is not None:
        _need(o, "o", out_dtype)
        _shape(o, "o", q_raw.shape)
    _outputs(None, None, None, S_T, (N, H, d, d))
    if workspace is not None:
        _need(workspace, "workspace")
    dev = _devices((q_raw, "q_raw"), (k_raw, "k_raw"), (v_raw, "v_raw"), (conv_w, "conv_w"),
                   (log_alpha, "log_alpha"), (beta, "beta"), (z, "z"), (S0, "S0"),
                   (norm_w, "norm_w"), (cu_seqlens, "cu_seqlens"), (o, "o"), (S_T, "S_T"),
                   (workspace, "workspace"))
    if o is None:
        o = torch.empty(q_raw.shape, dtype=out_dtype, device=dev)
    if S_T is None and want_state:
        S_T = torch.empty((N, H, d, d), dtype=torch.float32, device=dev)
    need = gdn_fused_workspace_size(rows, H, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    rc = lib.gdn_chunk_fwd_fused(_p(q_raw), _p(k_raw), _p(v_raw), _p(conv_w), _p(log_alpha),
                                 _p(beta), _p(S0), _p(z), _p(norm_w), float(l2_eps),
                                 float(rms_eps), _p(o), _p(S_T), _p(cu_seqlens), N, T, H, d, d,
                                 _dt(in_dtype), _dt(out_dtype), _p(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(dev))
    _check(rc, lib, "gdn_chunk_fwd_fused")
    return o, S_T


def gdn_version() -> int:
    return int(load_library().gdn_version())


# short aliases
chunk_fwd = gdn_chunk_fwd
decode_step = gdn_decode_step
