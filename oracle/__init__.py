"""Gated DeltaNet oracle: a plain, slow, obviously correct fp64 CPU reference.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The HIP library
never imports, links or calls it, and it shares no code with the HIP library.

Two implementations of the same definitions live here:

* ``gdn_oracle.c`` (plain C, OpenMP over (sequence, head, column block)),
  loaded with ctypes: the workhorse for large shapes and for the CPU baseline;
* ``ref_np.py`` (NumPy, pure Python token loop): a twin for tiny shapes.

What is computed, from the page "NLP——技术报告解读-Qwen3.8-Flash-Next"
(section "Gated DeltaNet 核心机制" for the recurrence, section
"GDN 参数化细节" for the front end, gates and output gate):

* the gated delta rule in its erase-write form and, separately, in its
  closed form alpha (I - beta k k^T) S + beta k v^T;
* the single-token decode update (one step of the same rule);
* ShortConv -> SiLU -> L2Norm front end and sigmoid(z) * zero-centred RMSNorm(y)
  output gate.

Pins (tests/test_oracle.py): the two forms agree; alpha = 1, beta = 0 leaves S
unchanged; orthonormal keys with beta = 1 retrieve the written values
(brute-forced over key orders); beta = 1, q = k, |k| = 1 returns y = v; pure
decay for beta = 0; the d = 1 scalar closed form; rotation invariance; the C
oracle equals the NumPy twin; conv against torch's conv1d and impulse
responses; L2Norm and RMSNorm output norms.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

FORM_ERASE_WRITE = 0
FORM_CLOSED = 1


def build(force: bool = False) -> str:
    """Compile gdn_oracle.c into liboracle.so with gcc (fp64, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
               "-fno-fast-math", "-ffp-contract=off", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _bind(path):
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int32)
    i = ctypes.c_int
    lib.oracle_gdn_fwd.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, ip,
                                   i, i, i, i, i, i, i, i]
    lib.oracle_gdn_fwd.restype = i
    lib.oracle_decode_step.argtypes = [dp, dp, dp, dp, dp, dp, dp,
                                       i, i, i, i, i]
    lib.oracle_decode_step.restype = i
    lib.oracle_frontend.argtypes = [dp, dp, dp, ip, i, i, i, i, i, i,
                                    ctypes.c_double, i]
    lib.oracle_frontend.restype = i
    lib.oracle_output_gate.argtypes = [dp, dp, dp, ctypes.c_double, dp,
                                       ctypes.c_int64, i, i]
    lib.oracle_output_gate.restype = i
    lib.oracle_gdn_bwd.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, ip, i, i, i, i, i,
                                   dp, dp, dp, dp, dp, dp, i]
    lib.oracle_gdn_bwd.restype = i
    lib.oracle_gates_from_raw_bwd.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, dp, dp,
                                              ctypes.c_int64, i]
    lib.oracle_gates_from_raw_bwd.restype = i
    lib.oracle_gates_from_raw.argtypes = [dp, dp, dp, dp, dp, dp,
                                          ctypes.c_int64, i]
    lib.oracle_gates_from_raw.restype = i
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = i
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            _lib = _bind(_LIB)
    return _lib


class use_library:
    """Context manager that points this module at another build of the C
    oracle (used by the mutation tests to run the pins against planted
    mistakes)."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        _load()
        self._saved = _lib
        _lib = _bind(self.path)
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self._saved
        return False


def _f64(a):
    """Exact upcast to a C-contiguous float64 ndarray (accepts torch tensors)."""
    if a is None:
        return None
    if hasattr(a, "detach"):
        import torch
        a = a.detach().to("cpu")
        if a.dtype != torch.float64:
            a = a.to(torch.float64)
        a = a.numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a, ctype=ctypes.c_double):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _cu(cu_seqlens):
    if cu_seqlens is None:
        return None
    if hasattr(cu_seqlens, "detach"):
        cu_seqlens = cu_seqlens.detach().cpu().numpy()
    return np.ascontiguousarray(cu_seqlens, dtype=np.int32)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def gdn_fwd(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None, N=None,
            form=FORM_ERASE_WRITE, nthreads=0, col_blocks=1, want_y=True):
    """Token-by-token recurrence over whole sequences.

    q, k: [sum_T, H, dk]; v: [sum_T, H, dv]; log_alpha, beta: [sum_T, H];
    S0: [N, H, dk, dv] or None (zeros); cu_seqlens: int32 [N+1] or None
    (then N equal-length sequences; N defaults to 1 and T = sum_T / N).
    Returns (y [sum_T, H, dv] float64 or None, S_T [N, H, dk, dv] float64).
    """
    lib = _load()
    q, k, v, la, b = (_f64(x) for x in (q, k, v, log_alpha, beta))
    S0 = _f64(S0)
    cu = _cu(cu_seqlens)
    total, H, dk = q.shape
    dv = v.shape[2]
    if cu is not None:
        N = cu.shape[0] - 1
        T = 0
    else:
        N = 1 if N is None else int(N)
        T = total // N if N else 0
        assert N * T == total
    y = np.zeros((total, H, dv), dtype=np.float64) if want_y else None
    S_T = np.zeros((N, H, dk, dv), dtype=np.float64)
    rc = lib.oracle_gdn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(b),
                            _ptr(S0), _ptr(y), _ptr(S_T),
                            _ptr(cu, ctypes.c_int32), N, T, H, dk, dv,
                            int(form), int(nthreads), int(col_blocks))
    assert rc == 0
    return y, S_T


def decode_step(q, k, v, log_alpha, beta, S, nthreads=0):
    """One decode step. q, k [N, H, dk]; v [N, H, dv]; gates [N, H];
    S [N, H, dk, dv]. Returns (y [N, H, dv], S_new) as float64 arrays."""
    lib = _load()
    q, k, v, la, b = (_f64(x) for x in (q, k, v, log_alpha, beta))
    S = _f64(S).copy()
    N, H, dk = q.shape
    dv = v.shape[2]
    y = np.zeros((N, H, dv), dtype=np.float64)
    rc = lib.oracle_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(b),
                                _ptr(S), _ptr(y), N, H, dk, dv, int(nthreads))
    assert rc == 0
    return y, S


def frontend(x, w, cu_seqlens=None, N=None, l2=True, eps=1e-6, nthreads=0):
    """ShortConv (causal, depthwise, no bias) -> SiLU [-> L2Norm] for one
    stream x [sum_T, H, d] with weights w [H*d, K]."""
    lib = _load()
    x = _f64(x)
    w = _f64(w)
    cu = _cu(cu_seqlens)
    total, H, d = x.shape
    K = w.shape[-1]
    assert w.shape == (H * d, K)
    if cu is not None:
        N = cu.shape[0] - 1
        T = 0
    else:
        N = 1 if N is None else int(N)
        T = total // N if N else 0
    out = np.zeros_like(x)
    rc = lib.oracle_frontend(_ptr(x), _ptr(w), _ptr(out), _ptr(cu, ctypes.c_int32),
                             N, T, H, d, K, 1 if l2 else 0, float(eps),
                             int(nthreads))
    assert rc == 0
    return out


def output_gate(y, z, w=None, eps=1e-6, nthreads=0):
    """o = sigmoid(z) * y / sqrt(mean(y^2) + eps) * (1 + w), per row of the
    last dimension."""
    lib = _load()
    y = _f64(y)
    z = _f64(z)
    w = _f64(w)
    d = y.shape[-1]
    rows = y.size // d
    o = np.zeros_like(y)
    rc = lib.oracle_output_gate(_ptr(y), _ptr(z), _ptr(w), float(eps), _ptr(o),
                                rows, d, int(nthreads))
    assert rc == 0
    return o


def gates_from_raw(a, b, A, b_alpha=None):
    """Gates from raw per-head pre-activations a, b [..., H]:
    log_alpha = -exp(A) * softplus(a + b_alpha), beta = sigmoid(b).
    Returns (log_alpha, beta) as float64 arrays of a's shape."""
    lib = _load()
    a = _f64(a)
    b = _f64(b)
    A = _f64(A)
    b_alpha = _f64(b_alpha)
    H = a.shape[-1]
    assert b.shape == a.shape and A.shape == (H,)
    assert b_alpha is None or b_alpha.shape == (H,)
    rows = a.size // H if H else 0
    la = np.zeros_like(a)
    bt = np.zeros_like(a)
    rc = lib.oracle_gates_from_raw(_ptr(a), _ptr(b), _ptr(A), _ptr(b_alpha),
                                   _ptr(la), _ptr(bt), rows, H)
    assert rc == 0
    return la, bt


def gdn_bwd(q, k, v, log_alpha, beta, S0, dy, dS_T=None, cu_seqlens=None, N=None, nthreads=0):
    """Gradients of L = <dy, y> + <dS_T, S_T> of the forward recurrence with
    respect to (q, k, v, log_alpha, beta, S0). Shapes as gdn_fwd; returns
    float64 arrays (dq, dk, dv, dlog_alpha, dbeta, dS0) with dS0 of shape
    [N, H, dk, dv]."""
    lib = _load()
    q, k, v, la, b, dy = (_f64(x) for x in (q, k, v, log_alpha, beta, dy))
    S0 = _f64(S0)
    dS_T = _f64(dS_T)
    H, dk = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    cu = _cu(cu_seqlens)
    total = q.size // (H * dk)
    if cu is not None:
        N = cu.size - 1
        T = 0
    else:
        if N is None:
            N = S0.shape[0] if S0 is not None else 1
        T = total // N if N else 0
        assert N * T == total
    dq, dk_, dv_ = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dla, db = np.zeros_like(la), np.zeros_like(b)
    dS0 = np.zeros((N, H, dk, dv))
    rc = lib.oracle_gdn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(b), _ptr(S0), _ptr(dy),
                            _ptr(dS_T), _ptr(cu, ctypes.c_int32), N, T, H, dk, dv, _ptr(dq),
                            _ptr(dk_), _ptr(dv_), _ptr(dla), _ptr(db), _ptr(dS0), int(nthreads))
    assert rc == 0
    return dq, dk_, dv_, dla, db, dS0


def gates_from_raw_bwd(a, b, A, b_alpha, dlog_alpha, dbeta):
    """Chain rule through gates_from_raw: returns (da, db, dA, db_alpha) with
    dA, db_alpha summed over all rows, one value per head."""
    lib = _load()
    a, b, A, dla, dbt = (_f64(x) for x in (a, b, A, dlog_alpha, dbeta))
    b_alpha = _f64(b_alpha)
    H = a.shape[-1]
    rows = a.size // H
    da, db = np.zeros_like(a), np.zeros_like(a)
    dA, dba = np.zeros(H), np.zeros(H)
    rc = lib.oracle_gates_from_raw_bwd(_ptr(a), _ptr(b), _ptr(A), _ptr(b_alpha), _ptr(dla),
                                       _ptr(dbt), _ptr(da), _ptr(db), _ptr(dA), _ptr(dba), rows, H)
    assert rc == 0
    return da, db, dA, dba
