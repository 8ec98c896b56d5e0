"""The C-ABI library loads, exports every entry point declared in
include/gdn.h, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")
LIB = os.path.join(ROOT, "gated_deltanet_amd", "libgdn.so")


def _ensure_built():
    if not os.path.exists(LIB):
        from gated_deltanet_amd import build
        build.build(verbose=False)


def declared_symbols():
    text = open(HEADER).read()
    return re.findall(r"GDN_API\s+[\w\s\*]+?\b(gdn_\w+)\s*\(", text)


def test_header_declares_entry_points():
    syms = declared_symbols()
    for s in ("gdn_chunk_fwd", "gdn_decode_step", "gdn_status_string", "gdn_last_error",
              "gdn_version"):
        assert s in syms


def test_library_exports_every_declared_symbol():
    _ensure_built()
    lib = ctypes.CDLL(LIB)
    missing = [s for s in declared_symbols() if not hasattr(lib, s)]
    assert not missing, missing


@pytest.fixture(scope="module")
def lib():
    _ensure_built()
    lib = ctypes.CDLL(LIB)
    lib.gdn_last_error.restype = ctypes.c_char_p
    lib.gdn_status_string.restype = ctypes.c_char_p
    v = ctypes.c_void_p
    lib.gdn_chunk_fwd.argtypes = [v] * 9 + [ctypes.c_int32] * 7 + [v]
    lib.gdn_decode_step.argtypes = [v] * 7 + [ctypes.c_int32] * 6 + [v]
    return lib


# fake, never dereferenced: validation must reject these calls before any launch
A = 0x7F0000000000
B = A + (1 << 30)


def _chunk(lib, **kw):
    args = dict(q=A, k=A + (1 << 26), v=A + (2 << 26), la=A + (3 << 26), b=A + (4 << 26), S0=None,
                y=B, ST=B + (1 << 28), cu=None, N=1, T=64, H=2, dk=128, dv=128, it=1, ot=1)
    args.update(kw)
    return lib.gdn_chunk_fwd(args["q"], args["k"], args["v"], args["la"], args["b"], args["S0"],
                             args["y"], args["ST"], args["cu"], args["N"], args["T"], args["H"],
                             args["dk"], args["dv"], args["it"], args["ot"], None)


def test_status_strings(lib):
    assert lib.gdn_status_string(0) == b"GDN_OK"
    assert lib.gdn_status_string(-2) == b"GDN_ERR_UNSUPPORTED"
    assert lib.gdn_status_string(-99) == b"GDN_ERR_UNKNOWN"
    assert lib.gdn_version() >= 100


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1),
    (dict(y=None), -1),
    (dict(N=-1), -1),
    (dict(H=0), -1),
    (dict(dk=96), -2),
    (dict(dv=32), -2),
    (dict(it=7), -2),
    (dict(ot=3), -2),
    (dict(q=A + 4), -3),
    (dict(ST=A + (1 << 26)), -1),   # S_T overlaps k
    (dict(y=A), -1),                # y overlaps q
    (dict(S0=B + (1 << 28) + 64), -1),  # S0 partially overlaps S_T
])
def test_chunk_fwd_rejects(lib, kw, code):
    rc = _chunk(lib, **kw)
    assert rc == code, (rc, lib.gdn_last_error())
    assert lib.gdn_last_error() != b""


def test_decode_rejects(lib):
    rc = lib.gdn_decode_step(A, A + 4096, A + 8192, A + 12288, A + 16384, None, B, 4, 2, 128, 128,
                             1, 1, None)
    assert rc == -1
    rc = lib.gdn_decode_step(A, A + 4096, A + 8192, A + 12288, A + 16384, B, B + 64, 4, 2, 128,
                             128, 1, 1, None)
    assert rc == -1  # S overlaps y
    rc = lib.gdn_decode_step(A, A + 4096, A + 8192, A + 12288, A + 16384, B, B + (1 << 24), 4, 2,
                             128, 100, 1, 1, None)
    assert rc == -2


def test_frontend_and_gate_reject(lib):
    v = ctypes.c_void_p
    lib.gdn_frontend_qkv.argtypes = [v, v, v, v, v, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_float, v, v, v, ctypes.c_int32,
                                     ctypes.c_int32, v]
    lib.gdn_output_gate.argtypes = [v, v, v, ctypes.c_float, v, ctypes.c_int64, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, v]
    base = [A, A + (1 << 26), A + (2 << 26), A + (3 << 26), None, 1, 64, 2, 128, 1e-6,
            B, B + (1 << 26), B + (2 << 26), 1, 1, None]
    bad = list(base); bad[8] = 96
    assert lib.gdn_frontend_qkv(*bad) == -2
    bad = list(base); bad[10] = A + 64          # q overlaps q_raw
    assert lib.gdn_frontend_qkv(*bad) == -1
    bad = list(base); bad[0] = A + 8            # misaligned
    assert lib.gdn_frontend_qkv(*bad) == -3
    bad = list(base); bad[9] = -1.0             # negative eps
    assert lib.gdn_frontend_qkv(*bad) == -1
    assert lib.gdn_output_gate(A, A + 4096, None, 1e-6, A + 64, 16, 128, 1, 1, 1, None) == -1
    assert lib.gdn_output_gate(A, A + 65536, None, 1e-6, B, 16, 100, 1, 1, 1, None) == -2
    assert lib.gdn_output_gate(None, A, None, 1e-6, B, 16, 128, 1, 1, 1, None) == -1
    assert lib.gdn_output_gate(A, A + 65536, None, 1e-6, B, 16, 128, 1, 5, 1, None) == -2


def test_fused_rejects(lib):
    v, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    lib.gdn_fused_workspace_size.argtypes = [ctypes.c_int64, i32, i32]
    lib.gdn_fused_workspace_size.restype = ctypes.c_size_t
    lib.gdn_chunk_fwd_fused.argtypes = [v] * 9 + [f32, f32, v, v, v] + [i32] * 7 + [
        v, ctypes.c_size_t, v]
    rows, H, d = 64, 2, 128
    need = lib.gdn_fused_workspace_size(rows, H, d)
    # fp16 q, k, v and y, each padded to 256 bytes
    assert need == 4 * rows * H * d * 2
    assert lib.gdn_fused_workspace_size(0, H, d) == 0
    assert lib.gdn_fused_workspace_size(rows, H, 96) == 0
    W = B + (1 << 29)
    base = [A, A + (1 << 26), A + (2 << 26), A + (3 << 26), A + (4 << 26), A + (5 << 26), None,
            A + (6 << 26), None, 1e-6, 1e-6, B, B + (1 << 26), None, 1, rows, H, d, d, 1, 1, W,
            need, None]

    def call(**kw):
        args = list(base)
        names = ["qr", "kr", "vr", "w", "la", "b", "S0", "z", "nw", "l2", "rms", "o", "ST", "cu",
                 "N", "T", "H", "dk", "dv", "it", "ot", "ws", "wsb", "st"]
        for key, val in kw.items():
            args[names.index(key)] = val
        return lib.gdn_chunk_fwd_fused(*args)

    assert call(wsb=need - 1) == -1          # workspace too small
    assert call(ws=None) == -1               # workspace missing
    assert call(ws=W + 16) == -3             # workspace not 256-byte aligned
    assert call(dv=64) == -2                 # dk != dv
    assert call(dk=96, dv=96) == -2
    assert call(z=None) == -1
    assert call(o=A + 64) == -1              # o overlaps q_raw
    assert call(ws=A) == -1                  # workspace overlaps the inputs
    assert call(ST=W + 4096) == -1           # S_T inside the workspace
    assert call(rms=-1.0) == -1
    assert call(it=9) == -2
    assert call(it=0) == -2                  # fp32 inputs: intermediates are fp16
    assert b"16-bit" in lib.gdn_last_error()
    assert lib.gdn_last_error() != b""


def test_gated_entry_points_reject(lib):
    v, i32 = ctypes.c_void_p, ctypes.c_int32
    lib.gdn_chunk_fwd_gated.argtypes = [v] * 11 + [i32] * 7 + [v]
    lib.gdn_decode_step_gated.argtypes = [v] * 9 + [i32] + [v] + [i32] * 6 + [v]

    def chunk(**kw):
        a = dict(q=A, k=A + (1 << 26), v=A + (2 << 26), a=A + (3 << 26), b=A + (4 << 26),
                 Ah=A + (5 << 26), ba=A + (5 << 26) + 256, S0=None, y=B, ST=B + (1 << 28),
                 cu=None, N=1, T=64, H=2, dk=128, dv=128, it=1, ot=1)
        a.update(kw)
        return lib.gdn_chunk_fwd_gated(a["q"], a["k"], a["v"], a["a"], a["b"], a["Ah"], a["ba"],
                                       a["S0"], a["y"], a["ST"], a["cu"], a["N"], a["T"], a["H"],
                                       a["dk"], a["dv"], a["it"], a["ot"], None)

    assert chunk(Ah=None) == -1            # A is required
    assert chunk(Ah=A + (5 << 26) + 2) == -3
    assert chunk(ba=B + 16) == -1          # b_alpha overlaps y
    assert chunk(Ah=B + (1 << 28)) == -1   # A overlaps S_T
    assert chunk(dk=96) == -2
    assert lib.gdn_last_error() != b""

    def dec(**kw):
        a = dict(q=A, k=A + 4096, v=A + 8192, a=A + 12288, b=A + 16384, Ah=A + 20480,
                 ba=None, S=B, idx=A + 24576, ns=8, y=B + (1 << 26), N=4, H=2, dk=128, dv=128)
        a.update(kw)
        return lib.gdn_decode_step_gated(a["q"], a["k"], a["v"], a["a"], a["b"], a["Ah"], a["ba"],
                                         a["S"], a["idx"], a["ns"], a["y"], a["N"], a["H"],
                                         a["dk"], a["dv"], 1, 1, None)

    assert dec(Ah=None) == -1
    assert dec(ns=-1) == -1
    assert dec(idx=B + 64) == -1            # state_idx overlaps the pool
    assert dec(idx=A + 24578) == -3
    assert dec(S=None) == -1                # a pool of 8 slots needs S
    # y past the first N states but inside the 8-slot pool (1 MiB)
    assert dec(y=B + (768 << 10)) == -1
    assert dec(dv=100) == -2


def test_decode_multi_rejects(lib):
    v, i32 = ctypes.c_void_p, ctypes.c_int32
    lib.gdn_decode_multi.argtypes = [v] * 9 + [i32] + [v] + [i32] * 7 + [v]

    def dec(**kw):
        a = dict(q=A, k=A + (1 << 20), v=A + (2 << 20), a=A + (3 << 20), b=A + (4 << 20),
                 Ah=None, ba=None, S=B, idx=None, ns=0, y=B + (1 << 26), N=4, nt=4, H=2, dk=128,
                 dv=128)
        a.update(kw)
        return lib.gdn_decode_multi(a["q"], a["k"], a["v"], a["a"], a["b"], a["Ah"], a["ba"],
                                    a["S"], a["idx"], a["ns"], a["y"], a["N"], a["nt"], a["H"],
                                    a["dk"], a["dv"], 1, 1, None)

    assert dec(nt=0) == -1
    assert dec(nt=9) == -1
    assert dec(y=B + 4096) == -1            # y overlaps the states
    # y rows of 4 tokens: 4*4*2*128*2 bytes = 8 KiB; q at y + 4 KiB overlaps
    assert dec(q=B + (1 << 26) + 4096) == -1
    # the index table [N, 1 + n_tok] = 80 bytes must not overlap the pool
    assert dec(idx=B + 64, ns=4) == -1
    assert dec(dk=32) == -2


def test_decode_fused_rejects(lib):
    v, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    lib.gdn_decode_fused.argtypes = ([v] * 11 + [i32] + [v, v, f32, f32, v] + [i32] * 6 + [v])

    def dec(**kw):
        a = dict(q=A, k=A + (1 << 20), v=A + (2 << 20), w=A + (3 << 20), cs=B + (1 << 28),
                 ga=A + (4 << 20), gb=A + (5 << 20), Ah=None, ba=None, S=B, idx=None, ns=0,
                 z=A + (6 << 20), nw=None, l2=1e-6, rms=1e-6, o=B + (1 << 26), N=4, nt=2, H=2,
                 d=128)
        a.update(kw)
        return lib.gdn_decode_fused(a["q"], a["k"], a["v"], a["w"], a["cs"], a["ga"], a["gb"],
                                    a["Ah"], a["ba"], a["S"], a["idx"], a["ns"], a["z"], a["nw"],
                                    a["l2"], a["rms"], a["o"], a["N"], a["nt"], a["H"], a["d"], 1,
                                    1, None)

    assert dec(d=96) == -2
    assert dec(l2=-1.0) == -1
    assert dec(w=None) == -1
    assert dec(z=None) == -1
    assert dec(cs=None) == -1
    assert dec(cs=B + 4096) == -1           # conv_state overlaps S
    assert dec(cs=A + (6 << 20)) == -1      # conv_state overlaps z
    assert dec(cs=B + (1 << 28) + 8) == -3


def test_chunk_bwd_workspace_run_hooks(lib, monkeypatch):
    """The run hooks size the partial sums: GDN_BWD_SEGMENT_ROWS (whole
    chunks) keeps segment + 32 rows, GDN_BWD_RUNS the proportional bound
    ceil((rows + 31 N) / runs) + 32 N rows; more than one run adds the
    carried state gradients and the runs' offset table."""
    i32, sz = ctypes.c_int32, ctypes.c_size_t
    lib.gdn_chunk_bwd_workspace_size.argtypes = [ctypes.c_int64, i32, i32, i32, i32, i32]
    lib.gdn_chunk_bwd_workspace_size.restype = sz
    monkeypatch.delenv("GDN_BWD_RUNS", raising=False)
    monkeypatch.delenv("GDN_BWD_SEGMENT_ROWS", raising=False)
    up = lambda x: (x + 255) // 256 * 256
    states = (500 // 32 + 3) * 2 * 64 * 64 * 4
    per_row = 2 * 2 * 130 * 4
    carry = 3 * 2 * 64 * 64 * 4
    one = states + up(500 * per_row)
    assert lib.gdn_chunk_bwd_workspace_size(500, 3, 2, 64, 64, 0) == one
    monkeypatch.setenv("GDN_BWD_SEGMENT_ROWS", "100")  # -> 96 rows, 6 runs
    assert lib.gdn_chunk_bwd_workspace_size(500, 3, 2, 64, 64, 0) == (
        states + up(128 * per_row) + carry + up(6 * 4 * 4))
    monkeypatch.setenv("GDN_BWD_SEGMENT_ROWS", "1000")  # longer than the problem: one run
    assert lib.gdn_chunk_bwd_workspace_size(500, 3, 2, 64, 64, 0) == one
    monkeypatch.delenv("GDN_BWD_SEGMENT_ROWS")
    monkeypatch.setenv("GDN_BWD_RUNS", "4")  # ceil(593 / 4) + 96 = 245 rows
    assert lib.gdn_chunk_bwd_workspace_size(500, 3, 2, 64, 64, 0) == (
        states + up(245 * per_row) + carry + up(4 * 4 * 4))
    monkeypatch.setenv("GDN_BWD_RUNS", "1")
    assert lib.gdn_chunk_bwd_workspace_size(500, 3, 2, 64, 64, 0) == one


def test_prefill_state_columns(lib, monkeypatch):
    """The prefill's column-tile width by batch shape (the rounds-times-step
    estimate): the timed shapes, an intermediate batch, fp32 inputs, dk = 64,
    the test hook, and invalid sizes."""
    i32 = ctypes.c_int32
    lib.gdn_prefill_state_columns.argtypes = [i32] * 5
    lib.gdn_prefill_state_columns.restype = i32
    monkeypatch.delenv("GDN_PREFILL_NS", raising=False)
    cols = lib.gdn_prefill_state_columns
    assert cols(4, 16, 128, 128, 1) == 32     # B4 H16: 256 workgroups, one round
    assert cols(1, 32, 128, 128, 1) == 16     # B1 H32: 16 columns fill the 256 CUs
    assert cols(64, 16, 128, 128, 2) == 128   # varlen front-end batch: whole heads
    assert cols(8, 16, 128, 128, 1) == 64     # 256 workgroups of 64 columns
    assert cols(64, 16, 128, 128, 0) == 32    # fp32 inputs: their own kernel
    assert cols(64, 16, 64, 64, 1) == 32      # dk = 64: two state waves
    assert cols(4, 16, 128, 64, 1) == 16      # dv = 64: 256 slabs, one round
    monkeypatch.setenv("GDN_PREFILL_NS", "4")
    assert cols(4, 16, 128, 128, 1) == 64
    assert cols(4, 16, 96, 128, 1) == 0
    assert cols(4, 0, 128, 128, 1) == 0
    assert cols(4, 16, 128, 128, 7) == 0


def test_chunk_bwd_rejects(lib):
    v, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.gdn_chunk_bwd_workspace_size.argtypes = [ctypes.c_int64, i32, i32, i32, i32, i32]
    lib.gdn_chunk_bwd_workspace_size.restype = sz
    lib.gdn_chunk_bwd.argtypes = [v] * 9 + [i32] * 5 + [v] * 6 + [i32, i32, v, sz, v]
    need = lib.gdn_chunk_bwd_workspace_size(64, 1, 2, 128, 128, 1)
    # states: (64/32 + 1) slots x 2 heads x 128 x 128 in fp16 for 16-bit
    # inputs (fp32 for fp32 inputs); partials: 4 tiles x 64 x 2 x 258 x 4 B
    assert need == 3 * 2 * 32768 + 4 * 64 * 2 * 258 * 4
    assert lib.gdn_chunk_bwd_workspace_size(64, 1, 2, 128, 128, 0) == 3 * 2 * 65536 + 4 * 64 * 2 * 258 * 4
    assert lib.gdn_chunk_bwd_workspace_size(64, 1, 2, 96, 128, 1) == 0
    assert lib.gdn_chunk_bwd_workspace_size(64, 1, 2, 128, 128, 5) == 0
    # long problems keep the partial sums of one run at a time (<= 192 MiB:
    # 3048 rows here) plus the carried state gradients: B4 H16 T4096 d128
    # takes 6 runs of 21 or 22 chunks of every sequence (bound
    # ceil(16508 / 6) + 128 = 2880 rows of partials); with bf16 inputs the
    # whole workspace stays under 0.5 GB
    per_row = 4 * 16 * 258 * 4
    ws = lib.gdn_chunk_bwd_workspace_size(16384, 4, 16, 128, 128, 1)
    assert ws == 516 * 16 * 32768 + 2880 * per_row + 4 * 16 * 65536 + 256
    assert ws < 500e6
    # many short sequences: 22 runs of 3008 consecutive rows (3016 rounded
    # down to whole chunks), 3040 rows of partials
    ws = lib.gdn_chunk_bwd_workspace_size(65536, 512, 16, 128, 128, 1)
    assert ws == ((2048 + 512) * 16 * 32768 + 3040 * per_row + 512 * 16 * 65536 +
                  (22 * 513 * 4 + 255) // 256 * 256)

    def bwd(**kw):
        a = dict(q=A, k=A + (1 << 26), v=A + (2 << 26), la=A + (3 << 26), b=A + (4 << 26),
                 S0=None, dy=A + (5 << 26), dST=None, cu=None, N=1, T=64, H=2, dk=128, dv=128,
                 dq=B, dko=B + (1 << 24), dvo=B + (2 << 24), dla=B + (3 << 24), db=B + (4 << 24),
                 dS0=None, it=1, gt=1, ws=B + (1 << 28), wsb=need)
        a.update(kw)
        return lib.gdn_chunk_bwd(a["q"], a["k"], a["v"], a["la"], a["b"], a["S0"], a["dy"],
                                 a["dST"], a["cu"], a["N"], a["T"], a["H"], a["dk"], a["dv"],
                                 a["dq"], a["dko"], a["dvo"], a["dla"], a["db"], a["dS0"], a["it"],
                                 a["gt"], a["ws"], a["wsb"], None)

    assert bwd(wsb=need - 1) == -1
    assert bwd(ws=None) == -1
    assert bwd(ws=B + (1 << 28) + 16) == -3
    assert bwd(dq=None) == -1
    assert bwd(dk=96) == -2
    assert bwd(gt=5) == -2
    assert bwd(dq=A) == -1                  # dq overlaps q
    assert bwd(dko=B + 64) == -1            # dk overlaps dq
    assert bwd(ws=B) == -1                  # workspace overlaps dq


def test_conv_state_and_gated_bwd_reject(lib):
    v, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.gdn_conv_state_from_prefill.argtypes = [v, v, v, v] + [i32] * 4 + [v, i32, v, i32, v]
    assert lib.gdn_conv_state_from_prefill(A, A + (1 << 20), A + (2 << 20), None, 2, 10, 2, 96,
                                           None, 0, B, 1, None) == -2
    assert lib.gdn_conv_state_from_prefill(A, A + (1 << 20), A + (2 << 20), None, 2, 10, 2, 64,
                                           None, 0, None, 1, None) == -1
    # conv_state (2 slots x 2 heads x 9 x 64 x 2 B) overlapping k_raw
    assert lib.gdn_conv_state_from_prefill(A, A + (1 << 20), A + (2 << 20), None, 2, 10, 2, 64,
                                           None, 0, A + (1 << 20) + 64, 1, None) == -1
    assert lib.gdn_conv_state_from_prefill(A, A + (1 << 20), A + (2 << 20), None, 2, 10, 2, 64,
                                           B, -1, B, 1, None) == -1  # slot table, n_slots < 0
    lib.gdn_chunk_bwd_gated.argtypes = [v] * 11 + [i32] * 5 + [v] * 8 + [i32, i32, v, sz, v]
    lib.gdn_chunk_bwd_workspace_size.argtypes = [ctypes.c_int64, i32, i32, i32, i32, i32]
    lib.gdn_chunk_bwd_workspace_size.restype = sz
    need = lib.gdn_chunk_bwd_workspace_size(64, 1, 2, 128, 128, 1)
    args = [A, A + (1 << 26), A + (2 << 26), A + (3 << 26), A + (4 << 26), None, None, None,
            A + (5 << 26), None, None, 1, 64, 2, 128, 128, B, B + (1 << 24), B + (2 << 24),
            B + (3 << 24), B + (4 << 24), B + (5 << 24), B + (5 << 24) + 64, None, 1, 1,
            B + (1 << 28), need, None]
    assert lib.gdn_chunk_bwd_gated(*args) == -1                     # A is NULL
    args[5] = A + (6 << 26)
    args[21] = None                                                  # dA missing
    assert lib.gdn_chunk_bwd_gated(*args) == -1


def test_segmented_rejects(lib):
    v, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.gdn_chunk_fwd_segmented_workspace_size.argtypes = [ctypes.c_int64] + [i32] * 6
    lib.gdn_chunk_fwd_segmented_workspace_size.restype = sz
    lib.gdn_chunk_fwd_segmented.argtypes = [v] * 9 + [i32] * 6 + [v, sz, i32, i32, v]
    # rows 64, N 1, H 2, d 128, 3 segments, bf16: bounds (256 B padded), two
    # sets of 2 states of 2 x 128 x 128 fp32 (zero-start finals of segments
    # 0 and 1, chained initial states of segments 1 and 2) and one transition
    # of segment 1; nothing scales with the row count
    need = lib.gdn_chunk_fwd_segmented_workspace_size(64, 1, 2, 128, 128, 3, 1)
    per = 2 * 128 * 128 * 4
    assert need == 256 + 2 * 2 * per + per
    assert need == lib.gdn_chunk_fwd_segmented_workspace_size(1 << 20, 1, 2, 128, 128, 3, 1)
    assert lib.gdn_chunk_fwd_segmented_workspace_size(64, 1, 2, 128, 128, 1, 1) == 0
    assert lib.gdn_chunk_fwd_segmented_workspace_size(64, 1, 2, 96, 128, 3, 1) == 0

    def seg(**kw):
        a = dict(q=A, k=A + (1 << 26), v=A + (2 << 26), la=A + (3 << 26), b=A + (4 << 26),
                 S0=None, y=B, ST=B + (1 << 24), cu=None, N=1, T=64, H=2, dk=128, dv=128, P=3,
                 ws=B + (1 << 28), wsb=need, it=1, ot=1)
        a.update(kw)
        return lib.gdn_chunk_fwd_segmented(a["q"], a["k"], a["v"], a["la"], a["b"], a["S0"],
                                           a["y"], a["ST"], a["cu"], a["N"], a["T"], a["H"],
                                           a["dk"], a["dv"], a["P"], a["ws"], a["wsb"], a["it"],
                                           a["ot"], None)

    assert seg(P=1) == -1
    assert seg(P=65) == -1
    assert seg(dk=96) == -2
    assert seg(ws=None) == -1
    assert seg(wsb=need - 1) == -1
    assert seg(ws=B + (1 << 28) + 16) == -3
    assert seg(ws=B + 4096) == -1           # workspace overlaps y
    assert seg(ws=A + (2 << 26)) == -1      # workspace overlaps v
