"""The seeded generators are deterministic and give the stated shapes and ranges."""
import torch

import gdn_inputs as gi


def test_prefill_deterministic_and_ranges():
    a = gi.prefill_inputs(2, 3, 70, 16, 8, "bf16", 0.02, seed=5)
    b = gi.prefill_inputs(2, 3, 70, 16, 8, "bf16", 0.02, seed=5)
    for key in ("q", "k", "v", "log_alpha", "beta", "S0"):
        assert torch.equal(a[key], b[key])
    assert a["q"].dtype == torch.bfloat16 and a["q"].shape == (140, 3, 16)
    n = a["k"].float().norm(dim=-1)
    assert torch.all((n - 1).abs() < 1e-2)
    assert torch.all(a["log_alpha"] < 0) and torch.all(a["log_alpha"] > -200)
    assert torch.all((a["beta"] > 0) & (a["beta"] < 1))
    c = gi.prefill_inputs(2, 3, 70, 16, 8, "bf16", 0.02, seed=6)
    assert not torch.equal(a["q"], c["q"])


def test_varlen_and_frontend_shapes():
    w = gi.WORKLOADS[4]
    lens = gi.seq_lengths(64, w.len_lo, w.len_hi, seed=4)
    assert int(lens.min()) >= 512 and int(lens.max()) <= 8192
    f = gi.frontend_inputs([5, 9, 1], 2, 8, 8, seed=4)
    assert f["cu_seqlens"].tolist() == [0, 5, 14, 15]
    assert f["conv_w"].shape == (3, 16, 4) and f["q_raw"].shape == (15, 2, 8)


def test_decode_inputs_shapes():
    d = gi.decode_inputs(4, 2, 8, 8, steps=3, seed=3)
    assert d["q"].shape == (3, 4, 2, 8) and d["log_alpha"].shape == (3, 4, 2)
    assert d["S0"].shape == (4, 2, 8, 8)


def test_raw_gates_are_the_draws_behind_gates():
    """With b_alpha = 0 the oracle's gate map applied to the raw draws gives
    the gates that ``gates`` produces (up to its float32 rounding)."""
    import numpy as np

    import oracle

    la, bt = gi.gates(50, 4, seed=9)
    a, b, A, b_alpha = gi.raw_gates(50, 4, seed=9)
    assert b_alpha.shape == (4,) and float(b_alpha.abs().max()) > 0
    la_o, bt_o = oracle.gates_from_raw(a, b, A, None)
    assert np.max(np.abs(la.double().numpy() - la_o)) < 1e-5 * max(1.0, np.abs(la_o).max())
    assert np.max(np.abs(bt.double().numpy() - bt_o)) < 1e-6
