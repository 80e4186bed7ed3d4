"""The recursive law Q_2^(x)L (appendix C) on the GPU against the oracle's tensor-power table.

qalg_forward, qalg_gated_forward, qalg_backward_dx and qalg_backward_dw with
QALG_FLAG_LAW_TENSOR use eq 36's supports (transposed for the VJPs); the oracle
evaluates the same products from tensor_power_table(L).  Types come from the cyclic schedule, from the
pilot's interval schedule floor((p mod 768) / 192) (appendix D.5), or are
random (with out-of-range rows).
"""
import numpy as np
import pytest

import gemm_qalg_forward_amd as Q
import synth
from gpu_common import make_tau, say, tau_dev, to_dev, to_f64, torch_cuda
from oracle import qalg_oracle as O
from qalg_check import (BF16_TOL, assert_groups, backward_elementwise, forward_elementwise, rel_frob_blocks,
                        rel_frob_col_groups)

pytestmark = pytest.mark.gpu

T = Q.QALG_FLAG_LAW_TENSOR


def _interval_tau(M, seq_len=1536, period=768, q=4):
    """The pilot's schedule over packed sequences of seq_len positions (computed on the device)."""
    torch = torch_cuda()
    pos = torch.from_numpy(synth.cyclic_positions(M, seq_len)).to("cuda")
    td = Q.qalg_type_schedule(pos, q, Q.QALG_SCHEDULE_INTERVAL, period)
    return td, O.type_schedule(synth.cyclic_positions(M, seq_len), q, "interval", period)


LAW_SHAPES = [
    # M, K, N, L, tau kind, offset, bad rows
    (3072, 768, 1536, 2, "interval", 0, 0),   # the pilot's up projection widths (two 1536-position sequences)
    (3072, 1536, 768, 2, "interval", 0, 0),   # the pilot's down projection
    (2048, 1024, 2048, 3, "cyclic", 5, 0),    # L = 3: four classes of 1, 2, 4, 8 segments
    (1000, 512, 1024, 2, "random", 0, 9),     # listed schedule, ragged types, out-of-range rows
    (777, 256, 512, 1, "cyclic", 1, 0),       # L = 1 is Q_2
    (50, 256, 512, 2, "cyclic", 0, 0),        # a few rows per type: ragged single tiles
    (1024, 4096, 2048, 4, "cyclic", 0, 0),    # L = 4, s = 256, r = 128
]


@pytest.mark.parametrize("shape", LAW_SHAPES, ids=[f"M{s[0]}K{s[1]}N{s[2]}L{s[3]}{s[4]}" for s in LAW_SHAPES])
def test_tensor_law_forward_matches_oracle(shape):
    torch = torch_cuda()
    M, K, N, L, kind, off, bad = shape
    q = 2 ** L
    say(f"[law] Q_2^{L}: M={M} K={K} N={N} tau={kind} offset={off} bad={bad}")
    X = synth.normal_operand(9300 + M + L, (M, K), 1.0, "bf16")
    W = synth.normal_operand(9400 + M + L, (K, N), K ** -0.5, "bf16")
    if kind == "interval":
        td, tau = _interval_tau(M)
    else:
        tau = make_tau(kind, M, q, seed=M + 3, offset=off, bad=bad)
        td = tau_dev(tau)
    Xd, Wd = to_dev(X), to_dev(W)
    ws = Q.workspace(q, M)
    Y = Q.qalg_forward(Xd, Wd, td, q, ws=ws, flags=T)
    Y2 = Q.qalg_forward(Xd, Wd, td, q, ws=ws, flags=T | Q.QALG_FLAG_INDEX_READY)
    torch.cuda.synchronize()
    assert Q.qalg_read_status(ws, q, M) == bad
    assert torch.equal(Y, Y2), "forward is not bitwise reproducible"
    Yr = O.row_typed_forward(X.f64, W.f64, tau, q, table=O.tensor_power_table(L))
    e = assert_groups(rel_frob_col_groups(to_f64(Y), Yr, q), BF16_TOL, "Y")
    forward_elementwise(to_f64(Y), Yr, X.f64, W.f64, tau, q, "bf16", "Y", table=O.tensor_power_table(L))
    say(f"    max rel err {e:.2e}")
    if bad:
        rows = np.where((tau < 0) | (tau >= q))[0]
        assert np.all(to_f64(Y)[rows] == 0.0)


def test_tensor_law_differs_from_complete_law():
    """At L = 2 the two laws have different supports: the far group of a type (Hamming distance 2)
    sums four segments under Q_2^(x)2 and two under Q_4."""
    torch = torch_cuda()
    M, K, N, q = 512, 256, 512, 4
    X = synth.normal_operand(9501, (M, K), 1.0, "bf16")
    W = synth.normal_operand(9502, (K, N), K ** -0.5, "bf16")
    tau = make_tau("cyclic", M, q)
    Xd, Wd, td = to_dev(X), to_dev(W), tau_dev(tau)
    Yt = Q.qalg_forward(Xd, Wd, td, q, flags=T)
    Yc = Q.qalg_forward(Xd, Wd, td, q)
    torch.cuda.synchronize()
    r = N // q
    rows0 = np.where(tau == 0)[0]
    yt, yc = to_f64(Yt)[rows0], to_f64(Yc)[rows0]
    # type 0: groups 0 (distance 0), 1 and 2 (distance 1) agree between the laws; group 3 does not
    np.testing.assert_array_equal(yt[:, :r], yc[:, :r])
    assert np.linalg.norm(yt[:, 3 * r:] - yc[:, 3 * r:]) > 0.1 * np.linalg.norm(yc[:, 3 * r:])


GATED_LAW_SHAPES = [
    (3072, 768, 1536, 2, "interval"),   # the pilot's SwiGLU gate/up (D = 768, F = 1536)
    (1024, 512, 1024, 3, "cyclic"),
]


@pytest.mark.parametrize("shape", GATED_LAW_SHAPES, ids=[f"M{s[0]}K{s[1]}F{s[2]}L{s[3]}{s[4]}" for s in GATED_LAW_SHAPES])
def test_tensor_law_gated_forward_matches_oracle(shape):
    torch = torch_cuda()
    M, K, F, L, kind = shape
    q = 2 ** L
    say(f"[law gated] Q_2^{L}: M={M} K={K} F={F} tau={kind}")
    X = synth.normal_operand(9600 + M, (M, K), 1.0, "bf16")
    Wg = synth.normal_operand(9700 + M, (K, F), K ** -0.5, "bf16")
    Wu = synth.normal_operand(9800 + M, (K, F), K ** -0.5, "bf16")
    if kind == "interval":
        td, tau = _interval_tau(M)
    else:
        tau = make_tau(kind, M, q)
        td = tau_dev(tau)
    Wgu = Q.qalg_merge_gate_up(to_dev(Wg), to_dev(Wu), q)
    H = Q.qalg_gated_forward(to_dev(X), Wgu, td, q, flags=T)
    torch.cuda.synchronize()
    Hr = O.gated_forward(X.f64, Wg.f64, Wu.f64, tau, q, table=O.tensor_power_table(L))
    e = assert_groups(rel_frob_col_groups(to_f64(H), Hr, q), BF16_TOL, "H")
    say(f"    max rel err {e:.2e}")


LAW_GRAD_SHAPES = [
    # M, K, N, L, tau kind, bad rows
    (3072, 768, 1536, 2, "interval", 0),    # the pilot's up projection
    (3072, 1536, 768, 2, "interval", 0),    # and down
    (1000, 512, 1024, 2, "random", 9),      # listed types, out-of-range rows
    (512, 256, 512, 3, "cyclic", 0),
    (777, 256, 512, 1, "cyclic", 0),        # L = 1 is Q_2
    # persistent dX / dW: 256- and 192-feature tiles, listed rows, ragged types, every class
    (1000, 1024, 1024, 2, "random", 9),     # ragged row counts (dW's last k-step of a type partly empty)
    (2050, 2048, 2048, 3, "cyclic", 0),     # L = 3, cyclic with M / q not a whole k-step
    (3000, 1536, 1536, 3, "random", 11),    # L = 3 on listed rows, 192 x 192 dW tiles
    (2000, 1024, 2048, 2, "absent", 4),     # a type without rows
]


@pytest.mark.parametrize("shape", LAW_GRAD_SHAPES, ids=[f"M{s[0]}K{s[1]}N{s[2]}L{s[3]}{s[4]}" for s in LAW_GRAD_SHAPES])
def test_tensor_law_gradients_match_oracle(shape):
    """dX and dW under Q_2^(x)L (App B's VJPs with the law's supports) against the oracle."""
    torch = torch_cuda()
    M, K, N, L, kind, bad = shape
    q = 2 ** L
    say(f"[law grads] Q_2^{L}: M={M} K={K} N={N} tau={kind} bad={bad}")
    X = synth.normal_operand(9310 + M + L, (M, K), 1.0, "bf16")
    W = synth.normal_operand(9410 + M + L, (K, N), K ** -0.5, "bf16")
    dY = synth.normal_operand(9510 + M + L, (M, N), 1.0, "bf16")
    if kind == "interval":
        td, tau = _interval_tau(M)
    else:
        tau = make_tau(kind, M, q, seed=M + 13, bad=bad)
        td = tau_dev(tau)
    Xd, Wd, dYd = to_dev(X), to_dev(W), to_dev(dY)
    ws = Q.workspace(q, M)
    Q.qalg_build_index(td, q, ws=ws)
    fl = T | Q.QALG_FLAG_INDEX_READY
    dX = Q.qalg_backward_dx(dYd, Wd, td, q, ws=ws, flags=fl)
    dW = Q.qalg_backward_dw(Xd, dYd, td, q, ws=ws, flags=fl)
    dX2 = Q.qalg_backward_dx(dYd, Wd, td, q, ws=ws, flags=fl)
    dW2 = Q.qalg_backward_dw(Xd, dYd, td, q, ws=ws, flags=fl)
    torch.cuda.synchronize()
    assert torch.equal(dX, dX2) and torch.equal(dW, dW2), "not bitwise reproducible"
    dXr, dWr = O.row_typed_backward(X.f64, W.f64, dY.f64, tau, q, table=O.tensor_power_table(L))
    e1 = assert_groups(rel_frob_col_groups(to_f64(dX), dXr, q), BF16_TOL, "dX")
    e2 = assert_groups(rel_frob_blocks(to_f64(dW), dWr, q), BF16_TOL, "dW")
    backward_elementwise(to_f64(dX), dXr, to_f64(dW), dWr, X.f64, W.f64, dY.f64, tau, q, "bf16",
                         table=O.tensor_power_table(L))
    say(f"    max rel err dX {e1:.2e}, dW {e2:.2e}")
    if bad:
        rows = np.where((tau < 0) | (tau >= q))[0]
        assert np.all(to_f64(dX)[rows] == 0.0)


def test_pilot_gated_training_step_matches_oracle():
    """The pilot's SwiGLU FFN training step under Q_2^(x)2 with its interval schedule (D = 768,
    F = 1536, two 1536-position sequences): merged forward, SwiGLU, down, then all VJPs."""
    from qalg_check import GATED_STEP_TOL
    torch = torch_cuda()
    M, D, F, q, L = 3072, 768, 1536, 4, 2
    say(f"[law train] pilot FFN Q_2^2 M={M} D={D} F={F}")
    X = synth.normal_operand(9601, (M, D), 1.0, "bf16")
    Wg = synth.normal_operand(9602, (D, F), D ** -0.5, "bf16")
    Wu = synth.normal_operand(9603, (D, F), D ** -0.5, "bf16")
    Wdn = synth.normal_operand(9604, (F, D), F ** -0.5, "bf16")
    dY = synth.normal_operand(9605, (M, D), 1.0, "bf16")
    td, tau = _interval_tau(M)
    ws = Q.workspace(q, M)
    Q.qalg_build_index(td, q, ws=ws)
    fl = T | Q.QALG_FLAG_INDEX_READY
    Xd, Wdd, dYd = to_dev(X), to_dev(Wdn), to_dev(dY)
    Wgu = Q.qalg_merge_gate_up(to_dev(Wg), to_dev(Wu), q)
    H, GU = Q.qalg_gated_forward_keep(Xd, Wgu, td, q, ws=ws, flags=fl)   # as the benchmark's pilot step
    Y = Q.qalg_forward(H, Wdd, td, q, ws=ws, flags=fl)
    dH = Q.qalg_backward_dx(dYd, Wdd, td, q, ws=ws, flags=fl)
    dWd = Q.qalg_backward_dw(H, dYd, td, q, ws=ws, flags=fl)
    dGU = Q.qalg_swiglu_backward(GU, dH, q)
    dX = Q.qalg_backward_dx(dGU, Wgu, td, q, ws=ws, flags=fl)
    dWg, dWu = Q.qalg_split_gate_up(Q.qalg_backward_dw(Xd, dGU, td, q, ws=ws, flags=fl), q)
    torch.cuda.synchronize()
    table = O.tensor_power_table(L)
    Yr, _ = O.gated_ffn_forward(X.f64, Wg.f64, Wu.f64, Wdn.f64, tau, q, table)
    dXr, dWgr, dWur, dWdr = O.gated_ffn_backward(X.f64, Wg.f64, Wu.f64, Wdn.f64, dY.f64, tau, q, table)
    e = {"Y": assert_groups(rel_frob_col_groups(to_f64(Y), Yr, q), GATED_STEP_TOL, "Y"),
         "dX": assert_groups(rel_frob_col_groups(to_f64(dX), dXr, q), GATED_STEP_TOL, "dX")}
    for name, got, ref in (("dW_gate", dWg, dWgr), ("dW_up", dWu, dWur), ("dW_down", dWd, dWdr)):
        e[name] = assert_groups(rel_frob_blocks(to_f64(got), ref, q), GATED_STEP_TOL, name)
    say("    " + ", ".join(f"{k} {v:.2e}" for k, v in e.items()))


SPLIT_SHAPES = [
    # M, K, N, L (0: Q_q), q, tau kind
    (3072, 768, 1536, 2, 4, "interval"),   # the pilot's up dW under Q_2^(x)2
    (3072, 1536, 768, 0, 4, "interval"),   # Q_4 on the interval schedule (listed rows)
    (1000, 512, 1024, 0, 4, "random"),
    (512, 256, 512, 3, 8, "cyclic"),       # the recursive law on a cyclic schedule
    (1000, 1024, 1024, 2, 4, "random"),    # persistent pieces of every class on listed rows
    (2050, 2048, 2048, 3, 8, "cyclic"),    # L = 3, all four classes split
]


@pytest.mark.parametrize("shape", SPLIT_SHAPES, ids=[f"M{s[0]}K{s[1]}N{s[2]}L{s[3]}q{s[4]}{s[5]}" for s in SPLIT_SHAPES])
def test_dw_split_contraction_matches_oracle(shape):
    """dW with a workspace of qalg_workspace_bytes_dw: each tile's contraction is split into pieces
    whose fp32 partials are summed in a fixed order (bitwise reproducible)."""
    torch = torch_cuda()
    M, K, N, L, q, kind = shape
    say(f"[dw split] M={M} K={K} N={N} L={L} q={q} tau={kind}")
    X = synth.normal_operand(9320 + M, (M, K), 1.0, "bf16")
    dY = synth.normal_operand(9520 + M, (M, N), 1.0, "bf16")
    if kind == "interval":
        td, tau = _interval_tau(M)
    else:
        tau = make_tau(kind, M, q, seed=M + 17, bad=5 if kind == "random" else 0)
        td = tau_dev(tau)
    Xd, dYd = to_dev(X), to_dev(dY)
    ws = Q.workspace(q, M, dw_shape=(K, N))
    assert ws.numel() == Q.qalg_workspace_bytes_dw(q, M, K, N)
    Q.qalg_build_index(td, q, ws=ws)
    fl = (T if L else 0) | Q.QALG_FLAG_INDEX_READY
    dW = Q.qalg_backward_dw(Xd, dYd, td, q, ws=ws, flags=fl)
    dW2 = Q.qalg_backward_dw(Xd, dYd, td, q, ws=ws, flags=fl)
    dW1 = Q.qalg_backward_dw(Xd, dYd, td, q, flags=fl & ~Q.QALG_FLAG_INDEX_READY)  # small workspace: no split
    torch.cuda.synchronize()
    assert torch.equal(dW, dW2), "split dW is not bitwise reproducible"
    table = O.tensor_power_table(L) if L else None
    _, dWr = O.row_typed_backward(X.f64, np.zeros((K, N)), dY.f64, tau, q, table=table)
    e = assert_groups(rel_frob_blocks(to_f64(dW), dWr, q), BF16_TOL, "dW (split)")
    e1 = assert_groups(rel_frob_blocks(to_f64(dW1), dWr, q), BF16_TOL, "dW")
    say(f"    max rel err split {e:.2e}, unsplit {e1:.2e}")
