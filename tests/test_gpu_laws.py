"""The recursive law Q_2^(x)L (appendix C) on the GPU against the oracle's tensor-power table.

qalg_forward and qalg_gated_forward with QALG_FLAG_LAW_TENSOR run the
persistent forward with eq 36's supports; the oracle evaluates the same rows
from tensor_power_table(L).  Types come from the cyclic schedule, from the
pilot's interval schedule floor((p mod 768) / 192) (appendix D.5), or are
random (with out-of-range rows).
"""
import numpy as np
import pytest

import gemm_qalg_forward_amd as Q
import synth
from gpu_common import make_tau, say, tau_dev, to_dev, to_f64, torch_cuda
from oracle import qalg_oracle as O
from qalg_check import BF16_TOL, assert_groups, rel_frob_col_groups

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
