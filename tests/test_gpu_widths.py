"""Unequal group widths (eq 18): forward, dX and dW of the complete-graph law against the oracle.

qalg_forward_widths / qalg_backward_dx_widths / qalg_backward_dw_widths take the
group widths along K and N; the oracle evaluates the same rows and VJPs with
row_typed_forward / row_typed_backward(in_widths=..., out_widths=...).
"""
import numpy as np
import pytest

import gemm_qalg_forward_amd as Q
import synth
from gpu_common import make_tau, say, tau_dev, to_dev, to_f64, torch_cuda
from oracle import qalg_oracle as O
from qalg_check import BF16_TOL, _rel, backward_elementwise, forward_elementwise

pytestmark = pytest.mark.gpu


def _bounds(widths):
    b = np.concatenate([[0], np.cumsum(widths)])
    return [(int(b[g]), int(b[g + 1])) for g in range(len(widths))]


def _col_errs(got, ref, widths):
    return [_rel(got[:, a:b], ref[:, a:b]) for a, b in _bounds(widths)]


def _block_errs(got, ref, kw, nw):
    return [_rel(got[a:b, c:d], ref[a:b, c:d]) for a, b in _bounds(kw) for c, d in _bounds(nw)]


CASES = [
    # M, in widths (K), out widths (N), tau kind, bad rows, split dW workspace
    (2048, [512, 256, 256, 1024], [1024, 512, 1536, 1024], "cyclic", 0, False),
    (1000, [64, 192, 128], [256, 128, 640], "random", 5, True),
    (777, [8, 120, 256, 40], [72, 8, 200, 32], "random", 0, False),
    (1536, [768, 256], [1024, 3072], "cyclic", 0, True),
    (1200, [256] * 4, [512] * 4, "random", 3, False),
    (1100, [192, 384, 576], [384, 128, 256], "random", 2, True),
    # the persistent kernels at their edges: one group (the plain product), and
    # two very unequal groups with barely 128 rows per type and out-of-range rows
    (300, [512], [768], "cyclic", 0, False),
    (265, [1792, 256], [256, 2304], "random", 4, True),
]


@pytest.mark.parametrize("case", CASES, ids=[f"M{c[0]}q{len(c[1])}K{sum(c[1])}N{sum(c[2])}{c[3]}" for c in CASES])
def test_widths_forward_and_gradients_match_oracle(case):
    torch = torch_cuda()
    M, kw, nw, kind, bad, split = case
    q, K, N = len(kw), sum(kw), sum(nw)
    say(f"[widths] M={M} in={kw} out={nw} tau={kind} bad={bad} split={split}")
    X = synth.normal_operand(9730 + M, (M, K), 1.0, "bf16")
    W = synth.normal_operand(9830 + M, (K, N), K ** -0.5, "bf16")
    dY = synth.normal_operand(9930 + M, (M, N), 1.0, "bf16")
    tau = make_tau(kind, M, q, seed=M + 37, bad=bad)
    Xd, Wd, dYd, td = to_dev(X), to_dev(W), to_dev(dY), tau_dev(tau)
    ws = Q.workspace(q, M, dw_shape=(K, N) if split else None)
    Y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    dX = torch.full((M, K), 7.0, dtype=torch.bfloat16, device="cuda")
    dW = torch.full((K, N), 7.0, dtype=torch.bfloat16, device="cuda")
    Q.qalg_forward_widths(Xd, Wd, td, q, kw, nw, Y=Y, ws=ws)
    Q.qalg_backward_dx_widths(dYd, Wd, td, q, kw, nw, dX=dX, ws=ws, flags=Q.QALG_FLAG_INDEX_READY)
    Q.qalg_backward_dw_widths(Xd, dYd, td, q, kw, nw, dW=dW, ws=ws, flags=Q.QALG_FLAG_INDEX_READY)
    dW2 = Q.qalg_backward_dw_widths(Xd, dYd, td, q, kw, nw, ws=ws, flags=Q.QALG_FLAG_INDEX_READY)
    torch.cuda.synchronize()
    assert torch.equal(dW, dW2), "dW not bitwise reproducible"
    Yr = O.row_typed_forward(X.f64, W.f64, tau, q, in_widths=kw, out_widths=nw)
    dXr, dWr = O.row_typed_backward(X.f64, W.f64, dY.f64, tau, q, in_widths=kw, out_widths=nw)
    e0 = max(_col_errs(to_f64(Y), Yr, nw))
    e1 = max(_col_errs(to_f64(dX), dXr, kw))
    e2 = max(_block_errs(to_f64(dW), dWr, kw, nw))
    say(f"    max rel err Y {e0:.2e}, dX {e1:.2e}, dW {e2:.2e}")
    assert e0 <= BF16_TOL and e1 <= BF16_TOL and e2 <= BF16_TOL
    law = {"in_widths": kw, "out_widths": nw}
    forward_elementwise(to_f64(Y), Yr, X.f64, W.f64, tau, q, "bf16", "Y", **law)
    backward_elementwise(to_f64(dX), dXr, to_f64(dW), dWr, X.f64, W.f64, dY.f64, tau, q, "bf16", **law)
    if bad:
        rows = np.where((tau < 0) | (tau >= q))[0]
        assert np.all(to_f64(Y)[rows] == 0.0) and np.all(to_f64(dX)[rows] == 0.0)
