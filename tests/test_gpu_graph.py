"""Graph laws Q_G (section 3.1, eq 9-12): forward and gradients against the oracle.

qalg_forward_graph / qalg_backward_dx_graph / qalg_backward_dw_graph take
per-type out-edge masks; the oracle evaluates the same rows and VJPs from
structure_table(q, edges).  The complete graph on the persistent forward must
reproduce qalg_forward bit for bit; blocks of absent edges must be exactly zero.
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


def _masks(q, edges):
    m = [0] * q
    for a, b in edges:
        m[a] |= 1 << b
    return np.array(m, dtype=np.uint64).view(np.int64)


def _random_graph(q, seed, p=0.5):
    g = np.random.Generator(np.random.PCG64(seed))
    return [(a, b) for a in range(q) for b in range(q) if a != b and g.random() < p]


GRAPH_CASES = [
    # M, K, N, q, tau kind, bad rows, graph
    (2048, 512, 2048, 4, "cyclic", 0, "cycle"),      # 0 -> 1 -> 2 -> 3 -> 0
    (1000, 512, 1024, 4, "random", 7, "random"),     # irregular, listed types, out-of-range rows
    (3072, 1024, 3072, 8, "cyclic", 0, "star"),      # type 0 reaches every group, the others none
    (777, 256, 512, 2, "cyclic", 0, "empty"),        # no edges: a block-diagonal law
    (3072, 768, 3072, 8, "cyclic", 0, "star"),       # K / q = 96: the register-staged forward
    (1111, 384, 2496, 3, "random", 5, "random"),     # q = 3, r = 832: register-staged, ragged tiles
]


def _graph(kind, q, seed):
    if kind == "cycle":
        return [(a, (a + 1) % q) for a in range(q)]
    if kind == "star":
        return [(0, b) for b in range(1, q)]
    if kind == "empty":
        return []
    return _random_graph(q, seed)


@pytest.mark.parametrize("case", GRAPH_CASES, ids=[f"M{c[0]}K{c[1]}N{c[2]}q{c[3]}{c[4]}{c[6]}" for c in GRAPH_CASES])
def test_graph_forward_matches_oracle(case):
    torch = torch_cuda()
    M, K, N, q, kind, bad, gk = case
    edges = _graph(gk, q, M)
    say(f"[graph] M={M} K={K} N={N} q={q} tau={kind} graph={gk} edges={len(edges)}")
    X = synth.normal_operand(9700 + M, (M, K), 1.0, "bf16")
    W = synth.normal_operand(9800 + M, (K, N), K ** -0.5, "bf16")
    tau = make_tau(kind, M, q, seed=M + 29, bad=bad)
    Xd, Wd, td = to_dev(X), to_dev(W), tau_dev(tau)
    adj = torch.from_numpy(_masks(q, edges)).to("cuda")
    ws = Q.workspace(q, M)
    Yd = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")  # every output element is written
    Y = Q.qalg_forward_graph(Xd, Wd, td, q, adj, Y=Yd, ws=ws)
    Y2 = Q.qalg_forward_graph(Xd, Wd, td, q, adj, ws=ws, flags=Q.QALG_FLAG_INDEX_READY)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2), "graph forward is not bitwise reproducible"
    Yr = O.row_typed_forward(X.f64, W.f64, tau, q, edges=edges)
    got = to_f64(Y)
    r = N // q
    e = assert_groups(rel_frob_col_groups(got, Yr, q), BF16_TOL, "Y")
    forward_elementwise(got, Yr, X.f64, W.f64, tau, q, "bf16", "Y", edges=edges)
    for i in range(q):
        rows = np.where(tau == i)[0]
        for j in range(q):
            if j != i and (i, j) not in edges:
                assert np.all(got[rows, j * r:(j + 1) * r] == 0.0), (i, j)
    if bad:
        rows = np.where((tau < 0) | (tau >= q))[0]
        assert np.all(got[rows] == 0.0)
    say(f"    max rel err {e:.2e}")


def test_complete_graph_is_qalg_forward_bitwise():
    torch = torch_cuda()
    M, K, N, q = 1536, 512, 2048, 4
    X = synth.normal_operand(9901, (M, K), 1.0, "bf16")
    W = synth.normal_operand(9902, (K, N), K ** -0.5, "bf16")
    td = tau_dev(make_tau("cyclic", M, q, offset=1))
    adj = torch.from_numpy(_masks(q, O.complete_graph_edges(q))).to("cuda")
    Yg = Q.qalg_forward_graph(to_dev(X), to_dev(W), td, q, adj)
    Yc = Q.qalg_forward(to_dev(X), to_dev(W), td, q)
    torch.cuda.synchronize()
    assert torch.equal(Yg, Yc)


GRAD_CASES = [
    # M, K, N, q, tau kind, bad rows, graph, split dW workspace
    (2048, 512, 1024, 4, "cyclic", 0, "cycle", False),
    (1000, 512, 1024, 4, "random", 7, "random", True),
    (3072, 1024, 3072, 8, "cyclic", 0, "star", True),
    (777, 256, 512, 2, "random", 0, "empty", False),
    (1111, 384, 2496, 3, "random", 5, "random", False),
    (1536, 512, 2048, 4, "cyclic", 0, "complete", True),
    # persistent dW as well (input groups of 192 or 256 features)
    (4096, 1024, 2048, 4, "cyclic", 0, "random", True),
    (3000, 1536, 1536, 3, "random", 5, "random", False),   # listed types, unsplit dW
    (2048, 768, 1536, 4, "cyclic", 0, "cycle", True),      # 192-feature dW tiles
    (4096, 2048, 2048, 8, "cyclic", 0, "star", True),      # one type reaches every group
    (1536, 1024, 1024, 4, "cyclic", 0, "empty", False),    # no edges: every off-diagonal tile is zero
]


@pytest.mark.parametrize("case", GRAD_CASES,
                         ids=[f"M{c[0]}K{c[1]}N{c[2]}q{c[3]}{c[4]}{c[6]}{'split' if c[7] else ''}" for c in GRAD_CASES])
def test_graph_gradients_match_oracle(case):
    """dX and dW under Q_G (appendix B's VJPs with the graph's supports transposed)."""
    torch = torch_cuda()
    M, K, N, q, kind, bad, gk, split = case
    edges = O.complete_graph_edges(q) if gk == "complete" else _graph(gk, q, M)
    say(f"[graph grads] M={M} K={K} N={N} q={q} tau={kind} graph={gk} edges={len(edges)} split={split}")
    X = synth.normal_operand(9720 + M, (M, K), 1.0, "bf16")
    W = synth.normal_operand(9820 + M, (K, N), K ** -0.5, "bf16")
    dY = synth.normal_operand(9920 + M, (M, N), 1.0, "bf16")
    tau = make_tau(kind, M, q, seed=M + 31, bad=bad)
    Xd, Wd, dYd, td = to_dev(X), to_dev(W), to_dev(dY), tau_dev(tau)
    adj = torch.from_numpy(_masks(q, edges)).to("cuda")
    ws = Q.workspace(q, M, dw_shape=(K, N) if split else None)
    dX = torch.full((M, K), 7.0, dtype=torch.bfloat16, device="cuda")
    dW = torch.full((K, N), 7.0, dtype=torch.bfloat16, device="cuda")
    Q.qalg_backward_dx_graph(dYd, Wd, td, q, adj, dX=dX, ws=ws)
    Q.qalg_backward_dw_graph(Xd, dYd, td, q, adj, dW=dW, ws=ws)
    dX2 = Q.qalg_backward_dx_graph(dYd, Wd, td, q, adj, ws=ws, flags=Q.QALG_FLAG_INDEX_READY)
    dW2 = Q.qalg_backward_dw_graph(Xd, dYd, td, q, adj, ws=ws, flags=Q.QALG_FLAG_INDEX_READY)
    torch.cuda.synchronize()
    assert torch.equal(dX, dX2) and torch.equal(dW, dW2), "not bitwise reproducible"
    dXr, dWr = O.row_typed_backward(X.f64, W.f64, dY.f64, tau, q, edges=edges)
    gx, gw = to_f64(dX), to_f64(dW)
    e1 = assert_groups(rel_frob_col_groups(gx, dXr, q), BF16_TOL, "dX")
    e2 = assert_groups(rel_frob_blocks(gw, dWr, q), BF16_TOL, "dW")
    backward_elementwise(gx, dXr, gw, dWr, X.f64, W.f64, dY.f64, tau, q, "bf16", edges=edges)
    s_, r_ = K // q, N // q
    for i in range(q):
        rows = np.where(tau == i)[0]
        for k in range(q):
            if k != i and (i, k) not in edges:
                assert np.all(gx[rows, k * s_:(k + 1) * s_] == 0.0), ("dX", i, k)
                assert np.all(gw[i * s_:(i + 1) * s_, k * r_:(k + 1) * r_] == 0.0), ("dW", i, k)
    if bad:
        rows = np.where((tau < 0) | (tau >= q))[0]
        assert np.all(gx[rows] == 0.0)
    say(f"    max rel err dX {e1:.2e}, dW {e2:.2e}")
