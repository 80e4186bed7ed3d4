"""Parity of the HIP path (through the C ABI) with the fp64 oracle on seeded inputs.

Sizes here span several tiles and ragged tails and still let the oracle finish
in seconds; full workload sizes are in test_gpu_workloads.py.
"""
import numpy as np
import pytest

import gemm_qalg_forward_amd as Q
import synth
from gpu_common import make_tau, say, tau_dev, to_dev, to_f64, torch_cuda
from oracle import qalg_oracle as O
from qalg_check import (BF16_TOL, F32_TOL, assert_groups, backward_elementwise, forward_elementwise, rel_frob_blocks,
                        rel_frob_col_groups)

pytestmark = pytest.mark.gpu

SHAPES = [
    # M, K, N, q, tau kind, offset, bad rows
    (64, 256, 256, 2, "cyclic", 0, 0),       # the fp32 workload's shape, in bf16
    (1000, 512, 768, 4, "cyclic", 1, 0),     # r = 192: ragged column tiles
    (3001, 384, 384, 3, "random", 0, 0),     # odd q, ragged row tiles
    (777, 192, 320, 8, "random", 0, 13),     # s = 24, r = 40: groups narrower than a tile; bad types
    (513, 1024, 512, 1, "zeros", 0, 0),      # q = 1: the dense product
    (300, 128, 128, 16, "cyclic", 5, 0),     # s = r = 8
    (2000, 504, 504, 63, "random", 0, 5),    # q = 63: the largest q whose index scans run in one wave
    (1500, 512, 512, 64, "cyclic", 3, 0),    # q = 64: the smallest with block-wide index scans
    (2048, 256, 512, 4, "random", 0, 0),     # some types with many row tiles
    (5000, 512, 1024, 4, "random", 0, 37),   # persistent 256x256 path: ragged row tiles, bad types
    (4099, 768, 768, 3, "cyclic", 2, 0),     # persistent path, odd q, type offset
    (2600, 1024, 2304, 4, "cyclic", 0, 0),   # persistent 256x192 tiles (r = 576 = 3 x 192)
    (2048, 1024, 1536, 4, "cyclic", 1, 0),   # persistent dX and dW (dW tiles 256x192)
    (4096, 2048, 2048, 8, "cyclic", 3, 0),   # persistent dX and dW (256x256), long/short balance
    (2100, 768, 512, 4, "random", 0, 7),     # listed types, ~525 rows per type: persistent dX, dW 192x128
    (3000, 1024, 1024, 4, "random", 0, 11),  # listed, ragged row counts: dW's last k-step of a type half empty
    (2500, 1536, 768, 3, "absent", 0, 6),    # listed, one type without rows: zero dW blocks, no dX tiles
]


def _inputs(M, K, N, dtype, seed):
    X = synth.normal_operand(seed + 1, (M, K), 1.0, dtype)
    W = synth.normal_operand(seed + 2, (K, N), K ** -0.5, dtype)
    dY = synth.normal_operand(seed + 3, (M, N), 1.0, dtype)
    return X, W, dY


@pytest.mark.parametrize("shape", SHAPES, ids=[f"M{s[0]}K{s[1]}N{s[2]}q{s[3]}{s[4]}" for s in SHAPES])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_forward_dx_dw_match_oracle(shape, dtype):
    torch = torch_cuda()
    M, K, N, q, kind, off, bad = shape
    if dtype == "f32" and (K // q) % 4:
        pytest.skip("fp32 needs group widths that are multiples of 4")
    say(f"[parity] {dtype} M={M} K={K} N={N} q={q} tau={kind} offset={off} bad={bad}")
    X, W, dY = _inputs(M, K, N, dtype, 7000 + M)
    tau = make_tau(kind, M, q, seed=M, offset=off, bad=bad)
    Xd, Wd, dYd, td = to_dev(X), to_dev(W), to_dev(dY), tau_dev(tau)
    ws = Q.workspace(q, M)
    Y = Q.qalg_forward(Xd, Wd, td, q, ws=ws)
    dX = Q.qalg_backward_dx(dYd, Wd, td, q, ws=ws, flags=Q.QALG_FLAG_INDEX_READY)
    dW = Q.qalg_backward_dw(Xd, dYd, td, q, ws=ws, flags=Q.QALG_FLAG_INDEX_READY)
    torch.cuda.synchronize()
    assert Q.qalg_read_status(ws, q, M) == bad
    Yr = O.row_typed_forward(X.f64, W.f64, tau, q)
    dXr, dWr = O.row_typed_backward(X.f64, W.f64, dY.f64, tau, q)
    tol = BF16_TOL if dtype == "bf16" else F32_TOL
    ey = assert_groups(rel_frob_col_groups(to_f64(Y), Yr, q), tol, "Y")
    ex = assert_groups(rel_frob_col_groups(to_f64(dX), dXr, q), tol, "dX")
    ew = assert_groups(rel_frob_blocks(to_f64(dW), dWr, q), tol, "dW")
    say(f"    max rel err  Y {ey:.2e}  dX {ex:.2e}  dW {ew:.2e}")
    ry = forward_elementwise(to_f64(Y), Yr, X.f64, W.f64, tau, q, dtype, "Y")
    rx, rw = backward_elementwise(to_f64(dX), dXr, to_f64(dW), dWr, X.f64, W.f64, dY.f64, tau, q, dtype)
    say(f"    per-element error / bound  Y {ry:.2f}  dX {rx:.2f}  dW {rw:.2f}")
    # rows of an out-of-range type are exactly zero in Y and dX
    badrows = (tau < 0) | (tau >= q)
    if badrows.any():
        assert not to_f64(Y)[badrows].any() and not to_f64(dX)[badrows].any()


@pytest.mark.parametrize("M", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("q,K,N", [(4, 512, 768), (8, 256, 768), (2, 1024, 64), (8, 192, 320)])
def test_small_m_paths_match_oracle(M, q, K, N):
    """The weight-streaming path and the tiled path at decode sizes, both against the oracle."""
    torch = torch_cuda()
    X, W, _ = _inputs(M, K, N, "bf16", 9100 + M)
    tau = make_tau("random", M, q, seed=M + q)
    if M >= 3:
        tau[1] = -5  # one row without a type
    Xd, Wd, td = to_dev(X), to_dev(W), tau_dev(tau)
    ws = Q.workspace(q, M)
    Ys = Q.qalg_forward(Xd, Wd, td, q, ws=ws, flags=Q.QALG_FLAG_FORCE_SMALL_M)
    Yt = Q.qalg_forward(Xd, Wd, td, q, ws=ws, flags=Q.QALG_FLAG_FORCE_TILED)
    torch.cuda.synchronize()
    Yr = O.row_typed_forward(X.f64, W.f64, tau, q)
    assert_groups(rel_frob_col_groups(to_f64(Ys), Yr, q), BF16_TOL, "Y small-M")
    assert_groups(rel_frob_col_groups(to_f64(Yt), Yr, q), BF16_TOL, "Y tiled")
    forward_elementwise(to_f64(Ys), Yr, X.f64, W.f64, tau, q, "bf16", "Y small-M")
    forward_elementwise(to_f64(Yt), Yr, X.f64, W.f64, tau, q, "bf16", "Y tiled")
    Ys2 = Q.qalg_forward(Xd, Wd, td, q, ws=ws, flags=Q.QALG_FLAG_FORCE_SMALL_M)
    torch.cuda.synchronize()
    assert torch.equal(Ys, Ys2), "small-M path is not bitwise reproducible"


# (128, 8, 4, ...) to (128, 1, 4, ...) reach the small-M kernel's 512-, 256- and
# (ragged) 128-column chunks, which it picks only when there are enough
# experts (and more 64-column chunks than fit one round); (64, 1, 4, ...) takes
# the 64-column chunks that do fit one round; the last three have groups that
# are not whole 128-byte lines (96 and 160 columns), which run as one chunk
# wider than the group
@pytest.mark.parametrize("E,M,q,K,N", [(3, 1, 4, 512, 256), (4, 8, 8, 256, 768), (5, 64, 4, 512, 192), (2, 300, 8, 256, 256),
                                       (128, 8, 4, 256, 2048), (64, 2, 4, 256, 2048), (128, 1, 4, 256, 768), (64, 1, 4, 256, 768),
                                       (64, 1, 8, 256, 768), (64, 5, 8, 256, 768), (64, 3, 8, 512, 1280)])
def test_batched_experts_match_oracle(E, M, q, K, N):
    torch = torch_cuda()
    Xs, Ws, taus = [], [], []
    for e in range(E):
        X, W, _ = _inputs(M, K, N, "bf16", 9500 + 10 * e)
        Xs.append(X)
        Ws.append(W)
        taus.append(O.type_schedule(synth.random_positions(9900 + e, M), q))
    Xd = torch.stack([to_dev(x) for x in Xs])
    Wd = torch.stack([to_dev(w) for w in Ws])
    td = tau_dev(np.stack(taus))
    Y = Q.qalg_forward_batched(Xd, Wd, td, q)
    torch.cuda.synchronize()
    Yh = to_f64(Y)
    for e in range(E):
        Yr = O.row_typed_forward(Xs[e].f64, Ws[e].f64, taus[e], q)
        assert_groups(rel_frob_col_groups(Yh[e], Yr, q), BF16_TOL, f"expert {e}")
        forward_elementwise(Yh[e], Yr, Xs[e].f64, Ws[e].f64, taus[e], q, "bf16", f"expert {e}")


@pytest.mark.parametrize("kind,q,M,period", [("cyclic", 8, 16384, 0), ("cyclic", 3, 1001, 0),
                                             ("interval", 4, 5000, 768), ("cyclic", 512, 7777, 0)])
def test_type_schedule_and_index_bit_exact(kind, q, M, period):
    torch = torch_cuda()
    pos = synth.random_positions(77 + q, M, 1 << 20) if q % 2 else synth.cyclic_positions(M, 1024, 3)
    code = Q.QALG_SCHEDULE_CYCLIC if kind == "cyclic" else Q.QALG_SCHEDULE_INTERVAL
    tau = Q.qalg_type_schedule(torch.from_numpy(pos).to("cuda"), q, code, period)
    want_tau = O.type_schedule(pos, q, kind, period)
    np.testing.assert_array_equal(tau.cpu().numpy(), want_tau)
    ws = Q.qalg_build_index(tau, q)
    torch.cuda.synchronize()
    _check_index(ws, want_tau, q)


def _check_index(ws, tau, q):
    M = tau.size
    counts, offsets, rows, bad = O.type_index(tau, q)
    lay = Q.qalg_index_layout(q, M)
    w = ws.view(dtype=torch_cuda().int32).cpu().numpy()
    assert w[lay[0]] == bad
    np.testing.assert_array_equal(w[lay[1]:lay[1] + q], counts)
    np.testing.assert_array_equal(w[lay[2]:lay[2] + q + 1], offsets)
    np.testing.assert_array_equal(w[lay[3]:lay[3] + offsets[-1]], rows)
    badrows = np.flatnonzero((tau < 0) | (tau >= q))
    np.testing.assert_array_equal(w[lay[3] + offsets[-1]:lay[3] + M], badrows)


@pytest.mark.parametrize("M,q,kind,bad", [(1, 1, "zeros", 0), (1, 4, "random", 1), (63, 2, "cyclic", 0),
                                          (64, 4, "cyclic", 0), (65, 4, "random", 3), (4096, 8, "random", 0),
                                          (20000, 7, "random", 111), (3000, 512, "random", 0),
                                          (5000, 63, "random", 9), (5000, 63, "cyclic", 0),
                                          (5000, 64, "random", 2), (5000, 64, "cyclic", 0)])
def test_index_edge_cases_bit_exact(M, q, kind, bad):
    torch = torch_cuda()
    tau = make_tau(kind, M, q, seed=M, bad=bad)
    ws = Q.qalg_build_index(tau_dev(tau), q)
    torch.cuda.synchronize()
    _check_index(ws, tau, q)
    assert Q.qalg_read_status(ws, q, M) == bad


@pytest.mark.parametrize("M,q,off,swap", [(16384, 8, 0, None), (20000, 8, 3, None), (4099, 3, 2, None),
                                          (16384, 8, 0, (0, 1)), (16384, 8, 0, (9000, 9001)),
                                          (20000, 8, 3, (19998, 19999)), (3000, 4, 1, (1500, 2999)),
                                          (4099, 63, 5, None), (4099, 64, 60, None)])
def test_cyclic_detection_bit_exact(M, q, off, swap):
    """The index recognises (o + m) mod q at any offset o (its rows are then computed, not listed) and
    rejects a schedule that breaks it anywhere: two rows of different types swapped (same counts)."""
    torch = torch_cuda()
    tau = make_tau("cyclic", M, q, offset=off)
    if swap is not None:
        a, b = swap
        tau[a], tau[b] = tau[b], tau[a]
    ws = Q.qalg_build_index(tau_dev(tau), q)
    torch.cuda.synchronize()
    _check_index(ws, tau, q)
    w = ws.view(dtype=torch.int32).cpu().numpy()
    assert w[4] == (off if swap is None else -1)


def test_unit_law_is_bitwise():
    """A diagonal bank of identity maps is the identity projection (section 4): Y == X exactly."""
    torch = torch_cuda()
    for q, K, M in ((4, 256, 1000), (8, 512, 3), (2, 128, 5)):
        X = synth.normal_operand(11, (M, K), 1.0, "bf16")
        Xd = to_dev(X)
        I = torch.eye(K, dtype=torch.bfloat16, device="cuda")
        tau = tau_dev(make_tau("random", M, q, seed=5))
        for flags in (Q.QALG_FLAG_FORCE_TILED, 0):
            Y = Q.qalg_forward(Xd, I, tau, q, flags=flags)
            torch.cuda.synchronize()
            assert torch.equal(Y, Xd)


def test_block_diagonal_bank_is_type_independent():
    """With W_ij = 0 off the diagonal every type computes X W: outputs for two schedules agree exactly."""
    torch = torch_cuda()
    q, K, N, M = 4, 512, 768, 999
    X = synth.normal_operand(21, (M, K), 1.0, "bf16")
    W = synth.normal_operand(22, (K, N), K ** -0.5, "bf16")
    Wd = to_dev(W)
    s, r = K // q, N // q
    mask = torch.zeros(K, N, dtype=torch.bool, device="cuda")
    for a in range(q):
        mask[a * s:(a + 1) * s, a * r:(a + 1) * r] = True
    Wd = torch.where(mask, Wd, torch.zeros_like(Wd))
    Xd = to_dev(X)
    Y1 = Q.qalg_forward(Xd, Wd, tau_dev(make_tau("cyclic", M, q)), q)
    Y2 = Q.qalg_forward(Xd, Wd, tau_dev(make_tau("random", M, q, seed=3)), q)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2)


@pytest.mark.parametrize("kind", ["random", "cyclic"])
def test_runs_are_bitwise_reproducible(kind):
    """Every output element has one owner: repeated runs are bitwise equal (both kernel families)."""
    torch = torch_cuda()
    q, K, N, M = 8, 2048, 2048, 4096
    X, W, dY = _inputs(M, K, N, "bf16", 31)
    Xd, Wd, dYd = to_dev(X), to_dev(W), to_dev(dY)
    td = tau_dev(make_tau(kind, M, q, seed=9, offset=5))
    outs = []
    for _ in range(2):
        ws = Q.workspace(q, M)
        outs.append((Q.qalg_forward(Xd, Wd, td, q, ws=ws), Q.qalg_backward_dx(dYd, Wd, td, q, ws=ws),
                     Q.qalg_backward_dw(Xd, dYd, td, q, ws=ws)))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_zero_rows_and_absent_types():
    torch = torch_cuda()
    q, K, N = 4, 256, 256
    # M = 0: dW is all zero; forward / dX are no-ops
    X = torch.empty(0, K, dtype=torch.bfloat16, device="cuda")
    dY = torch.empty(0, N, dtype=torch.bfloat16, device="cuda")
    t = torch.empty(0, dtype=torch.int32, device="cuda")
    dW = torch.full((K, N), 3.0, dtype=torch.bfloat16, device="cuda")
    Q.qalg_backward_dw(X, dY, t, q, dW=dW)
    torch.cuda.synchronize()
    assert not dW.any()
    # every row has type 2: off-diagonal dW blocks of other source types are exactly zero
    M = 100
    Xo, _, dYo = _inputs(M, K, N, "bf16", 41)
    tau = np.full(M, 2, np.int32)
    dW = Q.qalg_backward_dw(to_dev(Xo), to_dev(dYo), tau_dev(tau), q)
    torch.cuda.synchronize()
    dWh = to_f64(dW)
    _, dWr = O.row_typed_backward(Xo.f64, np.zeros((K, N)), dYo.f64, tau, q)
    s, r = K // q, N // q
    for b in range(q):
        for j in range(q):
            blk = dWh[b * s:(b + 1) * s, j * r:(j + 1) * r]
            if b != j and b != 2:
                assert not blk.any()
    assert_groups(rel_frob_blocks(dWh, dWr, q), BF16_TOL, "dW")


# ---------------------------------------------------------------------------
# gated (SwiGLU) gate/up forward over the merged bank
# ---------------------------------------------------------------------------

def _merged_reference(Wg_bits, Wu_bits, q):
    """The merged gate/up layout as include/qalg.h states it, built column by column."""
    K, F = Wg_bits.shape
    r = F // q
    out = np.empty((K, 2 * F), dtype=Wg_bits.dtype)
    for j in range(q):
        for t in range(r // 128):
            c0 = j * r + 128 * t
            base = j * 2 * r + 256 * t
            out[:, base:base + 64] = Wg_bits[:, c0:c0 + 64]
            out[:, base + 64:base + 128] = Wu_bits[:, c0:c0 + 64]
            out[:, base + 128:base + 192] = Wg_bits[:, c0 + 64:c0 + 128]
            out[:, base + 192:base + 256] = Wu_bits[:, c0 + 64:c0 + 128]
    return out


@pytest.mark.parametrize("q,K,F", [(4, 64, 1024), (1, 32, 384), (3, 16, 768)])
def test_merge_gate_up_layout_bit_exact(q, K, F):
    torch = torch_cuda()
    Wg = synth.normal_operand(9700 + q, (K, F), 1.0, "bf16")
    Wu = synth.normal_operand(9800 + q, (K, F), 1.0, "bf16")
    Wgu = Q.qalg_merge_gate_up(to_dev(Wg), to_dev(Wu), q)
    torch.cuda.synchronize()
    got = Wgu.view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got, _merged_reference(Wg.bits.view(np.uint16), Wu.bits.view(np.uint16), q))


GATED_SHAPES = [
    # M, K, F, q, tau kind, offset, bad rows
    (2048, 512, 1024, 4, "cyclic", 0, 0),     # r = 256: two 128-column pieces per group
    (1000, 768, 3072, 4, "cyclic", 3, 0),     # the 110M-LM FFN widths, type offset, ragged rows
    (700, 256, 256, 2, "random", 0, 9),       # listed schedule, out-of-range types
    (777, 256, 512, 1, "zeros", 0, 0),        # q = 1: a dense SwiGLU gate/up
    (4096, 1024, 2048, 8, "cyclic", 5, 0),    # q = 8, r = 256
]


@pytest.mark.parametrize("shape", GATED_SHAPES, ids=[f"M{s[0]}K{s[1]}F{s[2]}q{s[3]}{s[4]}" for s in GATED_SHAPES])
def test_gated_forward_matches_oracle(shape):
    torch = torch_cuda()
    M, K, F, q, kind, off, bad = shape
    say(f"[gated] M={M} K={K} F={F} q={q} tau={kind} offset={off} bad={bad}")
    X = synth.normal_operand(9100 + M, (M, K), 1.0, "bf16")
    Wg = synth.normal_operand(9200 + M, (K, F), K ** -0.5, "bf16")
    Wu = synth.normal_operand(9300 + M, (K, F), K ** -0.5, "bf16")
    tau = make_tau(kind, M, q, seed=M + 1, offset=off, bad=bad)
    Xd, td = to_dev(X), tau_dev(tau)
    Wgu = Q.qalg_merge_gate_up(to_dev(Wg), to_dev(Wu), q)
    ws = Q.workspace(q, M)
    H = Q.qalg_gated_forward(Xd, Wgu, td, q, ws=ws)
    H2 = Q.qalg_gated_forward(Xd, Wgu, td, q, ws=ws, flags=Q.QALG_FLAG_INDEX_READY)
    torch.cuda.synchronize()
    assert Q.qalg_read_status(ws, q, M) == bad
    assert torch.equal(H, H2), "gated forward is not bitwise reproducible"
    Hr = O.gated_forward(X.f64, Wg.f64, Wu.f64, tau, q)
    assert_groups(rel_frob_col_groups(to_f64(H), Hr, q), BF16_TOL, "H")
    if bad:
        rows = np.where((tau < 0) | (tau >= q))[0]
        assert np.all(to_f64(H)[rows] == 0.0)


DW_SPLIT_SHAPES = [
    # M, K, N, q, tau kind, offset: persistent dW shapes (cyclic) whose diagonal
    # tiles get split over several workgroups when the dW scratch is given
    (4096, 2048, 2048, 8, "cyclic", 3),   # 16 pieces of 8 k-steps per diagonal tile
    (2048, 1024, 1536, 4, "cyclic", 1),   # 256x192 tiles, 16 pieces
    (2048, 512, 512, 1, "zeros", 0),      # q = 1: every tile is diagonal
    (2048, 1024, 1536, 4, "random", 0),   # listed schedule: row ids from the index, split
    (3072, 768, 768, 3, "cyclic", 2),     # odd q: 16 pieces of 6 k-steps
    (3000, 768, 1536, 4, "random", 0),    # listed, 192-feature tiles, ragged types, short tiles split too
]


@pytest.mark.parametrize("shape", DW_SPLIT_SHAPES, ids=[f"M{s[0]}K{s[1]}N{s[2]}q{s[3]}{s[4]}" for s in DW_SPLIT_SHAPES])
def test_dw_split_contraction_matches_oracle(shape):
    """dW with the split-contraction scratch (App B eq 33-35): diagonal blocks summed from fp32
    pieces in a fixed order; against the oracle, bitwise the same on a second call, and within the
    bar of the unsplit launch."""
    torch = torch_cuda()
    M, K, N, q, kind, off = shape
    say(f"[dw split] M={M} K={K} N={N} q={q} tau={kind} offset={off}")
    X, _, dY = _inputs(M, K, N, "bf16", 7300 + M)
    tau = make_tau(kind, M, q, seed=M, offset=off)
    Xd, dYd, td = to_dev(X), to_dev(dY), tau_dev(tau)
    ws_split = Q.workspace(q, M, dw_shape=(K, N))
    ws_plain = Q.workspace(q, M)
    # the scratch holds stale partials of an earlier call: fill it with garbage first
    ws_split[Q.qalg_workspace_bytes(q, M):].fill_(0x7f)
    dW1 = torch.full((K, N), 3.0, dtype=torch.bfloat16, device="cuda")
    Q.qalg_backward_dw(Xd, dYd, td, q, dW=dW1, ws=ws_split)
    dW2 = Q.qalg_backward_dw(Xd, dYd, td, q, ws=ws_split, flags=Q.QALG_FLAG_INDEX_READY)
    dW0 = Q.qalg_backward_dw(Xd, dYd, td, q, ws=ws_plain)
    torch.cuda.synchronize()
    assert torch.equal(dW1, dW2), "split dW is not reproducible"
    _, dWr = O.row_typed_backward(X.f64, np.zeros((K, N)), dY.f64, tau, q)
    e1 = assert_groups(rel_frob_blocks(to_f64(dW1), dWr, q), BF16_TOL, "dW split")
    e0 = assert_groups(rel_frob_blocks(to_f64(dW0), dWr, q), BF16_TOL, "dW unsplit")
    say(f"    max rel err  dW split {e1:.2e}  unsplit {e0:.2e}")


FEW_ROWS_SHAPES = [
    # M, K, N, q, tau kind, offset, bad rows: forward tiles of 32 / 64 rows and 256 / 128
    # columns (few rows per type), every output element against the oracle
    (200, 512, 1024, 4, "random", 0, 0),   # 64 x 256 tiles (r = 256)
    (100, 768, 2048, 4, "random", 0, 5),   # 32 x 256 tiles (r = 512), rows without a type
    (150, 512, 768, 8, "random", 0, 0),    # 32 x 128 tiles (r = 96: one ragged tile per group)
    (400, 256, 768, 8, "cyclic", 3, 0),    # 64 x 128 tiles, type offset
    (120, 1024, 1536, 4, "random", 0, 0),  # 32 x 128 tiles (r = 384)
    (90, 512, 832, 4, "random", 0, 3),     # 32 x 256 tiles, ragged (r = 208)
]


@pytest.mark.parametrize("shape", FEW_ROWS_SHAPES, ids=[f"M{s[0]}K{s[1]}N{s[2]}q{s[3]}" for s in FEW_ROWS_SHAPES])
def test_few_rows_wide_tiles_match_oracle(shape):
    """The register-staged forward's few-rows tiles (eq 16-17), forced on one problem and as three
    experts of a batched call, every output group against the oracle; rows without a type are zero."""
    torch = torch_cuda()
    M, K, N, q, kind, off, bad = shape
    say(f"[few rows] M={M} K={K} N={N} q={q} tau={kind} bad={bad}")
    X, W, _ = _inputs(M, K, N, "bf16", 7700 + M)
    tau = make_tau(kind, M, q, seed=M + 1, offset=off, bad=bad)
    Y = Q.qalg_forward(to_dev(X), to_dev(W), tau_dev(tau), q, flags=Q.QALG_FLAG_FORCE_TILED)
    torch.cuda.synchronize()
    Yr = O.row_typed_forward(X.f64, W.f64, tau, q)
    e = assert_groups(rel_frob_col_groups(to_f64(Y), Yr, q), BF16_TOL, "Y")
    badrows = (tau < 0) | (tau >= q)
    assert not to_f64(Y)[badrows].any()
    # three experts: the same bank for all, types shifted per expert
    taus = np.stack([make_tau(kind, M, q, seed=M + 1 + x, offset=off, bad=bad) for x in range(3)])
    Xd = torch.stack([to_dev(X)] * 3)
    Wd = torch.stack([to_dev(W)] * 3)
    Yb = Q.qalg_forward_batched(Xd, Wd, tau_dev(taus), q)
    torch.cuda.synchronize()
    for x in range(3):
        Ybr = O.row_typed_forward(X.f64, W.f64, taus[x], q)
        assert_groups(rel_frob_col_groups(to_f64(Yb[x]), Ybr, q), BF16_TOL, f"Y expert {x}")
    say(f"    max rel err {e:.2e}")


def test_dw_split_then_smaller_problem_on_one_workspace():
    """Two split dW calls in a row on one workspace, the second smaller (fewer rows and types): the
    second result must not depend on the first call's partials left in the scratch."""
    torch = torch_cuda()
    big, small = (4096, 2048, 2048, 8), (2048, 1024, 1024, 4)
    ws = Q.workspace(big[3], big[0], dw_shape=(big[1], big[2]))
    for (M, K, N, q) in (big, small):
        say(f"[dw split reuse] M={M} K={K} N={N} q={q}")
        X, _, dY = _inputs(M, K, N, "bf16", 7400 + M)
        tau = make_tau("cyclic", M, q, offset=1)
        dW = Q.qalg_backward_dw(to_dev(X), to_dev(dY), tau_dev(tau), q, ws=ws)
        torch.cuda.synchronize()
        _, dWr = O.row_typed_backward(X.f64, np.zeros((K, N)), dY.f64, tau, q)
        assert_groups(rel_frob_blocks(to_f64(dW), dWr, q), BF16_TOL, "dW")
