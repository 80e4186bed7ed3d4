"""Parity at the full workload sizes, in the launch configuration the benchmark times.

Each workload's outputs are compared with the fp64 oracle on sampled rows (a
row's output depends only on that row, so the oracle evaluates the sampled
rows alone) or, where it finishes in seconds, on the whole output.  The bar is
the relative Frobenius error per output group: 5e-3 for bf16, 1e-5 for fp32.

Workloads:
  * Q_2 row-typed forward in fp32, M=64, K=N=256 (whole output, dX and dW too)
  * ~110M-LM FFN shapes, bf16, q=4: 768->3072 and 3072->768, M=8192
  * dense FFN (4096, 12288), bf16, q=8, M=16384: up and down projections (whole output)
  * narrow expert shapes, bf16, 64 experts: (7168,2048) q=4, (2048,768) q=4 and q=8
  * training gradients at (4096, 12288), q=8, M=16384: forward, dX and dW (whole outputs)
  * the graph law Q_G and unequal group widths at (4096, 12288), M=16384: forward, dX, dW
"""
import numpy as np
import pytest

import gemm_qalg_forward_amd as Q
import synth
from gpu_common import say, tau_dev, to_dev, to_f64, torch_cuda
from oracle import qalg_oracle as O
from qalg_check import (BF16_TOL, F32_TOL, GATED_STEP_TOL as STEP_TOL, assert_groups, backward_elementwise,
                        forward_elementwise, rel_frob_blocks, rel_frob_col_groups)

pytestmark = pytest.mark.gpu


def _sample_rows(M, q, n, seed):
    """n rows spread over all types, plus the first and last row."""
    g = np.random.Generator(np.random.PCG64(seed))
    pick = g.choice(M, size=min(n, M), replace=False)
    return np.unique(np.concatenate([pick, [0, M - 1]]))


def _sampled_forward_check(X, W, tau, q, Yd, rows, what):
    Yr = O.row_typed_forward(X.f64[rows], W.f64, tau[rows], q)
    got = to_f64(Yd[rows])
    forward_elementwise(got, Yr, X.f64[rows], W.f64, tau[rows], q, "bf16", what)
    return assert_groups(rel_frob_col_groups(got, Yr, q), BF16_TOL, what)


def test_q2_fp32_whole_output():
    torch = torch_cuda()
    c, M, K, N, q = 1, 64, 256, 256, 2
    say(f"[workload] Q_2 fp32 M={M} K={K} N={N}")
    X = synth.normal_operand(synth.seed_for(c, "X"), (M, K), 1.0, "f32")
    W = synth.normal_operand(synth.seed_for(c, "W"), (K, N), K ** -0.5, "f32")
    dY = synth.normal_operand(synth.seed_for(c, "dY"), (M, N), 1.0, "f32")
    tau = O.type_schedule(synth.cyclic_positions(M), q)
    Xd, Wd, dYd, td = to_dev(X), to_dev(W), to_dev(dY), tau_dev(tau)
    ws = Q.workspace(q, M)
    Q.qalg_build_index(td, q, ws=ws)
    r = Q.QALG_FLAG_INDEX_READY
    Y = Q.qalg_forward(Xd, Wd, td, q, ws=ws, flags=r)
    dX = Q.qalg_backward_dx(dYd, Wd, td, q, ws=ws, flags=r)
    dW = Q.qalg_backward_dw(Xd, dYd, td, q, ws=ws, flags=r)
    torch.cuda.synchronize()
    Yr = O.row_typed_forward(X.f64, W.f64, tau, q)
    dXr, dWr = O.row_typed_backward(X.f64, W.f64, dY.f64, tau, q)
    assert_groups(rel_frob_col_groups(to_f64(Y), Yr, q), F32_TOL, "Y")
    assert_groups(rel_frob_col_groups(to_f64(dX), dXr, q), F32_TOL, "dX")
    assert_groups(rel_frob_blocks(to_f64(dW), dWr, q), F32_TOL, "dW")
    forward_elementwise(to_f64(Y), Yr, X.f64, W.f64, tau, q, "f32", "Y")
    backward_elementwise(to_f64(dX), dXr, to_f64(dW), dWr, X.f64, W.f64, dY.f64, tau, q, "f32")
    # 6 of the 8 block products of the square form are used by the two row types
    assert O.mac_count(tau, q, K, N)[0] == 6


@pytest.mark.parametrize("K,N", [(768, 3072), (3072, 768)], ids=["up", "down"])
def test_lm_ffn_q4_whole_output(K, N):
    torch = torch_cuda()
    c, M, q = 2, 8192, 4
    say(f"[workload] 110M-LM FFN bf16 q=4 M={M} {K}->{N}")
    X = synth.normal_operand(synth.seed_for(c, "X") + (10 if K > N else 0), (M, K), 1.0, "bf16")
    W = synth.normal_operand(synth.seed_for(c, "W") + (10 if K > N else 0), (K, N), K ** -0.5, "bf16")
    tau = O.type_schedule(synth.cyclic_positions(M, seq_len=1024), q)
    Xd, Wd, td = to_dev(X), to_dev(W), tau_dev(tau)
    ws = Q.workspace(q, M)
    Q.qalg_build_index(td, q, ws=ws)
    Y = Q.qalg_forward(Xd, Wd, td, q, ws=ws, flags=Q.QALG_FLAG_INDEX_READY)
    torch.cuda.synchronize()
    Yr = O.row_typed_forward(X.f64, W.f64, tau, q)
    e = assert_groups(rel_frob_col_groups(to_f64(Y), Yr, q), BF16_TOL, "Y")
    r = forward_elementwise(to_f64(Y), Yr, X.f64, W.f64, tau, q, "bf16", "Y")
    say(f"    max rel err {e:.2e}; per-element error / bound {r:.2f}")


@pytest.mark.parametrize("proj", ["up", "down"])
def test_dense_ffn_q8_whole_output(proj):
    """The benchmark's workload: same seeds, same calls (schedule, index, forward with the index
    ready); every output element against the oracle (per group and per element)."""
    torch = torch_cuda()
    c, M, D, F, q = 3, 16384, 4096, 12288, 8
    K, N = (D, F) if proj == "up" else (F, D)
    off = 0 if proj == "up" else 10
    say(f"[workload] dense FFN bf16 q=8 M={M} {K}->{N}")
    X = synth.normal_operand(1000 * c + 1 + off, (M, K), 1.0, "bf16")
    W = synth.normal_operand(1000 * c + 2 + off, (K, N), K ** -0.5, "bf16")
    pos = torch.from_numpy(synth.cyclic_positions(M)).to("cuda")
    td = Q.qalg_type_schedule(pos, q)
    ws = Q.workspace(q, M)
    Q.qalg_build_index(td, q, ws=ws)
    Xd, Wd = to_dev(X), to_dev(W)
    Y = Q.qalg_forward(Xd, Wd, td, q, ws=ws, flags=Q.QALG_FLAG_INDEX_READY)
    torch.cuda.synchronize()
    tau = td.cpu().numpy()
    np.testing.assert_array_equal(tau, np.arange(M) % q)
    Yr = O.row_typed_forward(X.f64, W.f64, tau, q)
    got = to_f64(Y)
    e = assert_groups(rel_frob_col_groups(got, Yr, q), BF16_TOL, f"Y {proj}")
    r = forward_elementwise(got, Yr, X.f64, W.f64, tau, q, "bf16", f"Y {proj}")
    say(f"    max rel err over all {M} rows {e:.2e}; per-element error / bound {r:.2f}")
    del Yr, got
    # a second launch on the same inputs is bitwise identical
    Y2 = Q.qalg_forward(Xd, Wd, td, q, ws=ws, flags=Q.QALG_FLAG_INDEX_READY)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2)


_EXPERT_BANKS = {}


def _expert_banks(K, N, E, c=4):
    """The E experts' weight banks (host operands and one device tensor), drawn once per shape."""
    key = (K, N, E)
    if key not in _EXPERT_BANKS:
        from concurrent.futures import ThreadPoolExecutor
        torch = torch_cuda()
        with ThreadPoolExecutor(max_workers=8) as ex:
            Ws = list(ex.map(lambda e: synth.normal_operand(1000 * c + 100 + e, (K, N), K ** -0.5, "bf16"), range(E)))
        Wd = torch.empty((E, K, N), dtype=torch.bfloat16, device="cuda")
        for e in range(E):
            Wd[e].copy_(to_dev(Ws[e]))
        _EXPERT_BANKS.clear()
        _EXPERT_BANKS[key] = (Ws, Wd)
    return _EXPERT_BANKS[key]


@pytest.mark.parametrize("K,N,q", [(7168, 2048, 4), (2048, 768, 4), (2048, 768, 8)])
@pytest.mark.parametrize("M", [1, 8, 64, 256, 1024])
def test_experts_sampled(K, N, q, M):
    torch = torch_cuda()
    c, E = 4, 64
    say(f"[workload] experts E={E} M={M} {K}->{N} q={q}")
    Ws, Wd = _expert_banks(K, N, E, c)
    Xs = [synth.normal_operand(1000 * c + 300 + e, (M, K), 1.0, "bf16") for e in range(E)]
    taus = np.stack([O.type_schedule(synth.random_positions(1000 * c + 200 + e, M), q) for e in range(E)])
    Xd = torch.stack([to_dev(x) for x in Xs])
    Y = Q.qalg_forward_batched(Xd, Wd, tau_dev(taus), q)
    torch.cuda.synchronize()
    # oracle on a few experts, a sample of rows each
    for e in (0, 17, 63):
        rows = _sample_rows(M, q, 64, e)
        _sampled_forward_check(Xs[e], Ws[e], taus[e], q, Y[e], rows, f"expert {e}")


def test_training_grads_q8():
    torch = torch_cuda()
    c, M, K, N, q = 5, 16384, 4096, 12288, 8
    say(f"[workload] training q=8 M={M} {K}->{N}: forward, dX, dW")
    X = synth.normal_operand(synth.seed_for(c, "X"), (M, K), 1.0, "bf16")
    W = synth.normal_operand(synth.seed_for(c, "W"), (K, N), K ** -0.5, "bf16")
    dY = synth.normal_operand(synth.seed_for(c, "dY"), (M, N), 1.0, "bf16")
    tau = (np.arange(M) % q).astype(np.int32)
    Xd, Wd, dYd, td = to_dev(X), to_dev(W), to_dev(dY), tau_dev(tau)
    # the benchmark's launch configuration: the workspace carries the dW scratch,
    # so dW splits the contraction of its diagonal tiles
    ws = Q.workspace(q, M, dw_shape=(K, N))
    Q.qalg_build_index(td, q, ws=ws)
    r = Q.QALG_FLAG_INDEX_READY
    Y = Q.qalg_forward(Xd, Wd, td, q, ws=ws, flags=r)
    dX = Q.qalg_backward_dx(dYd, Wd, td, q, ws=ws, flags=r)
    dW = Q.qalg_backward_dw(Xd, dYd, td, q, ws=ws, flags=r)
    # and without the scratch (one workgroup per diagonal tile)
    ws0 = Q.workspace(q, M)
    dW0 = Q.qalg_backward_dw(Xd, dYd, td, q, ws=ws0)
    torch.cuda.synchronize()
    # every element of Y, dX and dW against the oracle (fp64 block GEMMs)
    Yr = O.row_typed_forward(X.f64, W.f64, tau, q)
    ey = assert_groups(rel_frob_col_groups(to_f64(Y), Yr, q), BF16_TOL, "Y")
    forward_elementwise(to_f64(Y), Yr, X.f64, W.f64, tau, q, "bf16", "Y")
    del Yr
    dXr, dWr = O.row_typed_backward(X.f64, W.f64, dY.f64, tau, q)
    ex = assert_groups(rel_frob_col_groups(to_f64(dX), dXr, q), BF16_TOL, "dX")
    e = assert_groups(rel_frob_blocks(to_f64(dW), dWr, q), BF16_TOL, "dW")
    e0 = assert_groups(rel_frob_blocks(to_f64(dW0), dWr, q), BF16_TOL, "dW unsplit")
    mdX, mdW = O.row_typed_backward(np.abs(X.f64), np.abs(W.f64), np.abs(dY.f64), tau, q)
    from qalg_check import assert_elementwise
    assert_elementwise(to_f64(dX), dXr, mdX, N, "bf16", "dX")
    assert_elementwise(to_f64(dW), dWr, mdW, M, "bf16", "dW")
    assert_elementwise(to_f64(dW0), dWr, mdW, M, "bf16", "dW unsplit")
    say(f"    max rel err over every element: Y {ey:.2e}, dX {ex:.2e}, dW {e:.2e} (unsplit {e0:.2e})")


def test_gated_ffn_q8_sampled():
    """The benchmark's gated FFN leg: same seeds and calls (merge once, gated gate/up, down)."""
    torch = torch_cuda()
    c, M, D, F, q = 6, 16384, 4096, 12288, 8
    say(f"[workload] gated FFN bf16 q=8 M={M} {D}->{F}->{D}")
    X = synth.normal_operand(1000 * c + 1, (M, D), 1.0, "bf16")
    Wg = synth.normal_operand(1000 * c + 2, (D, F), D ** -0.5, "bf16")
    Wu = synth.normal_operand(1000 * c + 3, (D, F), D ** -0.5, "bf16")
    Wd = synth.normal_operand(1000 * c + 4, (F, D), F ** -0.5, "bf16")
    pos = torch.from_numpy(synth.cyclic_positions(M)).to("cuda")
    td = Q.qalg_type_schedule(pos, q)
    ws = Q.workspace(q, M)
    Q.qalg_build_index(td, q, ws=ws)
    Wgu = Q.qalg_merge_gate_up(to_dev(Wg), to_dev(Wu), q)
    r = Q.QALG_FLAG_INDEX_READY
    H = Q.qalg_gated_forward(to_dev(X), Wgu, td, q, ws=ws, flags=r)
    Y = Q.qalg_forward(H, to_dev(Wd), td, q, ws=ws, flags=r)
    torch.cuda.synchronize()
    tau = td.cpu().numpy()
    rows = _sample_rows(M, q, 512, 61)
    Hr = O.gated_forward(X.f64[rows], Wg.f64, Wu.f64, tau[rows], q)
    e1 = assert_groups(rel_frob_col_groups(to_f64(H[rows]), Hr, q), BF16_TOL, "H")
    # the down projection consumes the GPU's bf16 H; the reference uses the exact H
    Yr = O.row_typed_forward(Hr, Wd.f64, tau[rows], q)
    e2 = assert_groups(rel_frob_col_groups(to_f64(Y[rows]), Yr, q), BF16_TOL, "Y")
    say(f"    max rel err over {rows.size} sampled rows: H {e1:.2e}, Y {e2:.2e}")


def test_gated_ffn_training_q8_sampled():
    """The benchmark's gated FFN training step at full size (same seeds and calls).  Y and dX on
    sampled rows (row-local in the oracle); dW on one column per group (q columns keep the group
    structure, so the oracle's table-driven VJP on the column subset is the subset of the full VJP)."""
    torch = torch_cuda()
    c, M, D, F, q = 6, 16384, 4096, 12288, 8
    say(f"[workload] gated FFN training bf16 q=8 M={M} {D}->{F}->{D}")
    X = synth.normal_operand(1000 * c + 1, (M, D), 1.0, "bf16")
    Wg = synth.normal_operand(1000 * c + 2, (D, F), D ** -0.5, "bf16")
    Wu = synth.normal_operand(1000 * c + 3, (D, F), D ** -0.5, "bf16")
    Wd = synth.normal_operand(1000 * c + 4, (F, D), F ** -0.5, "bf16")
    dY = synth.normal_operand(1000 * c + 5, (M, D), 1.0, "bf16")
    pos = torch.from_numpy(synth.cyclic_positions(M)).to("cuda")
    td = Q.qalg_type_schedule(pos, q)
    ws = Q.workspace(q, M, dw_shape=(D, 2 * F))  # as the benchmark: dW may split its diagonal tiles
    Q.qalg_build_index(td, q, ws=ws)
    r = Q.QALG_FLAG_INDEX_READY
    Xd, Wdd, dYd = to_dev(X), to_dev(Wd), to_dev(dY)
    Wgu = Q.qalg_merge_gate_up(to_dev(Wg), to_dev(Wu), q)
    H, GU = Q.qalg_gated_forward_keep(Xd, Wgu, td, q, ws=ws, flags=r)   # as the benchmark's step
    Y = Q.qalg_forward(H, Wdd, td, q, ws=ws, flags=r)
    dH = Q.qalg_backward_dx(dYd, Wdd, td, q, ws=ws, flags=r)
    dWd = Q.qalg_backward_dw(H, dYd, td, q, ws=ws, flags=r)
    dGU = Q.qalg_swiglu_backward(GU, dH, q)
    dX = Q.qalg_backward_dx(dGU, Wgu, td, q, ws=ws, flags=r)
    dWgu = Q.qalg_backward_dw(Xd, dGU, td, q, ws=ws, flags=r)
    dWg, dWu = Q.qalg_split_gate_up(dWgu, q)
    torch.cuda.synchronize()
    tau = td.cpu().numpy()
    # rows: Y and dX
    rows = _sample_rows(M, q, 256, 67)
    Yr, _ = O.gated_ffn_forward(X.f64[rows], Wg.f64, Wu.f64, Wd.f64, tau[rows], q)
    e = {"Y": assert_groups(rel_frob_col_groups(to_f64(Y[rows]), Yr, q), STEP_TOL, "Y")}
    dXr = O.gated_ffn_backward(X.f64[rows], Wg.f64, Wu.f64, Wd.f64, dY.f64[rows], tau[rows], q)[0]
    e["dX"] = assert_groups(rel_frob_col_groups(to_f64(dX[rows]), dXr, q), STEP_TOL, "dX")
    # columns: one per output group of each bank
    cf = np.array([j * (F // q) + 37 for j in range(q)])   # F-side columns (gate/up outputs, down inputs)
    cd = np.array([j * (D // q) + 5 for j in range(q)])    # D-side columns (down outputs)
    G_all = O.row_typed_forward(X.f64, Wg.f64, tau, q)
    U_all = O.row_typed_forward(X.f64, Wu.f64, tau, q)
    H_all = O.swiglu(G_all, U_all)
    dWd_r = O.row_typed_backward(H_all, Wd.f64[:, cd], dY.f64[:, cd], tau, q)[1]
    e["dW_down"] = assert_groups(rel_frob_blocks(to_f64(dWd[:, cd]), dWd_r, q), STEP_TOL, "dW_down")
    # dH on the down projection's input columns cf (all rows), then the SwiGLU VJP there
    dH_cf = O.row_typed_backward(H_all[:, cf], Wd.f64[cf], dY.f64, tau, q)[0]
    dG_cf, dU_cf = O.swiglu_backward(G_all[:, cf], U_all[:, cf], dH_cf)
    dWg_r = O.row_typed_backward(X.f64, Wg.f64[:, cf], dG_cf, tau, q)[1]
    dWu_r = O.row_typed_backward(X.f64, Wu.f64[:, cf], dU_cf, tau, q)[1]
    e["dW_gate"] = assert_groups(rel_frob_blocks(to_f64(dWg[:, cf]), dWg_r, q), STEP_TOL, "dW_gate")
    e["dW_up"] = assert_groups(rel_frob_blocks(to_f64(dWu[:, cf]), dWu_r, q), STEP_TOL, "dW_up")
    say("    " + ", ".join(f"{k} {v:.2e}" for k, v in e.items()))


def test_pilot_law_ffn_sampled():
    """The benchmark's pilot FFN leg under Q_2^(x)2 (same seeds, schedule and calls): fused gate/up
    then down, both with the recursive law; H and Y checked on sampled rows."""
    torch = torch_cuda()
    c, M, D, F, q, L = 7, 61440, 768, 1536, 4, 2
    say(f"[workload] pilot FFN Q_2^2 bf16 M={M} {D}->{F}->{D}, interval schedule")
    X = synth.normal_operand(1000 * c + 1, (M, D), 1.0, "bf16")
    Wg = synth.normal_operand(1000 * c + 2, (D, F), D ** -0.5, "bf16")
    Wu = synth.normal_operand(1000 * c + 3, (D, F), D ** -0.5, "bf16")
    Wd = synth.normal_operand(1000 * c + 4, (F, D), F ** -0.5, "bf16")
    positions = synth.cyclic_positions(M, 1536)
    td = Q.qalg_type_schedule(torch.from_numpy(positions).to("cuda"), q, Q.QALG_SCHEDULE_INTERVAL, 768)
    ws = Q.workspace(q, M)
    Q.qalg_build_index(td, q, ws=ws)
    fl = Q.QALG_FLAG_LAW_TENSOR | Q.QALG_FLAG_INDEX_READY
    Wgu = Q.qalg_merge_gate_up(to_dev(Wg), to_dev(Wu), q)
    H = Q.qalg_gated_forward(to_dev(X), Wgu, td, q, ws=ws, flags=fl)
    Y = Q.qalg_forward(H, to_dev(Wd), td, q, ws=ws, flags=fl)
    torch.cuda.synchronize()
    tau = td.cpu().numpy()
    np.testing.assert_array_equal(tau, O.type_schedule(positions, q, "interval", 768))
    table = O.tensor_power_table(L)
    rows = _sample_rows(M, q, 512, 71)
    Hr = O.gated_forward(X.f64[rows], Wg.f64, Wu.f64, tau[rows], q, table=table)
    e1 = assert_groups(rel_frob_col_groups(to_f64(H[rows]), Hr, q), BF16_TOL, "H")
    Yr = O.row_typed_forward(Hr, Wd.f64, tau[rows], q, table=table)
    e2 = assert_groups(rel_frob_col_groups(to_f64(Y[rows]), Yr, q), BF16_TOL, "Y")
    say(f"    max rel err over {rows.size} sampled rows: H {e1:.2e}, Y {e2:.2e}")


@pytest.mark.parametrize("direction", ["up", "down"])
def test_few_rows_q32_sampled(direction):
    """The benchmark's few-rows leg at the Qwen3-8B shape (q = 32, M = 2048, 64 rows per type;
    same seeds): the default (calibrated) tile choice on sampled rows."""
    torch = torch_cuda()
    c, M, q = 8, 2048, 32
    K, N = (4096, 12288) if direction == "up" else (12288, 4096)
    say(f"[workload] few rows per type: bf16 q={q} M={M} {K}->{N}")
    X = synth.normal_operand(1000 * c + 1, (M, K), 1.0, "bf16")
    W = synth.normal_operand(1000 * c + 2, (K, N), K ** -0.5, "bf16")
    tau = (np.arange(M) % q).astype(np.int32)
    Y = Q.qalg_forward(to_dev(X), to_dev(W), tau_dev(tau), q)
    torch.cuda.synchronize()
    rows = _sample_rows(M, q, 256, 73)
    e = _sampled_forward_check(X, W, tau, q, Y, rows, "Y")
    say(f"    max rel err over {rows.size} sampled rows: {e:.2e}")


@pytest.mark.parametrize("law", [0, 2])
def test_attention_bench_shape_sampled_heads(law):
    """The benchmark's attention leg (32 query heads over 8 key/value heads, S = 4096, d = 128,
    q = 4; same seeds): three query heads against the oracle, whole sequences."""
    torch = torch_cuda()
    c, Hq, Hkv, S, d, q = 9, 32, 8, 4096, 128, 4
    say(f"[workload] attention Hq={Hq} Hkv={Hkv} S={S} d={d} q={q} L={law}")
    Qo = synth.normal_operand(1000 * c + 1, (Hq, S, d), 1.0, "bf16")
    Ko = synth.normal_operand(1000 * c + 2, (Hkv, S, d), 1.0, "bf16")
    Vo = synth.normal_operand(1000 * c + 3, (Hkv, S, d), 1.0, "bf16")
    flags = Q.QALG_FLAG_LAW_TENSOR if law else 0
    Og = Q.qalg_attention_forward(to_dev(Qo), to_dev(Ko), to_dev(Vo), q, flags=flags)
    torch.cuda.synchronize()
    tau = np.arange(S) % q
    heads = [0, 13, 31]
    got = to_f64(Og[heads])
    kv = [h // (Hq // Hkv) for h in heads]
    Or = O.algebraic_attention(Qo.f64[heads], Ko.f64[kv], Vo.f64[kv], tau, q, law)
    errs = [float(np.linalg.norm(got[k] - Or[k]) / np.linalg.norm(Or[k])) for k in range(len(heads))]
    say(f"    max rel err over heads {heads}: {max(errs):.2e}")
    assert max(errs) <= BF16_TOL, errs


def test_graph_law_bench_shape_sampled():
    """The benchmark's graph-law leg: the same seeds, graph and calls (forward, dX, split dW)."""
    torch = torch_cuda()
    c, M, K, N, q = 9, 16384, 4096, 12288, 8
    g = np.random.Generator(np.random.PCG64(1000 * c + 4))
    edges = [(a, b) for a in range(q) for b in range(q) if a != b and g.random() < 0.5]
    say(f"[workload] graph law q={q} M={M} {K}->{N}, {len(edges)} edges: forward, dX, dW")
    masks = [0] * q
    for a, b in edges:
        masks[a] |= 1 << b
    X = synth.normal_operand(1000 * c + 1, (M, K), 1.0, "bf16")
    W = synth.normal_operand(1000 * c + 2, (K, N), K ** -0.5, "bf16")
    dY = synth.normal_operand(1000 * c + 3, (M, N), 1.0, "bf16")
    tau = (np.arange(M) % q).astype(np.int32)
    Xd, Wd, dYd, td = to_dev(X), to_dev(W), to_dev(dY), tau_dev(tau)
    adj = torch.tensor(masks, dtype=torch.int64, device="cuda")
    ws = Q.workspace(q, M, dw_shape=(K, N))
    Q.qalg_build_index(td, q, ws=ws)
    r = Q.QALG_FLAG_INDEX_READY
    Y = Q.qalg_forward_graph(Xd, Wd, td, q, adj, ws=ws, flags=r)
    dX = Q.qalg_backward_dx_graph(dYd, Wd, td, q, adj, ws=ws, flags=r)
    dW = Q.qalg_backward_dw_graph(Xd, dYd, td, q, adj, ws=ws, flags=r)
    torch.cuda.synchronize()
    rows = _sample_rows(M, q, 512, 9)
    Yr = O.row_typed_forward(X.f64[rows], W.f64, tau[rows], q, edges=edges)
    assert_groups(rel_frob_col_groups(to_f64(Y[rows]), Yr, q), BF16_TOL, "Y")
    dXr_s, _ = O.row_typed_backward(X.f64[rows], W.f64, dY.f64[rows], tau[rows], q, edges=edges)
    assert_groups(rel_frob_col_groups(to_f64(dX[rows]), dXr_s, q), BF16_TOL, "dX")
    _, dWr = O.row_typed_backward(X.f64, W.f64, dY.f64, tau, q, edges=edges)
    e = assert_groups(rel_frob_blocks(to_f64(dW), dWr, q), BF16_TOL, "dW")
    say(f"    dW max rel err {e:.2e}")


def test_unequal_widths_bench_shape_sampled():
    """The benchmark's unequal-widths leg: the same seeds, widths and calls (forward, dX, split dW)."""
    torch = torch_cuda()
    c, M, K, N = 10, 16384, 4096, 12288
    kw = [512, 768, 1024, 1792]
    nw = [3 * w for w in kw]
    q = len(kw)
    say(f"[workload] unequal widths q={q} M={M} {K}->{N} {kw}: forward, dX, dW")
    X = synth.normal_operand(1000 * c + 1, (M, K), 1.0, "bf16")
    W = synth.normal_operand(1000 * c + 2, (K, N), K ** -0.5, "bf16")
    dY = synth.normal_operand(1000 * c + 3, (M, N), 1.0, "bf16")
    tau = (np.arange(M) % q).astype(np.int32)
    Xd, Wd, dYd, td = to_dev(X), to_dev(W), to_dev(dY), tau_dev(tau)
    ws = Q.workspace(q, M, dw_shape=(K, N))
    Q.qalg_build_index(td, q, ws=ws)
    r = Q.QALG_FLAG_INDEX_READY
    Y = Q.qalg_forward_widths(Xd, Wd, td, q, kw, nw, ws=ws, flags=r)
    dX = Q.qalg_backward_dx_widths(dYd, Wd, td, q, kw, nw, ws=ws, flags=r)
    dW = Q.qalg_backward_dw_widths(Xd, dYd, td, q, kw, nw, ws=ws, flags=r)
    torch.cuda.synchronize()
    kb = np.concatenate([[0], np.cumsum(kw)])
    nb = np.concatenate([[0], np.cumsum(nw)])
    rows = _sample_rows(M, q, 512, 10)
    Yr = O.row_typed_forward(X.f64[rows], W.f64, tau[rows], q, in_widths=kw, out_widths=nw)
    dXr_s, _ = O.row_typed_backward(X.f64[rows], W.f64, dY.f64[rows], tau[rows], q, in_widths=kw, out_widths=nw)
    _, dWr = O.row_typed_backward(X.f64, W.f64, dY.f64, tau, q, in_widths=kw, out_widths=nw)
    gy, gx, gw = to_f64(Y[rows]), to_f64(dX[rows]), to_f64(dW)
    from qalg_check import _rel
    ey = max(_rel(gy[:, nb[j]:nb[j + 1]], Yr[:, nb[j]:nb[j + 1]]) for j in range(q))
    ex = max(_rel(gx[:, kb[j]:kb[j + 1]], dXr_s[:, kb[j]:kb[j + 1]]) for j in range(q))
    ew = max(_rel(gw[kb[b]:kb[b + 1], nb[j]:nb[j + 1]], dWr[kb[b]:kb[b + 1], nb[j]:nb[j + 1]])
             for b in range(q) for j in range(q))
    say(f"    max rel err Y {ey:.2e}, dX {ex:.2e}, dW {ew:.2e}")
    assert ey <= BF16_TOL and ex <= BF16_TOL and ew <= BF16_TOL


def test_attention_decode_bench_shape_sampled():
    """The benchmark's cached-decoding leg: 32 sequences, 32 query heads over 8 key/value heads,
    d = 128, 4096-slot caches (sequence b holds positions 0..4095-b), q = 4; same seeds and call.
    Four sequences (all query heads) against the oracle."""
    torch = torch_cuda()
    c, B, Hq, Hkv, N, d, q = 11, 32, 32, 8, 4096, 128, 4
    say(f"[workload] attention decode B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} q={q}")
    Qo = synth.normal_operand(1000 * c + 1, (B, Hq, d), 1.0, "bf16")
    Ko = synth.normal_operand(1000 * c + 2, (B, Hkv, N, d), 1.0, "bf16")
    Vo = synth.normal_operand(1000 * c + 3, (B, Hkv, N, d), 1.0, "bf16")
    lens = N - np.arange(B)
    key_pos = np.full((B, N), -1, np.int64)
    for b in range(B):
        key_pos[b, :lens[b]] = np.arange(lens[b])
    q_pos = (lens - 1).astype(np.int64)
    Og = Q.qalg_attention_decode(to_dev(Qo), to_dev(Ko), to_dev(Vo), torch.from_numpy(q_pos).to("cuda"),
                                 torch.from_numpy(key_pos).to("cuda"), q)
    torch.cuda.synchronize()
    got = to_f64(Og)
    seqs = [0, 1, 2, 31]   # query types 3, 2, 1, 0
    Or = O.algebraic_attention_decode(Qo.f64[seqs], Ko.f64[seqs], Vo.f64[seqs], q_pos[seqs], key_pos[seqs], q)
    errs = [float(np.linalg.norm(got[b, h] - Or[k, h]) / np.linalg.norm(Or[k, h]))
            for k, b in enumerate(seqs) for h in range(Hq)]
    say(f"    max rel err over {len(errs)} rows {max(errs):.2e}")
    assert max(errs) <= BF16_TOL, max(errs)
