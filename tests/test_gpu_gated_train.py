"""The gated (SwiGLU) FFN's training step on the GPU against the fp64 oracle.

The step runs through the C ABI on the merged gate/up layout: merged forward
(qalg_forward with N = 2F), qalg_swiglu_forward, the down forward, then the
down projection's dX and dW, qalg_swiglu_backward, and the merged bank's dX and
dW (split back into gate and up banks with qalg_split_gate_up).  The oracle
evaluates the same FFN unmerged (gated_ffn_forward / gated_ffn_backward).
"""
import numpy as np
import pytest

import gemm_qalg_forward_amd as Q
import synth
from gpu_common import make_tau, merge_perm, say, tau_dev, to_dev, to_f64, torch_cuda
from oracle import qalg_oracle as O
from qalg_check import GATED_STEP_TOL as STEP_TOL, assert_groups, rel_frob_blocks, rel_frob_col_groups

pytestmark = pytest.mark.gpu


def _bits(t):
    torch = torch_cuda()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("q,K,F", [(4, 64, 1024), (1, 48, 384), (3, 16, 768)])
def test_split_inverts_merge_bit_exact(q, K, F):
    torch = torch_cuda()
    Wg = synth.normal_operand(9710 + q, (K, F), 1.0, "bf16")
    Wu = synth.normal_operand(9810 + q, (K, F), 1.0, "bf16")
    Wgu = Q.qalg_merge_gate_up(to_dev(Wg), to_dev(Wu), q)
    g, u = Q.qalg_split_gate_up(Wgu, q)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_bits(g), Wg.bits.view(np.uint16))
    np.testing.assert_array_equal(_bits(u), Wu.bits.view(np.uint16))
    # the merged layout itself, from the documented column map
    cat = np.concatenate([Wg.bits.view(np.uint16), Wu.bits.view(np.uint16)], axis=1)
    np.testing.assert_array_equal(_bits(Wgu), cat[:, merge_perm(F, q)])


def _pointwise_inputs(M, F, seed):
    """bf16 pre-activations N(0, 2^2) plus tails and exact zeros, and N(0,1) upstream gradients."""
    GU = synth.normal_operand(seed, (M, 2 * F), 2.0, "bf16")
    dH = synth.normal_operand(seed + 1, (M, F), 1.0, "bf16")
    bits = GU.bits.view(np.uint16).copy()
    special = np.array([0.0, -0.0, 30.0, -30.0, 90.0, -90.0, 1.0, -1.25], dtype=np.float32)
    sb = (special.view(np.uint32) >> 16).astype(np.uint16)   # all exact in bf16
    bits[0, :sb.size] = sb
    bits[1, 64:64 + sb.size] = sb
    return bits, dH


def _from_bits(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("M,F,q", [(257, 1024, 4), (64, 384, 1), (1000, 768, 3)])
def test_swiglu_pointwise_matches_oracle(M, F, q):
    """Elementwise bound: one RNE rounding (2^-9 relative) plus fp32 evaluation error, taken as
    2^-8 |ref| + 2^-20 x (the magnitudes that enter the fp32 products)."""
    torch = torch_cuda()
    say(f"[swiglu] M={M} F={F} q={q}")
    bits, dH = _pointwise_inputs(M, F, 9900 + M)
    GUd = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to("cuda")
    dHd = to_dev(dH)
    H = Q.qalg_swiglu_forward(GUd, q)
    dGU = Q.qalg_swiglu_backward(GUd, dHd, q)
    torch.cuda.synchronize()
    perm = merge_perm(F, q)
    cat = np.empty_like(bits)
    cat[:, perm] = bits                      # merged -> [gate | up]
    G, U = _from_bits(cat[:, :F]), _from_bits(cat[:, F:])
    dh = dH.f64
    Hr = O.swiglu(G, U)
    dGr, dUr = O.swiglu_backward(G, U, dh)
    got = to_f64(dGU)
    dcat = np.empty_like(got)
    dcat[:, perm] = got
    for name, g_, ref, mag in (("H", to_f64(H), Hr, np.abs(G * U)),
                               ("dgate", dcat[:, :F], dGr, np.abs(dh * U) * (1 + np.abs(G))),
                               ("dup", dcat[:, F:], dUr, np.abs(dh * G))):
        err = np.abs(g_ - ref)
        bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -20 * mag
        bad = np.argwhere(err > bound)
        assert bad.size == 0, (name, bad[:5], g_[tuple(bad[0])], ref[tuple(bad[0])])
        big = np.abs(ref) > 1e-3
        say(f"    {name}: max |err| / |ref| over |ref| > 1e-3: {np.max(err[big] / np.abs(ref[big])):.2e}")


TRAIN_SHAPES = [
    # M, D, F, q, tau kind, offset, bad rows
    (2048, 512, 1024, 4, "cyclic", 0, 0),
    (1000, 768, 3072, 4, "cyclic", 3, 0),     # the 110M-LM FFN widths, ragged rows, type offset
    (700, 256, 512, 2, "random", 0, 7),       # listed schedule, out-of-range types
    (512, 256, 512, 1, "zeros", 0, 0),        # q = 1: a dense SwiGLU FFN
]



@pytest.mark.parametrize("shape", TRAIN_SHAPES, ids=[f"M{s[0]}D{s[1]}F{s[2]}q{s[3]}{s[4]}" for s in TRAIN_SHAPES])
def test_gated_ffn_training_step_matches_oracle(shape):
    torch = torch_cuda()
    M, D, F, q, kind, off, bad = shape
    say(f"[gated train] M={M} D={D} F={F} q={q} tau={kind} offset={off} bad={bad}")
    X = synth.normal_operand(9400 + M, (M, D), 1.0, "bf16")
    Wg = synth.normal_operand(9500 + M, (D, F), D ** -0.5, "bf16")
    Wu = synth.normal_operand(9600 + M, (D, F), D ** -0.5, "bf16")
    Wd = synth.normal_operand(9700 + M, (F, D), F ** -0.5, "bf16")
    dY = synth.normal_operand(9800 + M, (M, D), 1.0, "bf16")
    tau = make_tau(kind, M, q, seed=M + 7, offset=off, bad=bad)
    Xd, td, Wdd, dYd = to_dev(X), tau_dev(tau), to_dev(Wd), to_dev(dY)
    Wgu = Q.qalg_merge_gate_up(to_dev(Wg), to_dev(Wu), q)
    ws = Q.workspace(q, M)
    Q.qalg_build_index(td, q, ws=ws)
    r = Q.QALG_FLAG_INDEX_READY
    GU = Q.qalg_forward(Xd, Wgu, td, q, ws=ws, flags=r)
    H = Q.qalg_swiglu_forward(GU, q)
    Y = Q.qalg_forward(H, Wdd, td, q, ws=ws, flags=r)
    dH = Q.qalg_backward_dx(dYd, Wdd, td, q, ws=ws, flags=r)
    dWd = Q.qalg_backward_dw(H, dYd, td, q, ws=ws, flags=r)
    dGU = Q.qalg_swiglu_backward(GU, dH, q)
    dX = Q.qalg_backward_dx(dGU, Wgu, td, q, ws=ws, flags=r)
    dWgu = Q.qalg_backward_dw(Xd, dGU, td, q, ws=ws, flags=r)
    dWg, dWu = Q.qalg_split_gate_up(dWgu, q)
    torch.cuda.synchronize()
    assert Q.qalg_read_status(ws, q, M) == bad
    Yr, _ = O.gated_ffn_forward(X.f64, Wg.f64, Wu.f64, Wd.f64, tau, q)
    dXr, dWgr, dWur, dWdr = O.gated_ffn_backward(X.f64, Wg.f64, Wu.f64, Wd.f64, dY.f64, tau, q)
    errs = {}
    errs["Y"] = assert_groups(rel_frob_col_groups(to_f64(Y), Yr, q), STEP_TOL, "Y")
    errs["dX"] = assert_groups(rel_frob_col_groups(to_f64(dX), dXr, q), STEP_TOL, "dX")
    for name, got, ref in (("dW_gate", dWg, dWgr), ("dW_up", dWu, dWur), ("dW_down", dWd, dWdr)):
        errs[name] = assert_groups(rel_frob_blocks(to_f64(got), ref, q), STEP_TOL, name)
    say("    " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    if bad:
        rows = np.where((tau < 0) | (tau >= q))[0]
        assert np.all(to_f64(Y)[rows] == 0.0) and np.all(to_f64(dX)[rows] == 0.0)


KEEP_SHAPES = [
    # M, K, F, q, tau kind, offset, bad rows, law
    (2048, 512, 1024, 4, "cyclic", 0, 0, "complete"),
    (1000, 768, 3072, 4, "cyclic", 3, 0, "complete"),   # ragged rows, type offset
    (700, 256, 1024, 2, "random", 0, 7, "complete"),    # listed schedule, out-of-range types
    (1536, 768, 1536, 4, "interval", 0, 0, "tensor"),   # the pilot's law and schedule (Q_2^(x)2)
]


@pytest.mark.parametrize("shape", KEEP_SHAPES, ids=[f"M{s[0]}K{s[1]}F{s[2]}q{s[3]}{s[4]}{s[7]}" for s in KEEP_SHAPES])
def test_gated_forward_keep_is_unfused_path_bitwise(shape):
    """qalg_gated_forward_keep's GU and H are bit for bit the merged forward followed by the pointwise
    SwiGLU (same tiles, same fp32 sums, H from the rounded pre-activations)."""
    torch = torch_cuda()
    M, K, F, q, kind, off, bad, law = shape
    say(f"[gated keep] M={M} K={K} F={F} q={q} tau={kind} law={law} bad={bad}")
    X = synth.normal_operand(9450 + M, (M, K), 1.0, "bf16")
    Wg = synth.normal_operand(9550 + M, (K, F), K ** -0.5, "bf16")
    Wu = synth.normal_operand(9650 + M, (K, F), K ** -0.5, "bf16")
    if kind == "interval":
        pos = torch.arange(M, dtype=torch.int64, device="cuda") % 1536
        td = Q.qalg_type_schedule(pos, q, Q.QALG_SCHEDULE_INTERVAL, 768)
        tau = td.cpu().numpy()
    else:
        tau = make_tau(kind, M, q, seed=M + 5, offset=off, bad=bad)
        td = tau_dev(tau)
    fl = Q.QALG_FLAG_LAW_TENSOR if law == "tensor" else 0
    Xd = to_dev(X)
    Wgu = Q.qalg_merge_gate_up(to_dev(Wg), to_dev(Wu), q)
    ws = Q.workspace(q, M)
    # garbage in the outputs first: every element must be written
    H = torch.full((M, F), 7.0, dtype=torch.bfloat16, device="cuda")
    GU = torch.full((M, 2 * F), -3.0, dtype=torch.bfloat16, device="cuda")
    Q.qalg_gated_forward_keep(Xd, Wgu, td, q, H=H, GU=GU, ws=ws, flags=fl)
    GU0 = Q.qalg_forward(Xd, Wgu, td, q, ws=ws, flags=fl | Q.QALG_FLAG_INDEX_READY)
    H0 = Q.qalg_swiglu_forward(GU0, q)
    torch.cuda.synchronize()
    assert torch.equal(GU, GU0), "pre-activations differ from the merged forward"
    assert torch.equal(H, H0), "H differs from the pointwise SwiGLU of the pre-activations"
    if bad:
        rows = np.where((tau < 0) | (tau >= q))[0]
        assert np.all(to_f64(H)[rows] == 0.0) and np.all(to_f64(GU)[rows] == 0.0)
    # and against the oracle: H (rounded pre-activations, then H: the gated step's bar) per group
    table = O.tensor_power_table(int(np.log2(q))) if law == "tensor" else None
    Gr = O.row_typed_forward(X.f64, Wg.f64, tau, q, table=table)
    Ur = O.row_typed_forward(X.f64, Wu.f64, tau, q, table=table)
    e = assert_groups(rel_frob_col_groups(to_f64(H), O.swiglu(Gr, Ur), q), STEP_TOL, "H")
    say(f"    bitwise equal to the unfused path; H max rel err {e:.2e}")
