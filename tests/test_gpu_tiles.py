"""Tile heights of the persistent forward (few rows per type) against the oracle.

Every tile height the shape admits (QALG_FLAG_TILE_M64 / M128 / M256) and the
default choice must give the oracle's result within the bf16 bar, bitwise
reproducibly, on cyclic, offset and listed schedules with ragged types.
"""
import numpy as np
import pytest

import gemm_qalg_forward_amd as Q
import synth
from gpu_common import make_tau, say, tau_dev, to_dev, to_f64, torch_cuda
from oracle import qalg_oracle as O
from qalg_check import BF16_TOL, assert_groups, forward_elementwise, rel_frob_col_groups

pytestmark = pytest.mark.gpu

TILE_SHAPES = [
    # M, K, N, q, tau kind, offset, bad rows, law L (0: Q_q)
    (2048, 512, 2048, 8, "cyclic", 0, 0, 0),     # 256 rows per type
    (1000, 1024, 4096, 16, "random", 0, 11, 0),  # about 62 rows per type, out-of-range rows
    (600, 256, 1024, 4, "cyclic", 3, 0, 0),      # 150 rows per type, type offset
    (700, 512, 1024, 8, "cyclic", 0, 0, 0),      # N / q = 128: 128- and 256-row tiles only
    (512, 512, 2048, 8, "cyclic", 1, 0, 3),      # the recursive law at 64 rows per type
    (1500, 768, 768, 4, "cyclic", 1, 0, 0),      # N / q = 192: 128 x 192 and 256 x 192 tiles
    (900, 512, 2304, 4, "random", 0, 5, 0),      # N / q = 576 = 3 x 192, listed types, out-of-range rows
]
FLAGS = [("default", 0), ("m64", Q.QALG_FLAG_TILE_M64), ("m128", Q.QALG_FLAG_TILE_M128),
         ("m256", Q.QALG_FLAG_TILE_M256)]


@pytest.mark.parametrize("shape", TILE_SHAPES, ids=[f"M{s[0]}K{s[1]}N{s[2]}q{s[3]}{s[4]}L{s[7]}" for s in TILE_SHAPES])
def test_tile_heights_match_oracle(shape):
    torch = torch_cuda()
    M, K, N, q, kind, off, bad, L = shape
    X = synth.normal_operand(9900 + M, (M, K), 1.0, "bf16")
    W = synth.normal_operand(9950 + M, (K, N), K ** -0.5, "bf16")
    tau = make_tau(kind, M, q, seed=M + 5, offset=off, bad=bad)
    Xd, Wd, td = to_dev(X), to_dev(W), tau_dev(tau)
    ws = Q.workspace(q, M)
    Q.qalg_build_index(td, q, ws=ws)
    law = Q.QALG_FLAG_LAW_TENSOR if L else 0
    table = O.tensor_power_table(L) if L else None
    Yr = O.row_typed_forward(X.f64, W.f64, tau, q, table=table)
    ran = []
    for name, flag in FLAGS:
        fl = flag | law | Q.QALG_FLAG_INDEX_READY
        if name == "m64" and (N // q) % 256:
            with pytest.raises(Q.QalgError):
                Q.qalg_forward(Xd, Wd, td, q, ws=ws, flags=fl)
            continue
        say(f"[tiles] M={M} K={K} N={N} q={q} tau={kind} L={L} tile={name}")
        Y = Q.qalg_forward(Xd, Wd, td, q, ws=ws, flags=fl)
        Y2 = Q.qalg_forward(Xd, Wd, td, q, ws=ws, flags=fl)
        torch.cuda.synchronize()
        assert torch.equal(Y, Y2), f"{name}: not bitwise reproducible"
        e = assert_groups(rel_frob_col_groups(to_f64(Y), Yr, q), BF16_TOL, f"Y ({name})")
        forward_elementwise(to_f64(Y), Yr, X.f64, W.f64, tau, q, "bf16", f"Y ({name})", table=table)
        if bad:
            rows = np.where((tau < 0) | (tau >= q))[0]
            assert np.all(to_f64(Y)[rows] == 0.0)
        ran.append(f"{name} {e:.2e}")
    say("    " + ", ".join(ran))


TWO_STAGE_SHAPES = [
    # E, M, K, N, q, tau kind, bad rows
    (1, 64, 256, 256, 2, "cyclic", 0),
    (1, 777, 192, 320, 8, "random", 13),     # s = 24, r = 40: ragged tiles, out-of-range rows
    (1, 3001, 384, 384, 3, "random", 0),     # odd q, row tiles spanning types in the first stage
    (1, 300, 128, 128, 16, "cyclic", 0),     # s = r = 8
    (1, 5000, 512, 1024, 4, "random", 37),
    (1, 513, 1024, 512, 1, "zeros", 0),      # q = 1: the first stage is the whole product
    (4, 64, 1024, 512, 4, "positions", 0),   # experts: 16 rows per type
    (3, 256, 512, 768, 8, "positions", 3),   # experts: 32 rows per type, out-of-range rows
    (2, 8, 512, 256, 4, "positions", 0),     # a few rows, some types absent
]


@pytest.mark.parametrize("sched", ["two_stage", "masked"])
@pytest.mark.parametrize("shape", TWO_STAGE_SHAPES, ids=[f"E{s[0]}M{s[1]}K{s[2]}N{s[3]}q{s[4]}{s[5]}" for s in TWO_STAGE_SHAPES])
def test_two_stage_forward_matches_oracle(shape, sched):
    """Section 5.3's second schedule (diagonal maps over all rows, then the type-dependent maps,
    one rounding) and the masked few-rows schedule (one tile over all rows, every block read once,
    masked per row) against the oracle (group and per-element bars), bitwise reproducible."""
    torch = torch_cuda()
    E, M, K, N, q, kind, bad = shape
    say(f"[{sched}] E={E} M={M} K={K} N={N} q={q} tau={kind} bad={bad}")
    Xs = [synth.normal_operand(9960 + 7 * e + M, (M, K), 1.0, "bf16") for e in range(E)]
    Ws = [synth.normal_operand(9970 + 7 * e + M, (K, N), K ** -0.5, "bf16") for e in range(E)]
    taus = []
    for e in range(E):
        if kind == "positions":
            t = O.type_schedule(synth.random_positions(9980 + e, M), q)
            if bad:
                t[:bad] = -1
        else:
            t = make_tau(kind, M, q, seed=M + e, bad=bad)
        taus.append(t.astype(np.int32))
    Xd = torch.stack([to_dev(x) for x in Xs])
    Wd = torch.stack([to_dev(w) for w in Ws])
    td = tau_dev(np.stack(taus))
    ws = Q.workspace(q, M, E, two_stage_N=N) if sched == "two_stage" else Q.workspace(q, M, E)
    fl = Q.QALG_FLAG_TWO_STAGE if sched == "two_stage" else Q.QALG_FLAG_MASKED
    Y = torch.full((E, M, N), 5.0, dtype=torch.bfloat16, device="cuda")
    if E == 1:
        Q.qalg_forward(Xd[0], Wd[0], td[0], q, Y=Y[0], ws=ws, flags=fl)
        Y2 = Q.qalg_forward(Xd[0], Wd[0], td[0], q, ws=ws, flags=fl)[None]
        Yf = Q.qalg_forward(Xd[0], Wd[0], td[0], q)[None]
    else:
        Q.qalg_forward_batched(Xd, Wd, td, q, Y=Y, ws=ws, flags=fl)
        Y2 = Q.qalg_forward_batched(Xd, Wd, td, q, ws=ws, flags=fl)
        Yf = Q.qalg_forward_batched(Xd, Wd, td, q)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2), "two-stage forward not bitwise reproducible"
    got, fused = to_f64(Y), to_f64(Yf)
    for e in range(E):
        Yr = O.row_typed_forward(Xs[e].f64, Ws[e].f64, taus[e], q)
        assert_groups(rel_frob_col_groups(got[e], Yr, q), BF16_TOL, f"Y two-stage e={e}")
        forward_elementwise(got[e], Yr, Xs[e].f64, Ws[e].f64, taus[e], q, "bf16", f"Y two-stage e={e}")
        badrows = (taus[e] < 0) | (taus[e] >= q)
        assert not got[e][badrows].any()
        # the fused schedule on the same inputs meets the same per-element bound (the two differ
        # only in the fp32 summation order)
        forward_elementwise(fused[e], Yr, Xs[e].f64, Ws[e].f64, taus[e], q, "bf16", f"Y fused e={e}")
    say("    ok")
