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
