"""qalg_forward_noalloc (the forward with the type index in the library's own
device array, for callers that cannot allocate) against qalg_forward with a
caller workspace: same kernels, so the outputs must be bitwise equal, and both
meet the oracle bar.  Two calls in a row, the second smaller (the array keeps
the first call's index, which the second must not reuse), then a listed
schedule, a cyclic one and out-of-range rows; argument errors on the host."""
import numpy as np
import pytest

import gemm_qalg_forward_amd as Q
import synth
from gpu_common import make_tau, say, tau_dev, to_dev, to_f64, torch_cuda
from oracle import qalg_oracle as O
from qalg_check import BF16_TOL, assert_groups, forward_elementwise, rel_frob_col_groups

pytestmark = pytest.mark.gpu

CALLS = [
    # M, K, N, q, tau kind, offset, bad rows
    (5000, 512, 1024, 4, "random", 0, 37),   # listed schedule, persistent 256x256 forward
    (777, 192, 320, 8, "cyclic", 3, 0),      # smaller, cyclic with an offset: register-staged tiles
    (3, 512, 768, 4, "random", 0, 0),        # small-M weight-streaming path
    (4096, 2048, 2048, 8, "cyclic", 0, 0),   # larger again
]


def test_noalloc_forward_matches_workspace_forward():
    torch = torch_cuda()
    for k, (M, K, N, q, kind, off, bad) in enumerate(CALLS):
        say(f"[no-alloc] call {k}: M={M} K={K} N={N} q={q} tau={kind} offset={off} bad={bad}")
        X = synth.normal_operand(8800 + M, (M, K), 1.0, "bf16")
        W = synth.normal_operand(8900 + M, (K, N), K ** -0.5, "bf16")
        tau = make_tau(kind, M, q, seed=M + 5, offset=off, bad=bad)
        Xd, Wd, td = to_dev(X), to_dev(W), tau_dev(tau)
        Yn = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
        Q.qalg_forward_noalloc(Xd, Wd, td, q, Yn)
        Yw = Q.qalg_forward(Xd, Wd, td, q, ws=Q.workspace(q, M))
        torch.cuda.synchronize()
        assert torch.equal(Yn, Yw), f"call {k}: no-alloc output differs from the workspace forward"
        Yr = O.row_typed_forward(X.f64, W.f64, tau, q)
        e = assert_groups(rel_frob_col_groups(to_f64(Yn), Yr, q), BF16_TOL, f"Y call {k}")
        forward_elementwise(to_f64(Yn), Yr, X.f64, W.f64, tau, q, "bf16", f"Y call {k}")
        say(f"    bitwise equal to the workspace forward; max rel err {e:.2e}")


def test_noalloc_argument_errors():
    torch = torch_cuda()
    M, K, N, q = 64, 256, 256, 2
    X = torch.zeros(M, K, dtype=torch.bfloat16, device="cuda")
    W = torch.zeros(K, N, dtype=torch.bfloat16, device="cuda")
    tau = torch.zeros(M, dtype=torch.int32, device="cuda")
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(Q.QalgError, match="QALG_ERR_ARG"):
        Q.qalg_forward_noalloc(X, W, tau, q, Y, flags=Q.QALG_FLAG_INDEX_READY)
    with pytest.raises(Q.QalgError, match="QALG_ERR_Q"):
        Q.qalg_forward_noalloc(X, W, tau, 3, Y)
    # an index larger than the library's array: refused on the host, nothing launched
    big = (Q.QALG_NOALLOC_SCRATCH_BYTES // 4) + 1024
    st = Q.lib().qalg_forward_noalloc(X.data_ptr(), W.data_ptr(), tau.data_ptr(), q, big, K, N, Y.data_ptr(),
                                      Q.QALG_BF16, 0, None)
    assert st == 6, Q.qalg_status_string(st)
    # M = 0: nothing to do
    assert Q.lib().qalg_forward_noalloc(None, None, None, q, 0, K, N, None, Q.QALG_BF16, 0, None) == 0
    torch.cuda.synchronize()
