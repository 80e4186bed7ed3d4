"""The C-ABI library on the CPU: it loads, exports every declared entry point,
and rejects bad arguments before touching the device (no GPU calls here)."""
import ctypes
import pathlib
import re

import pytest

import gemm_qalg_forward_amd as Q

HEADER = pathlib.Path(__file__).resolve().parents[1] / "include" / "qalg.h"


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qalg_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not Q.lib_path.exists():
        pytest.skip("libqalg.so not built")
    return Q.lib()


def test_header_declares_the_projection_api():
    names = declared_functions()
    for n in ("qalg_forward", "qalg_backward_dx", "qalg_backward_dw", "qalg_build_index",
              "qalg_type_schedule", "qalg_forward_batched", "qalg_workspace_bytes", "qalg_read_status"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(declared_functions()) == set(Q._SIGS), "binding and header disagree"


def test_version_and_status_strings(lib):
    assert Q.qalg_version() == 1
    for code in range(9):
        assert Q.qalg_status_string(code).startswith("QALG_")
    assert "unknown" in Q.qalg_status_string(99)


def test_dw_workspace_size(lib):
    for q, M, K, N in ((4, 3072, 768, 1536), (1, 10, 64, 64)):
        base = Q.qalg_workspace_bytes(q, M)
        assert Q.qalg_workspace_bytes_dw(q, M, K, N) == base + 16 * K * N * 4
    assert Q.qalg_workspace_bytes_dw(0, 10, 64, 64) == 0
    assert Q.qalg_workspace_bytes_dw(4, 10, 0, 64) == 0


def test_workspace_layout(lib):
    for q, M in ((1, 0), (2, 64), (8, 16384), (512, 1000)):
        n = Q.qalg_workspace_bytes(q, M)
        assert n % 256 == 0 and n >= 4 * (M + 2 * q)
        lay = Q.qalg_index_layout(q, M)
        assert lay[0] == 0 and lay[1] < lay[2] < lay[3] and lay[3] * 4 + 4 * M <= n
    assert Q.qalg_workspace_bytes(0, 10) == 0
    assert Q.qalg_workspace_bytes(513, 10) == 0
    assert Q.qalg_workspace_bytes(4, -1) == 0


FAKE = 0x10000  # 16-byte aligned non-null address; never dereferenced on these paths


def call_fwd(lib, X=FAKE, W=FAKE, tau=FAKE, q=2, M=64, K=16, N=16, Y=FAKE, dt=1, ws=FAKE,
             wsb=1 << 20, flags=0, fn="qalg_forward"):
    return getattr(lib, fn)(X, W, tau, q, M, K, N, Y, dt, ws, wsb, flags, None)


@pytest.mark.parametrize("fn", ["qalg_forward", "qalg_backward_dx", "qalg_backward_dw"])
def test_argument_errors_are_synchronous(lib, fn):
    assert call_fwd(lib, q=0, fn=fn) == 3
    assert call_fwd(lib, q=3, fn=fn) == 3            # 3 does not divide 16
    assert call_fwd(lib, q=513, K=513 * 8, N=513 * 8, fn=fn) == 3
    assert call_fwd(lib, M=-1, fn=fn) == 2
    assert call_fwd(lib, K=0, fn=fn) == 2
    assert call_fwd(lib, N=-4, fn=fn) == 2
    assert call_fwd(lib, dt=7, fn=fn) == 5
    assert call_fwd(lib, X=None, fn=fn) == 1
    assert call_fwd(lib, tau=None, fn=fn) == 1
    assert call_fwd(lib, Y=None, fn=fn) == 1
    assert call_fwd(lib, ws=None, fn=fn) == 1
    assert call_fwd(lib, X=FAKE + 2, fn=fn) == 4     # misaligned operand
    assert call_fwd(lib, q=4, K=16, N=16, fn=fn) == 4  # bf16 group width 4 < 8
    assert call_fwd(lib, wsb=16, fn=fn) == 6         # workspace too small
    assert call_fwd(lib, ws=FAKE + 4, fn=fn) == 6    # workspace misaligned
    assert call_fwd(lib, flags=64, fn=fn) == 8       # unknown flag
    assert call_fwd(lib, flags=2 | 4, fn=fn) == 8    # contradictory forced paths
    if fn != "qalg_forward":
        assert call_fwd(lib, M=4, flags=4, fn=fn) == 8   # small-M path is forward only
    else:
        assert call_fwd(lib, M=64, flags=4, fn=fn) == 8  # forced small-M path needs M <= 8
        assert call_fwd(lib, M=4, ws=None, fn=fn) == 1   # the workspace is checked on every path


def test_zero_rows_forward_is_a_no_op(lib):
    # M = 0: nothing to compute; no pointer is touched
    assert call_fwd(lib, M=0, X=None, tau=None, Y=None, ws=None) == 0
    assert call_fwd(lib, M=0, X=None, tau=None, Y=None, ws=None, fn="qalg_backward_dx") == 0
    # dW with M = 0 still needs its output (it is zero-filled)
    assert call_fwd(lib, M=0, X=None, tau=None, Y=None, ws=None, fn="qalg_backward_dw") == 1


def test_batched_and_index_errors(lib):
    assert lib.qalg_forward_batched(0, FAKE, FAKE, FAKE, 2, 4, 16, 16, FAKE, 1, FAKE, 1 << 20, 0, None) == 2
    assert lib.qalg_build_index(FAKE, 0, 4, FAKE, 1 << 20, None) == 3
    assert lib.qalg_build_index(None, 2, 4, FAKE, 1 << 20, None) == 1
    assert lib.qalg_build_index(FAKE, 2, 4, FAKE, 8, None) == 6
    assert lib.qalg_build_index_batched(0, FAKE, 2, 4, FAKE, 1 << 20, None) == 2
    assert lib.qalg_type_schedule(FAKE, 4, 2, 9, 0, FAKE, None) == 8
    assert lib.qalg_type_schedule(FAKE, 4, 4, 1, 6, FAKE, None) == 8   # period not a multiple of q
    assert lib.qalg_type_schedule(FAKE, -1, 4, 0, 0, FAKE, None) == 2
    assert lib.qalg_type_schedule(None, 0, 4, 0, 0, None, None) == 0   # M = 0
    out = (ctypes.c_int64 * 4)()
    assert lib.qalg_index_layout(0, 4, out) == 3
    assert lib.qalg_read_status(None, 1, 2, 4, None, None) == 1


def test_binding_refuses_cpu_tensors(lib):
    torch = pytest.importorskip("torch")
    X = torch.zeros(4, 16, dtype=torch.bfloat16)
    W = torch.zeros(16, 16, dtype=torch.bfloat16)
    tau = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        Q.qalg_forward(X, W, tau, 2, Y=torch.empty(4, 16, dtype=torch.bfloat16), ws=torch.empty(4096, dtype=torch.uint8))


def test_binding_checks_caller_outputs_before_any_launch(lib):
    """A caller-supplied output of the wrong shape, dtype or device is refused in
    Python (the library trusts the sizes it is given and would write out of
    bounds); the checks run before any pointer is taken, so CPU tensors suffice."""
    torch = pytest.importorskip("torch")
    bf = torch.bfloat16
    M, K, N, q, F = 4, 16, 16, 2, 256
    X, W, dY = torch.zeros(M, K, dtype=bf), torch.zeros(K, N, dtype=bf), torch.zeros(M, N, dtype=bf)
    tau = torch.zeros(M, dtype=torch.int32)
    ws = torch.empty(4096, dtype=torch.uint8)
    adj = torch.zeros(q, dtype=torch.int64)
    wid = [K // q] * q
    cases = [
        (lambda o: Q.qalg_forward(X, W, tau, q, Y=o, ws=ws), (M, N)),
        (lambda o: Q.qalg_backward_dx(dY, W, tau, q, dX=o, ws=ws), (M, K)),
        (lambda o: Q.qalg_backward_dw(X, dY, tau, q, dW=o, ws=ws), (K, N)),
        (lambda o: Q.qalg_forward_graph(X, W, tau, q, adj, Y=o, ws=ws), (M, N)),
        (lambda o: Q.qalg_backward_dx_graph(dY, W, tau, q, adj, dX=o, ws=ws), (M, K)),
        (lambda o: Q.qalg_backward_dw_graph(X, dY, tau, q, adj, dW=o, ws=ws), (K, N)),
        (lambda o: Q.qalg_forward_widths(X, W, tau, q, wid, wid, Y=o, ws=ws), (M, N)),
        (lambda o: Q.qalg_backward_dx_widths(dY, W, tau, q, wid, wid, dX=o, ws=ws), (M, K)),
        (lambda o: Q.qalg_backward_dw_widths(X, dY, tau, q, wid, wid, dW=o, ws=ws), (K, N)),
        (lambda o: Q.qalg_forward_batched(X[None], W[None], tau[None], q, Y=o, ws=ws), (1, M, N)),
        (lambda o: Q.qalg_gated_forward(X, torch.zeros(K, 2 * F, dtype=bf), tau, q, H=o, ws=ws), (M, F)),
        (lambda o: Q.qalg_gated_forward_keep(X, torch.zeros(K, 2 * F, dtype=bf), tau, q, H=o, ws=ws), (M, F)),
        (lambda o: Q.qalg_gated_forward_keep(X, torch.zeros(K, 2 * F, dtype=bf), tau, q, GU=o, ws=ws), (M, 2 * F)),
        (lambda o: Q.qalg_merge_gate_up(torch.zeros(K, F, dtype=bf), torch.zeros(K, F, dtype=bf), q, Wgu=o), (K, 2 * F)),
        (lambda o: Q.qalg_split_gate_up(torch.zeros(K, 2 * F, dtype=bf), q, Wg=o), (K, F)),
        (lambda o: Q.qalg_swiglu_forward(torch.zeros(M, 2 * F, dtype=bf), q, H=o), (M, F)),
        (lambda o: Q.qalg_swiglu_backward(torch.zeros(M, 2 * F, dtype=bf), torch.zeros(M, F, dtype=bf), q, dGU=o),
         (M, 2 * F)),
        (lambda o: Q.qalg_attention_forward(torch.zeros(2, 8, 64, dtype=bf), torch.zeros(1, 8, 64, dtype=bf),
                                            torch.zeros(1, 8, 64, dtype=bf), 2, O=o), (2, 8, 64)),
    ]
    for call, shape in cases:
        short = (shape[0] - 1,) + tuple(shape[1:])
        with pytest.raises(ValueError, match="shape"):
            call(torch.empty(short, dtype=bf))
        with pytest.raises(TypeError, match="dtype"):
            call(torch.empty(shape, dtype=torch.float32))
        # the right output gets as far as the device check of the inputs
        with pytest.raises(ValueError, match="GPU"):
            call(torch.empty(shape, dtype=bf))
    with pytest.raises(ValueError, match="tau must be int32"):
        Q.qalg_type_schedule(torch.zeros(M, dtype=torch.int64), q, tau=torch.empty(M - 1, dtype=torch.int32))
    with pytest.raises(TypeError, match="share a dtype"):
        Q.qalg_forward_graph(X, W.float(), tau, q, adj, ws=ws)


def call_gated(lib, X=FAKE, W=FAKE, tau=FAKE, q=2, M=64, K=256, F=512, H=FAKE, dt=1, ws=FAKE,
               wsb=1 << 20, flags=0):
    return lib.qalg_gated_forward(X, W, tau, q, M, K, F, H, dt, ws, wsb, flags, None)


def test_gated_argument_errors_are_synchronous(lib):
    assert call_gated(lib, dt=0) == 5                 # bf16 only
    assert call_gated(lib, flags=2) == 8              # only QALG_FLAG_INDEX_READY
    assert call_gated(lib, q=0) == 3
    assert call_gated(lib, q=3) == 3                  # 3 does not divide 256
    assert call_gated(lib, F=384) == 4                # F / q = 192: not a multiple of 128
    assert call_gated(lib, K=128, q=4) == 4           # K / q = 32: not a multiple of 64
    assert call_gated(lib, M=-1) == 2
    assert call_gated(lib, X=None) == 1
    assert call_gated(lib, H=None) == 1
    assert call_gated(lib, ws=None) == 1
    assert call_gated(lib, X=FAKE + 2) == 4
    assert call_gated(lib, wsb=16) == 6               # workspace too small
    assert call_gated(lib, M=0, X=None, H=None) == 0  # no rows: nothing to do, no launch


def call_gated_keep(lib, X=FAKE, W=FAKE, tau=FAKE, q=2, M=64, K=256, F=512, H=FAKE, GU=FAKE, dt=1, ws=FAKE,
                    wsb=1 << 20, flags=0):
    return lib.qalg_gated_forward_keep(X, W, tau, q, M, K, F, H, GU, dt, ws, wsb, flags, None)


def test_gated_keep_argument_errors_are_synchronous(lib):
    """The gated forward that keeps the pre-activations: the gated forward's checks plus its GU."""
    assert call_gated_keep(lib, GU=None) == 1                 # GU is required when there are rows
    assert call_gated_keep(lib, GU=FAKE + 8) == 4             # 16-byte aligned
    assert call_gated_keep(lib, dt=0) == 5
    assert call_gated_keep(lib, F=384) == 4                   # F / q = 192: not a multiple of 128
    assert call_gated_keep(lib, H=None) == 1
    assert call_gated_keep(lib, wsb=16) == 6
    assert call_gated_keep(lib, M=0, X=None, H=None, GU=None) == 0  # no rows: nothing to do, no launch


def test_merge_argument_errors_are_synchronous(lib):
    m = lambda **k: lib.qalg_merge_gate_up(k.get("Wg", FAKE), k.get("Wu", FAKE), k.get("q", 2), k.get("K", 64),  # noqa: E731
                                           k.get("F", 512), k.get("Wgu", FAKE), k.get("dt", 1), None)
    assert m(dt=0) == 5
    assert m(F=384) == 4
    assert m(q=3) == 3
    assert m(K=0) == 2
    assert m(Wu=None) == 1
    assert m(Wgu=FAKE + 4) == 4


def test_split_argument_errors_are_synchronous(lib):
    sp = lambda **k: lib.qalg_split_gate_up(k.get("Wgu", FAKE), k.get("q", 2), k.get("K", 64), k.get("F", 512),  # noqa: E731
                                            k.get("Wg", FAKE), k.get("Wu", FAKE), k.get("dt", 1), None)
    assert sp(dt=0) == 5
    assert sp(F=384) == 4
    assert sp(q=3) == 3
    assert sp(K=0) == 2
    assert sp(Wg=None) == 1
    assert sp(Wu=FAKE + 8) == 4


def test_swiglu_argument_errors_are_synchronous(lib):
    fw = lambda **k: lib.qalg_swiglu_forward(k.get("GU", FAKE), k.get("q", 2), k.get("M", 64), k.get("F", 512),  # noqa: E731
                                             k.get("H", FAKE), k.get("dt", 1), None)
    bw = lambda **k: lib.qalg_swiglu_backward(k.get("GU", FAKE), k.get("dH", FAKE), k.get("q", 2),  # noqa: E731
                                              k.get("M", 64), k.get("F", 512), k.get("dGU", FAKE), k.get("dt", 1), None)
    for f in (fw, bw):
        assert f(dt=0) == 5                 # bf16 only
        assert f(M=-1) == 2
        assert f(F=0) == 2
        assert f(q=0) == 3
        assert f(q=3) == 3                  # 3 does not divide 512
        assert f(F=384) == 4                # F / q = 192: not a multiple of 128
        assert f(GU=None) == 1
        assert f(GU=FAKE + 2) == 4
        assert f(M=0, GU=None) == 0         # no rows: nothing to do, no launch
    assert fw(H=None) == 1
    assert bw(dH=None) == 1
    assert bw(dGU=FAKE + 4) == 4


def test_tensor_law_flag_errors_are_synchronous(lib):
    T = Q.QALG_FLAG_LAW_TENSOR
    fwd = lambda **k: lib.qalg_forward(FAKE, FAKE, FAKE, k.get("q", 4), k.get("M", 64), k.get("K", 256),  # noqa: E731
                                       k.get("N", 512), FAKE, k.get("dt", 1), FAKE, 1 << 20, k.get("flags", T), None)
    assert fwd(q=3, K=192, N=384) == 3            # not a power of two
    assert fwd(q=6, K=384, N=768) == 3
    assert fwd(dt=0) == 8                          # bf16 only
    assert fwd(flags=T | Q.QALG_FLAG_FORCE_TILED) == 8
    assert fwd(flags=T | Q.QALG_FLAG_FORCE_SMALL_M) == 8
    assert fwd(K=128) == 4                         # K / q = 32: not a multiple of 64
    assert fwd(N=320) == 4                         # N / q = 80: no tile width divides it
    assert fwd(flags=512) == 8                     # unknown flag
    # dX and dW accept the law (bf16, one bank); the checks still come first
    dx = lib.qalg_backward_dx(FAKE, FAKE, FAKE, 6, 64, 384, 768, FAKE, 1, FAKE, 1 << 20, T, None)
    dw = lib.qalg_backward_dw(FAKE, FAKE, FAKE, 4, 64, 256, 512, FAKE, 0, FAKE, 1 << 20, T, None)
    bt = lib.qalg_forward_batched(2, FAKE, FAKE, FAKE, 4, 64, 256, 512, FAKE, 1, FAKE, 1 << 20, T, None)
    assert dx == 3 and dw == 8 and bt == 8         # q = 6 not 2^L; fp32; several banks
    assert call_gated(lib, q=3, K=192, F=384, flags=T) == 3


def test_tile_flags_errors_are_synchronous(lib):
    fwd = lambda **k: lib.qalg_forward(FAKE, FAKE, FAKE, k.get("q", 4), k.get("M", 64), k.get("K", 256),  # noqa: E731
                                       k.get("N", 1024), FAKE, k.get("dt", 1), FAKE, 1 << 20, k.get("flags", 0), None)
    assert fwd(flags=Q.QALG_FLAG_TILE_M64 | Q.QALG_FLAG_TILE_M128) == 8    # one height at most
    assert fwd(flags=Q.QALG_FLAG_TILE_M64, dt=0) == 8                      # bf16 only
    assert fwd(flags=Q.QALG_FLAG_TILE_M64 | Q.QALG_FLAG_FORCE_TILED) == 8
    assert fwd(flags=Q.QALG_FLAG_TILE_M64, N=512) == 8                     # N / q = 128: no 64-row tiles
    assert fwd(flags=Q.QALG_FLAG_TILE_M128, N=640) == 8                    # N / q = 160
    assert fwd(flags=Q.QALG_FLAG_TILE_M256, K=128) == 8                    # K / q = 32
    dx = lib.qalg_backward_dx(FAKE, FAKE, FAKE, 4, 64, 256, 1024, FAKE, 1, FAKE, 1 << 20, Q.QALG_FLAG_TILE_M64, None)
    assert dx == 8
    assert fwd(flags=Q.QALG_FLAG_TILE_M64, M=0) == 0                       # no rows: nothing to do


def test_attention_argument_errors_are_synchronous(lib):
    at = lambda **k: lib.qalg_attention_forward(k.get("Qp", FAKE), FAKE, FAKE, k.get("Hq", 4), k.get("Hkv", 2),  # noqa: E731
                                                k.get("S", 64), k.get("d", 128), k.get("q", 4), k.get("O", FAKE),
                                                k.get("dt", 1), k.get("flags", 0), None)
    assert at(dt=0) == 5
    assert at(flags=2) == 8
    assert at(Hkv=3) == 2          # Hkv must divide Hq
    assert at(d=96) == 2           # d is 64 or 128
    assert at(q=3) == 3            # q divides d
    assert at(q=16) == 4           # d / q = 8: not a multiple of 16
    assert at(q=8, d=64) == 4
    assert at(Qp=None) == 1
    assert at(O=FAKE + 4) == 4
    assert at(S=0, Qp=None) == 0   # no positions: nothing to do


def test_graph_argument_errors_are_synchronous(lib):
    """Every graph-law entry point rejects bad arguments before any launch (the pointers are fake)."""
    for fn in ("qalg_forward_graph", "qalg_backward_dx_graph", "qalg_backward_dw_graph"):
        f = getattr(lib, fn)
        g = lambda **k: f(FAKE, FAKE, FAKE, k.get("q", 4), k.get("adj", FAKE), k.get("M", 64),  # noqa: E731
                          k.get("K", 256), k.get("N", 512), k.get("Y", FAKE), k.get("dt", 1),
                          k.get("ws", FAKE), k.get("wsb", 1 << 20), k.get("flags", 0), None)
        assert g(dt=0) == 5, fn
        assert g(flags=Q.QALG_FLAG_LAW_TENSOR) == 8, fn
        assert g(flags=Q.QALG_FLAG_FORCE_TILED) == 8, fn
        assert g(q=65, K=65 * 64, N=65 * 128) == 3, fn   # at most 64 groups (one mask word per type)
        assert g(q=3) == 3, fn                          # 3 divides neither 256 nor 512
        assert g(adj=None) == 1, fn
        assert g(Y=None) == 1, fn
        assert g(adj=FAKE + 4) == 4, fn                 # masks are 8-byte words
        assert g(K=48) == 4, fn                         # K / q = 12: not a multiple of 8
        assert g(M=1 << 20, K=1 << 12) == 2, fn         # M K >= 2^31
        assert g(ws=None) == 1, fn
        assert g(wsb=16) == 6, fn
        assert g(M=-1) == 2, fn
    assert lib.qalg_forward_graph(FAKE, FAKE, FAKE, 4, None, 0, 256, 512, FAKE, 1, FAKE, 0, 0, None) == 0
    assert lib.qalg_backward_dx_graph(FAKE, FAKE, FAKE, 4, None, 0, 256, 512, FAKE, 1, FAKE, 0, 0, None) == 0
    assert lib.qalg_backward_dw_graph(FAKE, FAKE, FAKE, 4, None, 0, 256, 512, None, 1, FAKE, 0, 0, None) == 1


def test_widths_argument_errors_are_synchronous(lib):
    """The unequal-width entry points reject bad arguments before any launch (the pointers are fake)."""
    import ctypes
    arr = lambda *v: (ctypes.c_int64 * len(v))(*v)  # noqa: E731
    for fn in ("qalg_forward_widths", "qalg_backward_dx_widths", "qalg_backward_dw_widths"):
        f = getattr(lib, fn)
        g = lambda **k: f(FAKE, FAKE, FAKE, k.get("q", 3), k.get("kw", arr(64, 128, 64)),  # noqa: E731
                          k.get("nw", arr(256, 128, 128)), k.get("M", 64), k.get("K", 256), k.get("N", 512),
                          k.get("Y", FAKE), k.get("dt", 1), k.get("ws", FAKE), k.get("wsb", 1 << 20),
                          k.get("flags", 0), None)
        assert g(dt=0) == 5, fn
        assert g(flags=Q.QALG_FLAG_LAW_TENSOR) == 8, fn
        assert g(q=65) == 3, fn
        assert g(kw=None) == 1, fn
        assert g(nw=None) == 1, fn
        assert g(kw=arr(64, 132, 60)) == 4, fn           # widths are multiples of 8
        assert g(kw=arr(64, 192, 0)) == 2, fn            # and positive
        assert g(kw=arr(64, 128, 72)) == 2, fn           # summing to K
        assert g(nw=arr(256, 128, 120)) == 2, fn         # and to N
        assert g(Y=None) == 1, fn
        assert g(ws=None) == 1, fn
        assert g(wsb=16) == 6, fn
        assert g(M=1 << 24) == 2, fn                     # M K >= 2^31
    assert lib.qalg_forward_widths(FAKE, FAKE, FAKE, 3, arr(64, 128, 64), arr(256, 128, 128), 0, 256, 512,
                                   FAKE, 1, FAKE, 0, 0, None) == 0
    assert lib.qalg_backward_dw_widths(FAKE, FAKE, FAKE, 3, arr(64, 128, 64), arr(256, 128, 128), 0, 256, 512,
                                       None, 1, FAKE, 0, 0, None) == 1


def test_attention_decode_argument_errors_are_synchronous(lib):
    def dec(B=2, Hq=4, Hkv=2, N=16, d=128, q=4, kind=0, period=0, dt=1, ws=FAKE, wsb=1 << 20, flags=0,
            Qn=FAKE, qp=FAKE, kp=FAKE):
        return lib.qalg_attention_decode(Qn, FAKE, FAKE, qp, kp, B, Hq, Hkv, N, d, q, kind, period, FAKE, dt, ws, wsb,
                                         flags, None)
    assert dec(dt=0) == 5
    assert dec(flags=1) == 8
    assert dec(Hkv=3) == 2                 # Hkv does not divide Hq
    assert dec(Hq=18, Hkv=2) == 2          # more than 8 query heads per key/value head
    assert dec(d=96) == 2
    assert dec(N=0) == 2
    assert dec(q=3) == 3
    assert dec(q=32) == 4                  # d / q = 4 is not a multiple of 8
    assert dec(q=4, kind=1, period=6) == 8
    assert dec(q=4, kind=7) == 8
    assert dec(Qn=None) == 1
    assert dec(qp=FAKE + 4) == 4
    assert dec(wsb=16) == 6
    assert dec(ws=None) == 1
    assert dec(B=0, Qn=None, qp=None, kp=None, ws=None) == 0
    need = Q.qalg_attention_decode_workspace_bytes(2, 4, 16, 128)
    assert need >= 2 * 4 * 1 * 132 * 4 and need % 256 == 0
    assert Q.qalg_attention_decode_workspace_bytes(2, 4, 0, 128) == 0
    # the offset prefill: a negative first position is refused
    assert lib.qalg_attention_forward_at(FAKE, FAKE, FAKE, 2, 1, 8, 64, 2, -1, FAKE, 1, 0, None) == 2



def test_attention_training_argument_errors_are_synchronous(lib):
    def fwd(Hq=4, Hkv=2, S=64, d=128, q=4, p0=0, dt=1, flags=0, lse=FAKE, O=FAKE):
        return lib.qalg_attention_forward_train(FAKE, FAKE, FAKE, Hq, Hkv, S, d, q, p0, O, lse, dt, flags, None)
    assert fwd(dt=0) == 5
    assert fwd(flags=2) == 8
    assert fwd(Hkv=3) == 2
    assert fwd(p0=-1) == 2
    assert fwd(q=16) == 4
    assert fwd(lse=None) == 1
    assert fwd(lse=FAKE + 2) == 4
    assert fwd(S=0, lse=None) == 0

    def bwd(Hq=4, Hkv=2, S=64, d=128, q=4, p0=0, dt=1, flags=0, ws=FAKE, wsb=1 << 20, dO=FAKE, dK=FAKE, lse=FAKE):
        return lib.qalg_attention_backward(FAKE, FAKE, FAKE, FAKE, dO, lse, Hq, Hkv, S, d, q, p0, FAKE, dK, FAKE, dt,
                                           ws, wsb, flags, None)
    assert bwd(dt=0) == 5
    assert bwd(flags=4) == 8
    assert bwd(Hkv=3) == 2
    assert bwd(d=96) == 2
    assert bwd(q=3) == 3
    assert bwd(q=8, d=64) == 4
    assert bwd(dO=None) == 1
    assert bwd(ws=None) == 1
    assert bwd(dK=FAKE + 8) == 4
    assert bwd(lse=FAKE + 1) == 4
    assert bwd(wsb=64) == 6
    assert bwd(ws=FAKE + 8) == 6
    assert bwd(S=0, dO=None) == 0
    # per (head, type): ceil(S / q) rounded up to 64 pairs of fp32, plus 64 spare pairs; with an
    # even number of query heads per key/value head also two shares of fp32 dK and dV
    one = Q.qalg_attention_backward_workspace_bytes(3, 3, 300, 128, 4)
    assert one >= (3 * 4 * 128 + 64) * 8 and one % 256 == 0
    two = Q.qalg_attention_backward_workspace_bytes(4, 2, 300, 128, 4)
    assert two >= (4 * 4 * 128 + 64) * 8 + 2 * 2 * 2 * 300 * 128 * 4 and two % 256 == 0
    assert Q.qalg_attention_backward_workspace_bytes(0, 1, 300, 128, 4) == 0
    assert Q.qalg_attention_backward_workspace_bytes(4, 3, 300, 128, 4) == 0

def test_two_stage_flag_errors_are_synchronous(lib):
    ts = 128
    q, M, K, N = 2, 64, 16, 16
    need = Q.qalg_workspace_bytes_two_stage(q, M, N)
    assert need == Q.qalg_workspace_bytes(q, M) + (M * N * 4 + 255) // 256 * 256
    assert Q.qalg_workspace_bytes_two_stage(0, M, N) == 0 and Q.qalg_workspace_bytes_two_stage(q, M, 0) == 0
    base = Q.qalg_workspace_bytes(q, M)
    assert call_fwd(lib, flags=ts, wsb=base) == 6                      # no room for the diagonal maps
    assert call_fwd(lib, flags=ts, dt=0, wsb=need) == 8                 # bf16 only
    assert call_fwd(lib, flags=ts | 8, wsb=need) == 8                   # not with the recursive law
    assert call_fwd(lib, flags=ts | 2, wsb=need) == 8                   # not with a forced path
    assert call_fwd(lib, flags=ts | 16, wsb=need) == 8                  # not with a tile flag
    assert call_fwd(lib, flags=ts, fn="qalg_backward_dx", wsb=need) == 8
    assert lib.qalg_forward_batched(2, FAKE, FAKE, FAKE, q, M, K, N, FAKE, 1, FAKE, need, ts, None) == 6
