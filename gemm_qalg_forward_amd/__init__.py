"""Python binding of libqalg, the row-typed Q_q projection for MI355X (gfx950).

Argument marshalling only: every step runs in the HIP kernels of libqalg.so,
called through its C ABI (include/qalg.h).  PyTorch supplies device memory and
the current stream.  There is no CPU fallback: if libqalg.so is missing or a
tensor is not on the GPU, the call raises.

Functions carry the C names:
    qalg_forward, qalg_forward_graph, qalg_backward_dx, qalg_backward_dw, qalg_forward_batched,
    qalg_backward_dx_graph, qalg_backward_dw_graph, qalg_forward_widths, qalg_backward_dx_widths,
    qalg_backward_dw_widths,
    qalg_gated_forward, qalg_gated_forward_keep, qalg_merge_gate_up, qalg_split_gate_up, qalg_swiglu_forward, qalg_swiglu_backward,
    qalg_attention_forward, qalg_attention_forward_at, qalg_attention_decode,
    qalg_attention_decode_workspace_bytes, qalg_attention_forward_train, qalg_attention_backward,
    qalg_attention_backward_workspace_bytes, qalg_forward_noalloc,
    qalg_type_schedule, qalg_build_index, qalg_build_index_batched,
    qalg_read_status, qalg_workspace_bytes, qalg_index_layout,
    qalg_status_string, qalg_version.
"""
from __future__ import annotations

import ctypes
import pathlib

__all__ = [
    "QalgError", "lib", "lib_path",
    "QALG_F32", "QALG_BF16", "QALG_FLAG_INDEX_READY", "QALG_FLAG_FORCE_TILED",
    "QALG_FLAG_FORCE_SMALL_M", "QALG_FLAG_LAW_TENSOR",
    "QALG_FLAG_TILE_M64", "QALG_FLAG_TILE_M128", "QALG_FLAG_TILE_M256", "QALG_FLAG_TWO_STAGE", "QALG_FLAG_MASKED",
    "qalg_workspace_bytes_two_stage", "QALG_SCHEDULE_CYCLIC", "QALG_SCHEDULE_INTERVAL", "QALG_MAX_Q",
    "qalg_version", "qalg_status_string", "qalg_workspace_bytes", "qalg_workspace_bytes_dw", "qalg_index_layout",
    "qalg_type_schedule", "qalg_build_index", "qalg_build_index_batched",
    "qalg_forward", "qalg_forward_graph", "qalg_backward_dx", "qalg_backward_dw", "qalg_forward_batched",
    "qalg_backward_dx_graph", "qalg_backward_dw_graph", "qalg_forward_widths", "qalg_backward_dx_widths",
    "qalg_backward_dw_widths",
    "qalg_gated_forward", "qalg_gated_forward_keep", "qalg_merge_gate_up", "qalg_split_gate_up", "qalg_swiglu_forward",
    "qalg_swiglu_backward", "qalg_attention_forward", "qalg_read_status", "workspace",
    "qalg_forward_noalloc", "QALG_NOALLOC_SCRATCH_BYTES", "qalg_attention_forward_at", "qalg_attention_decode",
    "qalg_attention_decode_workspace_bytes", "qalg_attention_forward_train", "qalg_attention_backward",
    "qalg_attention_backward_workspace_bytes",
]

QALG_F32 = 0
QALG_BF16 = 1
QALG_FLAG_INDEX_READY = 1
QALG_FLAG_FORCE_TILED = 2
QALG_FLAG_FORCE_SMALL_M = 4
QALG_FLAG_LAW_TENSOR = 8
QALG_FLAG_TILE_M64 = 16
QALG_FLAG_TILE_M128 = 32
QALG_FLAG_TILE_M256 = 64
QALG_FLAG_TWO_STAGE = 128
QALG_FLAG_MASKED = 256
QALG_SCHEDULE_CYCLIC = 0
QALG_SCHEDULE_INTERVAL = 1
QALG_MAX_Q = 512
QALG_NOALLOC_SCRATCH_BYTES = 4 << 20

_PKG = pathlib.Path(__file__).resolve().parent
lib_path = _PKG / "libqalg.so"
_lib = None

_c_size = ctypes.c_size_t
_c_i32 = ctypes.c_int32
_c_i64 = ctypes.c_int64
_c_u32 = ctypes.c_uint32
_vp = ctypes.c_void_p

_SIGS = {
    "qalg_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "qalg_version": (ctypes.c_int, []),
    "qalg_workspace_bytes": (_c_size, [_c_i32, _c_i64]),
    "qalg_workspace_bytes_dw": (_c_size, [_c_i32, _c_i64, _c_i64, _c_i64]),
    "qalg_workspace_bytes_two_stage": (_c_size, [_c_i32, _c_i64, _c_i64]),
    "qalg_index_layout": (ctypes.c_int, [_c_i32, _c_i64, ctypes.POINTER(_c_i64)]),
    "qalg_type_schedule": (ctypes.c_int, [_vp, _c_i64, _c_i32, _c_i32, _c_i64, _vp, _vp]),
    "qalg_build_index": (ctypes.c_int, [_vp, _c_i32, _c_i64, _vp, _c_size, _vp]),
    "qalg_build_index_batched": (ctypes.c_int, [_c_i32, _vp, _c_i32, _c_i64, _vp, _c_size, _vp]),
    "qalg_forward": (ctypes.c_int, [_vp, _vp, _vp, _c_i32, _c_i64, _c_i64, _c_i64, _vp, _c_i32, _vp, _c_size, _c_u32, _vp]),
    "qalg_forward_graph": (ctypes.c_int, [_vp, _vp, _vp, _c_i32, _vp, _c_i64, _c_i64, _c_i64, _vp, _c_i32, _vp, _c_size,
                                          _c_u32, _vp]),
    "qalg_backward_dx_graph": (ctypes.c_int, [_vp, _vp, _vp, _c_i32, _vp, _c_i64, _c_i64, _c_i64, _vp, _c_i32, _vp, _c_size,
                                              _c_u32, _vp]),
    "qalg_backward_dw_graph": (ctypes.c_int, [_vp, _vp, _vp, _c_i32, _vp, _c_i64, _c_i64, _c_i64, _vp, _c_i32, _vp, _c_size,
                                              _c_u32, _vp]),
    "qalg_forward_widths": (ctypes.c_int, [_vp, _vp, _vp, _c_i32, ctypes.POINTER(_c_i64), ctypes.POINTER(_c_i64),
                                           _c_i64, _c_i64, _c_i64, _vp, _c_i32, _vp, _c_size, _c_u32, _vp]),
    "qalg_backward_dx_widths": (ctypes.c_int, [_vp, _vp, _vp, _c_i32, ctypes.POINTER(_c_i64), ctypes.POINTER(_c_i64),
                                               _c_i64, _c_i64, _c_i64, _vp, _c_i32, _vp, _c_size, _c_u32, _vp]),
    "qalg_backward_dw_widths": (ctypes.c_int, [_vp, _vp, _vp, _c_i32, ctypes.POINTER(_c_i64), ctypes.POINTER(_c_i64),
                                               _c_i64, _c_i64, _c_i64, _vp, _c_i32, _vp, _c_size, _c_u32, _vp]),
    "qalg_backward_dx": (ctypes.c_int, [_vp, _vp, _vp, _c_i32, _c_i64, _c_i64, _c_i64, _vp, _c_i32, _vp, _c_size, _c_u32, _vp]),
    "qalg_backward_dw": (ctypes.c_int, [_vp, _vp, _vp, _c_i32, _c_i64, _c_i64, _c_i64, _vp, _c_i32, _vp, _c_size, _c_u32, _vp]),
    "qalg_forward_batched": (ctypes.c_int, [_c_i32, _vp, _vp, _vp, _c_i32, _c_i64, _c_i64, _c_i64, _vp, _c_i32, _vp, _c_size, _c_u32, _vp]),
    "qalg_gated_forward": (ctypes.c_int, [_vp, _vp, _vp, _c_i32, _c_i64, _c_i64, _c_i64, _vp, _c_i32, _vp, _c_size, _c_u32, _vp]),
    "qalg_gated_forward_keep": (ctypes.c_int, [_vp, _vp, _vp, _c_i32, _c_i64, _c_i64, _c_i64, _vp, _vp, _c_i32, _vp,
                                               _c_size, _c_u32, _vp]),
    "qalg_merge_gate_up": (ctypes.c_int, [_vp, _vp, _c_i32, _c_i64, _c_i64, _vp, _c_i32, _vp]),
    "qalg_split_gate_up": (ctypes.c_int, [_vp, _c_i32, _c_i64, _c_i64, _vp, _vp, _c_i32, _vp]),
    "qalg_swiglu_forward": (ctypes.c_int, [_vp, _c_i32, _c_i64, _c_i64, _vp, _c_i32, _vp]),
    "qalg_swiglu_backward": (ctypes.c_int, [_vp, _vp, _c_i32, _c_i64, _c_i64, _vp, _c_i32, _vp]),
    "qalg_attention_forward": (ctypes.c_int, [_vp, _vp, _vp, _c_i32, _c_i32, _c_i64, _c_i32, _c_i32, _vp, _c_i32,
                                              _c_u32, _vp]),
    "qalg_read_status": (ctypes.c_int, [_vp, _c_i32, _c_i32, _c_i64, _vp, ctypes.POINTER(_c_i64)]),
    "qalg_forward_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _c_i32, _c_i64, _c_i64, _c_i64, _vp, _c_i32, _c_u32, _vp]),
    "qalg_attention_forward_at": (ctypes.c_int, [_vp, _vp, _vp, _c_i32, _c_i32, _c_i64, _c_i32, _c_i32, _c_i64, _vp,
                                                 _c_i32, _c_u32, _vp]),
    "qalg_attention_decode_workspace_bytes": (_c_size, [_c_i32, _c_i32, _c_i64, _c_i32]),
    "qalg_attention_decode": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i64, _c_i32, _c_i32,
                                             _c_i32, _c_i64, _vp, _c_i32, _vp, _c_size, _c_u32, _vp]),
    "qalg_attention_forward_train": (ctypes.c_int, [_vp, _vp, _vp, _c_i32, _c_i32, _c_i64, _c_i32, _c_i32, _c_i64,
                                                    _vp, _vp, _c_i32, _c_u32, _vp]),
    "qalg_attention_backward_workspace_bytes": (_c_size, [_c_i32, _c_i32, _c_i64, _c_i32, _c_i32]),
    "qalg_attention_backward": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i64, _c_i32, _c_i32,
                                               _c_i64, _vp, _vp, _vp, _c_i32, _vp, _c_size, _c_u32, _vp]),
}


class QalgError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {qalg_status_string(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """The loaded libqalg.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not lib_path.exists():
            raise RuntimeError(f"{lib_path} is missing: build it with `python -m gemm_qalg_forward_amd.build`")
        handle = ctypes.CDLL(str(lib_path))
        for name, (res, args) in _SIGS.items():
            f = getattr(handle, name)
            f.restype = res
            f.argtypes = args
        _lib = handle
    return _lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise QalgError(fn, status)


def qalg_version() -> int:
    return lib().qalg_version()


def qalg_status_string(status: int) -> str:
    return lib().qalg_status_string(status).decode()


def qalg_workspace_bytes(q: int, M: int) -> int:
    return lib().qalg_workspace_bytes(q, M)


def qalg_workspace_bytes_dw(q: int, M: int, K: int, N: int) -> int:
    return lib().qalg_workspace_bytes_dw(q, M, K, N)


def qalg_workspace_bytes_two_stage(q: int, M: int, N: int) -> int:
    return lib().qalg_workspace_bytes_two_stage(q, M, N)


def qalg_index_layout(q: int, M: int) -> tuple[int, int, int, int]:
    out = (_c_i64 * 4)()
    _check("qalg_index_layout", lib().qalg_index_layout(q, M, out))
    return tuple(out)


# ---------------------------------------------------------------------------
# tensor marshalling (torch is imported lazily: the CPU tests need only ctypes)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dev_ptr(t, name: str):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU (libqalg has no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major, packed)")
    return t.data_ptr()


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return QALG_BF16
    if t.dtype == torch.float32:
        return QALG_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def workspace(q: int, M: int, E: int = 1, device="cuda", dw_shape=None, two_stage_N=None):
    """A device workspace of the size the projections need (uint8 tensor); with dw_shape = (K, N)
    large enough for qalg_backward_dw to split its contraction (qalg_workspace_bytes_dw); with
    two_stage_N = N large enough for the two-stage forward (qalg_workspace_bytes_two_stage)."""
    torch = _torch()
    if two_stage_N is not None:
        n = qalg_workspace_bytes_two_stage(q, M, two_stage_N) * E
    elif dw_shape is not None and E == 1:
        n = qalg_workspace_bytes_dw(q, M, dw_shape[0], dw_shape[1])
    else:
        n = qalg_workspace_bytes(q, M) * E
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def _tau_check(tau, M: int, E: int = 1, like=None):
    torch = _torch()
    if tau.dtype != torch.int32 or tau.numel() != M * E:
        raise ValueError(f"tau must be int32 with {M * E} elements")
    if like is not None:
        _same_device(tau, like, "tau")


def _same_device(t, like, name: str) -> None:
    if t.device != like.device:
        raise ValueError(f"{name} is on {t.device}, the operands on {like.device}")


def _check_out(t, shape, like, name: str):
    """A caller-supplied output must have exactly the shape, dtype and device the
    kernels write: the library trusts the sizes it is given, so an undersized or
    mistyped buffer would be written out of bounds on the device.  Checked before
    any pointer is taken, so the error is raised without touching the GPU."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != like.dtype:
        raise TypeError(f"{name} must have dtype {like.dtype}, got {t.dtype}")
    _same_device(t, like, name)
    return t


def _same_operand(t, like, name: str) -> None:
    if t.dtype != like.dtype:
        raise TypeError("operands must share a dtype")
    _same_device(t, like, name)


def _new_or_check(t, shape, like, name: str):
    torch = _torch()
    if t is None:
        return torch.empty(tuple(shape), dtype=like.dtype, device=like.device)
    return _check_out(t, shape, like, name)


def _ws_or_new(ws, q: int, M: int, like, E: int = 1, dw_shape=None):
    if ws is None:
        return workspace(q, M, E, device=like.device, dw_shape=dw_shape)
    _same_device(ws, like, "ws")
    return ws


def qalg_type_schedule(positions, q: int, kind: int = QALG_SCHEDULE_CYCLIC, period: int = 0,
                       tau=None, stream=None):
    """tau[m] = tau(positions[m]) on the device (int64 positions -> int32 types)."""
    torch = _torch()
    if positions.dtype != torch.int64:
        raise TypeError("positions must be int64")
    M = positions.numel()
    if tau is None:
        tau = torch.empty(M, dtype=torch.int32, device=positions.device)
    elif tau.dtype != torch.int32 or tau.numel() != M:
        raise ValueError(f"tau must be int32 with {M} elements")
    else:
        _same_device(tau, positions, "tau")
    _check("qalg_type_schedule", lib().qalg_type_schedule(
        _dev_ptr(positions, "positions"), M, q, kind, period, _dev_ptr(tau, "tau"), _stream(stream)))
    return tau


def qalg_build_index(tau, q: int, ws=None, stream=None):
    M = tau.numel()
    ws = _ws_or_new(ws, q, M, tau)
    _check("qalg_build_index", lib().qalg_build_index(
        _dev_ptr(tau, "tau"), q, M, _dev_ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream)))
    return ws


def qalg_build_index_batched(tau, q: int, ws=None, stream=None):
    E, M = tau.shape
    ws = _ws_or_new(ws, q, M, tau, E)
    _check("qalg_build_index_batched", lib().qalg_build_index_batched(
        E, _dev_ptr(tau, "tau"), q, M, _dev_ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream)))
    return ws


def _proj(fn: str, A, B, tau, q: int, out, out_shape, ws, flags: int, stream, M: int, K: int, N: int):
    if A.dtype != B.dtype:
        raise TypeError("operands must share a dtype")
    dt = _dtype_code(A)
    _same_device(B, A, "B")
    _tau_check(tau, M, like=A)
    out = _new_or_check(out, out_shape, A, "out")
    ws = _ws_or_new(ws, q, M, A)
    _check(fn, getattr(lib(), fn)(
        _dev_ptr(A, "A"), _dev_ptr(B, "B"), _dev_ptr(tau, "tau"), q, M, K, N, _dev_ptr(out, "out"),
        dt, _dev_ptr(ws, "ws"), ws.numel() * ws.element_size(), flags, _stream(stream)))
    return out


def qalg_forward(X, W, tau, q: int, Y=None, ws=None, flags: int = 0, stream=None):
    """Y = X *_{Q_q} W: X [M, K], W [K, N], tau int32 [M] -> Y [M, N]."""
    M, K = X.shape
    K2, N = W.shape
    if K2 != K:
        raise ValueError("X and W inner sizes differ")
    return _proj("qalg_forward", X, W, tau, q, Y, (M, N), ws, flags, stream, M, K, N)


def _adjacency_check(adjacency, q: int, like=None) -> None:
    torch = _torch()
    if adjacency.dtype != torch.int64 or adjacency.numel() != q:
        raise ValueError("adjacency must be int64 with q elements")
    if like is not None:
        _same_device(adjacency, like, "adjacency")


def qalg_forward_graph(X, W, tau, q: int, adjacency, Y=None, ws=None, flags: int = 0, stream=None):
    """Y = X *_{Q_G} W under a graph law: adjacency is an int64 device tensor of q out-edge masks."""
    torch = _torch()
    M, K = X.shape
    K2, N = W.shape
    if K2 != K:
        raise ValueError("X and W inner sizes differ")
    _adjacency_check(adjacency, q, like=X)
    _same_operand(W, X, "W")
    _tau_check(tau, M, like=X)
    Y = _new_or_check(Y, (M, N), X, "Y")
    ws = _ws_or_new(ws, q, M, X)
    _check("qalg_forward_graph", lib().qalg_forward_graph(
        _dev_ptr(X, "X"), _dev_ptr(W, "W"), _dev_ptr(tau, "tau"), q, _dev_ptr(adjacency, "adjacency"), M, K, N,
        _dev_ptr(Y, "Y"), _dtype_code(X), _dev_ptr(ws, "ws"), ws.numel() * ws.element_size(), flags,
        _stream(stream)))
    return Y


def qalg_backward_dx_graph(dY, W, tau, q: int, adjacency, dX=None, ws=None, flags: int = 0, stream=None):
    """dX of the graph-law projection: dY [M, N], W [K, N] -> dX [M, K]."""
    torch = _torch()
    M, N = dY.shape
    K, N2 = W.shape
    if N2 != N:
        raise ValueError("dY and W widths differ")
    _adjacency_check(adjacency, q, like=dY)
    _same_operand(W, dY, "W")
    _tau_check(tau, M, like=dY)
    dX = _new_or_check(dX, (M, K), dY, "dX")
    ws = _ws_or_new(ws, q, M, dY)
    _check("qalg_backward_dx_graph", lib().qalg_backward_dx_graph(
        _dev_ptr(dY, "dY"), _dev_ptr(W, "W"), _dev_ptr(tau, "tau"), q, _dev_ptr(adjacency, "adjacency"), M, K, N,
        _dev_ptr(dX, "dX"), _dtype_code(dY), _dev_ptr(ws, "ws"), ws.numel() * ws.element_size(), flags,
        _stream(stream)))
    return dX


def qalg_backward_dw_graph(X, dY, tau, q: int, adjacency, dW=None, ws=None, flags: int = 0, stream=None):
    """dW of the graph-law projection: X [M, K], dY [M, N] -> dW [K, N]."""
    torch = _torch()
    M, K = X.shape
    M2, N = dY.shape
    if M2 != M:
        raise ValueError("X and dY row counts differ")
    _adjacency_check(adjacency, q, like=X)
    _same_operand(dY, X, "dY")
    _tau_check(tau, M, like=X)
    dW = _new_or_check(dW, (K, N), X, "dW")
    ws = _ws_or_new(ws, q, M, X)
    _check("qalg_backward_dw_graph", lib().qalg_backward_dw_graph(
        _dev_ptr(X, "X"), _dev_ptr(dY, "dY"), _dev_ptr(tau, "tau"), q, _dev_ptr(adjacency, "adjacency"), M, K, N,
        _dev_ptr(dW, "dW"), _dtype_code(X), _dev_ptr(ws, "ws"), ws.numel() * ws.element_size(), flags,
        _stream(stream)))
    return dW


def qalg_backward_dx(dY, W, tau, q: int, dX=None, ws=None, flags: int = 0, stream=None):
    """dX of the projection: dY [M, N], W [K, N] -> dX [M, K]."""
    M, N = dY.shape
    K, N2 = W.shape
    if N2 != N:
        raise ValueError("dY and W widths differ")
    return _proj("qalg_backward_dx", dY, W, tau, q, dX, (M, K), ws, flags, stream, M, K, N)


def qalg_backward_dw(X, dY, tau, q: int, dW=None, ws=None, flags: int = 0, stream=None):
    """dW of the projection: X [M, K], dY [M, N] -> dW [K, N]."""
    M, K = X.shape
    M2, N = dY.shape
    if M2 != M:
        raise ValueError("X and dY row counts differ")
    return _proj("qalg_backward_dw", X, dY, tau, q, dW, (K, N), ws, flags, stream, M, K, N)


def _widths_arg(widths, q: int, total: int, what: str):
    w = [int(x) for x in widths]
    if len(w) != q or sum(w) != total:
        raise ValueError(f"{what} must hold q = {q} widths summing to {total}")
    return (_c_i64 * q)(*w)


def qalg_forward_widths(X, W, tau, q: int, in_widths, out_widths, Y=None, ws=None, flags: int = 0, stream=None):
    """Y = X *_{Q_q} W on groups of unequal widths (in_widths over K, out_widths over N; host ints)."""
    torch = _torch()
    M, K = X.shape
    K2, N = W.shape
    if K2 != K:
        raise ValueError("X and W inner sizes differ")
    kw, nw = _widths_arg(in_widths, q, K, "in_widths"), _widths_arg(out_widths, q, N, "out_widths")
    _same_operand(W, X, "W")
    _tau_check(tau, M, like=X)
    Y = _new_or_check(Y, (M, N), X, "Y")
    ws = _ws_or_new(ws, q, M, X)
    _check("qalg_forward_widths", lib().qalg_forward_widths(
        _dev_ptr(X, "X"), _dev_ptr(W, "W"), _dev_ptr(tau, "tau"), q, kw, nw, M, K, N, _dev_ptr(Y, "Y"),
        _dtype_code(X), _dev_ptr(ws, "ws"), ws.numel() * ws.element_size(), flags, _stream(stream)))
    return Y


def qalg_backward_dx_widths(dY, W, tau, q: int, in_widths, out_widths, dX=None, ws=None, flags: int = 0,
                            stream=None):
    """dX of the unequal-width projection: dY [M, N], W [K, N] -> dX [M, K]."""
    torch = _torch()
    M, N = dY.shape
    K, N2 = W.shape
    if N2 != N:
        raise ValueError("dY and W widths differ")
    kw, nw = _widths_arg(in_widths, q, K, "in_widths"), _widths_arg(out_widths, q, N, "out_widths")
    _same_operand(W, dY, "W")
    _tau_check(tau, M, like=dY)
    dX = _new_or_check(dX, (M, K), dY, "dX")
    ws = _ws_or_new(ws, q, M, dY)
    _check("qalg_backward_dx_widths", lib().qalg_backward_dx_widths(
        _dev_ptr(dY, "dY"), _dev_ptr(W, "W"), _dev_ptr(tau, "tau"), q, kw, nw, M, K, N, _dev_ptr(dX, "dX"),
        _dtype_code(dY), _dev_ptr(ws, "ws"), ws.numel() * ws.element_size(), flags, _stream(stream)))
    return dX


def qalg_backward_dw_widths(X, dY, tau, q: int, in_widths, out_widths, dW=None, ws=None, flags: int = 0,
                            stream=None):
    """dW of the unequal-width projection: X [M, K], dY [M, N] -> dW [K, N]."""
    torch = _torch()
    M, K = X.shape
    M2, N = dY.shape
    if M2 != M:
        raise ValueError("X and dY row counts differ")
    kw, nw = _widths_arg(in_widths, q, K, "in_widths"), _widths_arg(out_widths, q, N, "out_widths")
    _same_operand(dY, X, "dY")
    _tau_check(tau, M, like=X)
    dW = _new_or_check(dW, (K, N), X, "dW")
    ws = _ws_or_new(ws, q, M, X)
    _check("qalg_backward_dw_widths", lib().qalg_backward_dw_widths(
        _dev_ptr(X, "X"), _dev_ptr(dY, "dY"), _dev_ptr(tau, "tau"), q, kw, nw, M, K, N, _dev_ptr(dW, "dW"),
        _dtype_code(X), _dev_ptr(ws, "ws"), ws.numel() * ws.element_size(), flags, _stream(stream)))
    return dW


def qalg_merge_gate_up(Wg, Wu, q: int, Wgu=None, stream=None):
    """Merged gate/up bank (layout in include/qalg.h): Wg, Wu [K, F] -> Wgu [K, 2F]."""
    torch = _torch()
    K, F = Wg.shape
    if tuple(Wu.shape) != (K, F) or Wu.dtype != Wg.dtype:
        raise ValueError("gate and up weights must have the same shape and dtype")
    _same_device(Wu, Wg, "Wu")
    Wgu = _new_or_check(Wgu, (K, 2 * F), Wg, "Wgu")
    _check("qalg_merge_gate_up", lib().qalg_merge_gate_up(
        _dev_ptr(Wg, "Wg"), _dev_ptr(Wu, "Wu"), q, K, F, _dev_ptr(Wgu, "Wgu"), _dtype_code(Wg), _stream(stream)))
    return Wgu


def qalg_split_gate_up(Wgu, q: int, Wg=None, Wu=None, stream=None):
    """Inverse of the merge: Wgu [K, 2F] -> (Wg, Wu), each [K, F]."""
    torch = _torch()
    K, F2 = Wgu.shape
    if F2 % 2:
        raise ValueError("Wgu must have an even number of columns")
    F = F2 // 2
    Wg = _new_or_check(Wg, (K, F), Wgu, "Wg")
    Wu = _new_or_check(Wu, (K, F), Wgu, "Wu")
    _check("qalg_split_gate_up", lib().qalg_split_gate_up(
        _dev_ptr(Wgu, "Wgu"), q, K, F, _dev_ptr(Wg, "Wg"), _dev_ptr(Wu, "Wu"), _dtype_code(Wgu), _stream(stream)))
    return Wg, Wu


def qalg_swiglu_forward(GU, q: int, H=None, stream=None):
    """H = silu(gate) * up on merged pre-activations: GU [M, 2F] -> H [M, F]."""
    torch = _torch()
    M, F2 = GU.shape
    if F2 % 2:
        raise ValueError("GU must have an even number of columns")
    H = _new_or_check(H, (M, F2 // 2), GU, "H")
    _check("qalg_swiglu_forward", lib().qalg_swiglu_forward(
        _dev_ptr(GU, "GU"), q, M, F2 // 2, _dev_ptr(H, "H"), _dtype_code(GU), _stream(stream)))
    return H


def qalg_swiglu_backward(GU, dH, q: int, dGU=None, stream=None):
    """(dgate, dup) of H = silu(gate) * up, merged: GU [M, 2F], dH [M, F] -> dGU [M, 2F]."""
    torch = _torch()
    M, F2 = GU.shape
    if F2 % 2 or tuple(dH.shape) != (M, F2 // 2) or dH.dtype != GU.dtype:
        raise ValueError("GU must be [M, 2F] and dH [M, F] of the same dtype")
    _same_device(dH, GU, "dH")
    dGU = _new_or_check(dGU, (M, F2), GU, "dGU")
    _check("qalg_swiglu_backward", lib().qalg_swiglu_backward(
        _dev_ptr(GU, "GU"), _dev_ptr(dH, "dH"), q, M, F2 // 2, _dev_ptr(dGU, "dGU"), _dtype_code(GU),
        _stream(stream)))
    return dGU


def qalg_attention_forward(Qh, Kh, Vh, q: int, O=None, flags: int = 0, stream=None):
    """Causal attention with the algebraic score: Q [Hq, S, d], K and V [Hkv, S, d] -> O [Hq, S, d]."""
    torch = _torch()
    Hq, S, d = Qh.shape
    Hkv = Kh.shape[0]
    if tuple(Kh.shape) != (Hkv, S, d) or tuple(Vh.shape) != (Hkv, S, d):
        raise ValueError("K and V must be [Hkv, S, d] with the S and d of Q")
    if Kh.dtype != Qh.dtype or Vh.dtype != Qh.dtype:
        raise TypeError("Q, K and V must share a dtype")
    _same_device(Kh, Qh, "K")
    _same_device(Vh, Qh, "V")
    O = _new_or_check(O, (Hq, S, d), Qh, "O")
    _check("qalg_attention_forward", lib().qalg_attention_forward(
        _dev_ptr(Qh, "Q"), _dev_ptr(Kh, "K"), _dev_ptr(Vh, "V"), Hq, Hkv, S, d, q, _dev_ptr(O, "O"),
        _dtype_code(Qh), flags, _stream(stream)))
    return O


def qalg_attention_forward_at(Qh, Kh, Vh, q: int, first_position: int, O=None, flags: int = 0, stream=None):
    """qalg_attention_forward for a chunk whose row 0 sits at absolute position first_position
    (row s: position first_position + s, type (first_position + s) mod q)."""
    Hq, S, d = Qh.shape
    Hkv = Kh.shape[0]
    if tuple(Kh.shape) != (Hkv, S, d) or tuple(Vh.shape) != (Hkv, S, d):
        raise ValueError("K and V must be [Hkv, S, d] with the S and d of Q")
    if Kh.dtype != Qh.dtype or Vh.dtype != Qh.dtype:
        raise TypeError("Q, K and V must share a dtype")
    _same_device(Kh, Qh, "K")
    _same_device(Vh, Qh, "V")
    O = _new_or_check(O, (Hq, S, d), Qh, "O")
    _check("qalg_attention_forward_at", lib().qalg_attention_forward_at(
        _dev_ptr(Qh, "Q"), _dev_ptr(Kh, "K"), _dev_ptr(Vh, "V"), Hq, Hkv, S, d, q, int(first_position),
        _dev_ptr(O, "O"), _dtype_code(Qh), flags, _stream(stream)))
    return O



def _attn_operands(Qh, Kh, Vh):
    Hq, S, d = Qh.shape
    Hkv = Kh.shape[0]
    if tuple(Kh.shape) != (Hkv, S, d) or tuple(Vh.shape) != (Hkv, S, d):
        raise ValueError("K and V must be [Hkv, S, d] with the S and d of Q")
    if Kh.dtype != Qh.dtype or Vh.dtype != Qh.dtype:
        raise TypeError("Q, K and V must share a dtype")
    _same_device(Kh, Qh, "K")
    _same_device(Vh, Qh, "V")
    return Hq, Hkv, S, d


def qalg_attention_forward_train(Qh, Kh, Vh, q: int, first_position: int = 0, O=None, lse=None, flags: int = 0,
                                 stream=None):
    """The forward for training: O [Hq, S, d] and lse [Hq, S] (fp32, natural log of each query's
    softmax denominator), for qalg_attention_backward; returns (O, lse)."""
    torch = _torch()
    Hq, Hkv, S, d = _attn_operands(Qh, Kh, Vh)
    O = _new_or_check(O, (Hq, S, d), Qh, "O")
    if lse is None:
        lse = torch.empty((Hq, S), dtype=torch.float32, device=Qh.device)
    elif tuple(lse.shape) != (Hq, S) or lse.dtype != torch.float32:
        raise ValueError(f"lse must be float32 [{Hq}, {S}]")
    else:
        _same_device(lse, Qh, "lse")
    _check("qalg_attention_forward_train", lib().qalg_attention_forward_train(
        _dev_ptr(Qh, "Q"), _dev_ptr(Kh, "K"), _dev_ptr(Vh, "V"), Hq, Hkv, S, d, q, int(first_position),
        _dev_ptr(O, "O"), _dev_ptr(lse, "lse"), _dtype_code(Qh), flags, _stream(stream)))
    return O, lse


def qalg_attention_backward_workspace_bytes(Hq: int, Hkv: int, S: int, d: int, q: int) -> int:
    return lib().qalg_attention_backward_workspace_bytes(Hq, Hkv, S, d, q)


def qalg_attention_backward(Qh, Kh, Vh, Oh, dOh, lse, q: int, first_position: int = 0, dQ=None, dK=None, dV=None,
                            ws=None, flags: int = 0, stream=None):
    """Gradients of the algebraic-score attention (Algorithm 2, step 9) from the forward's O and lse
    and the output gradient dO [Hq, S, d]; returns (dQ [Hq, S, d], dK, dV [Hkv, S, d])."""
    torch = _torch()
    Hq, Hkv, S, d = _attn_operands(Qh, Kh, Vh)
    for t, n in ((Oh, "O"), (dOh, "dO")):
        _check_out(t, (Hq, S, d), Qh, n)
    if tuple(lse.shape) != (Hq, S) or lse.dtype != torch.float32:
        raise ValueError(f"lse must be float32 [{Hq}, {S}]")
    _same_device(lse, Qh, "lse")
    dQ = _new_or_check(dQ, (Hq, S, d), Qh, "dQ")
    dK = _new_or_check(dK, (Hkv, S, d), Qh, "dK")
    dV = _new_or_check(dV, (Hkv, S, d), Qh, "dV")
    need = qalg_attention_backward_workspace_bytes(Hq, Hkv, S, d, q)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=Qh.device)
    else:
        _same_device(ws, Qh, "ws")
    _check("qalg_attention_backward", lib().qalg_attention_backward(
        _dev_ptr(Qh, "Q"), _dev_ptr(Kh, "K"), _dev_ptr(Vh, "V"), _dev_ptr(Oh, "O"), _dev_ptr(dOh, "dO"),
        _dev_ptr(lse, "lse"), Hq, Hkv, S, d, q, int(first_position), _dev_ptr(dQ, "dQ"), _dev_ptr(dK, "dK"),
        _dev_ptr(dV, "dV"), _dtype_code(Qh), _dev_ptr(ws, "ws"), ws.numel() * ws.element_size(), flags,
        _stream(stream)))
    return dQ, dK, dV

def qalg_attention_decode_workspace_bytes(B: int, Hq: int, N: int, d: int) -> int:
    return lib().qalg_attention_decode_workspace_bytes(B, Hq, N, d)


def qalg_attention_decode(Qn, Kc, Vc, q_pos, key_pos, q: int, kind: int = QALG_SCHEDULE_CYCLIC, period: int = 0,
                          O=None, ws=None, flags: int = 0, stream=None):
    """Cached decoding (Algorithm 3): Qn [B, Hq, d] new rows at positions q_pos (int64 [B]) against
    caches Kc, Vc [B, Hkv, N, d] with slot positions key_pos (int64 [B, N], negative: empty) -> O [B, Hq, d]."""
    torch = _torch()
    B, Hq, d = Qn.shape
    B2, Hkv, N, d2 = Kc.shape
    if B2 != B or d2 != d or tuple(Vc.shape) != tuple(Kc.shape):
        raise ValueError("Kc and Vc must be [B, Hkv, N, d] with the B and d of Qn")
    if Kc.dtype != Qn.dtype or Vc.dtype != Qn.dtype:
        raise TypeError("Qn, Kc and Vc must share a dtype")
    if q_pos.dtype != torch.int64 or tuple(q_pos.shape) != (B,):
        raise ValueError(f"q_pos must be int64 [{B}]")
    if key_pos.dtype != torch.int64 or tuple(key_pos.shape) != (B, N):
        raise ValueError(f"key_pos must be int64 [{B}, {N}]")
    for t, n in ((Kc, "Kc"), (Vc, "Vc"), (q_pos, "q_pos"), (key_pos, "key_pos")):
        _same_device(t, Qn, n)
    O = _new_or_check(O, (B, Hq, d), Qn, "O")
    need = qalg_attention_decode_workspace_bytes(B, Hq, N, d)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=Qn.device)
    else:
        _same_device(ws, Qn, "ws")
    _check("qalg_attention_decode", lib().qalg_attention_decode(
        _dev_ptr(Qn, "Qn"), _dev_ptr(Kc, "Kc"), _dev_ptr(Vc, "Vc"), _dev_ptr(q_pos, "q_pos"), _dev_ptr(key_pos, "key_pos"),
        B, Hq, Hkv, N, d, q, kind, period, _dev_ptr(O, "O"), _dtype_code(Qn), _dev_ptr(ws, "ws"),
        ws.numel() * ws.element_size(), flags, _stream(stream)))
    return O


def qalg_gated_forward(X, Wgu, tau, q: int, H=None, ws=None, flags: int = 0, stream=None):
    """H = silu(X *_{Q_q} W_gate) * (X *_{Q_q} W_up): X [M, K], merged Wgu [K, 2F] -> H [M, F]."""
    M, K = X.shape
    K2, F2 = Wgu.shape
    if K2 != K or F2 % 2:
        raise ValueError("X and Wgu shapes differ (Wgu is K x 2F)")
    return _proj("qalg_gated_forward", X, Wgu, tau, q, H, (M, F2 // 2), ws, flags, stream, M, K, F2 // 2)


def qalg_gated_forward_keep(X, Wgu, tau, q: int, H=None, GU=None, ws=None, flags: int = 0, stream=None):
    """The training step's gated forward: GU = bf16 merged pre-activations [M, 2F] and
    H = silu(gate) * up [M, F] from those rounded values, one launch; returns (H, GU)."""
    torch = _torch()
    M, K = X.shape
    K2, F2 = Wgu.shape
    if K2 != K or F2 % 2:
        raise ValueError("X and Wgu shapes differ (Wgu is K x 2F)")
    if X.dtype != Wgu.dtype:
        raise TypeError("operands must share a dtype")
    _same_device(Wgu, X, "Wgu")
    _tau_check(tau, M, like=X)
    H = _new_or_check(H, (M, F2 // 2), X, "H")
    GU = _new_or_check(GU, (M, F2), X, "GU")
    ws = _ws_or_new(ws, q, M, X)
    _check("qalg_gated_forward_keep", lib().qalg_gated_forward_keep(
        _dev_ptr(X, "X"), _dev_ptr(Wgu, "Wgu"), _dev_ptr(tau, "tau"), q, M, K, F2 // 2, _dev_ptr(H, "H"),
        _dev_ptr(GU, "GU"), _dtype_code(X), _dev_ptr(ws, "ws"), ws.numel() * ws.element_size(), flags,
        _stream(stream)))
    return H, GU


def qalg_forward_batched(X, W, tau, q: int, Y=None, ws=None, flags: int = 0, stream=None):
    """E projections with their own weight banks: X [E, M, K], W [E, K, N], tau [E, M] -> Y [E, M, N]."""
    torch = _torch()
    E, M, K = X.shape
    E2, K2, N = W.shape
    if E2 != E or K2 != K:
        raise ValueError("X and W shapes differ")
    if X.dtype != W.dtype:
        raise TypeError("operands must share a dtype")
    _same_device(W, X, "W")
    _tau_check(tau, M, E, like=X)
    Y = _new_or_check(Y, (E, M, N), X, "Y")
    ws = _ws_or_new(ws, q, M, X, E)
    _check("qalg_forward_batched", lib().qalg_forward_batched(
        E, _dev_ptr(X, "X"), _dev_ptr(W, "W"), _dev_ptr(tau, "tau"), q, M, K, N, _dev_ptr(Y, "Y"),
        _dtype_code(X), _dev_ptr(ws, "ws"), ws.numel() * ws.element_size(), flags, _stream(stream)))
    return Y


def qalg_forward_noalloc(X, W, tau, q: int, Y, flags: int = 0, stream=None):
    """Y = X *_{Q_q} W with the index in the library's own device array (no workspace, no
    allocation by the library or here: Y is the caller's).  X [M, K], W [K, N], tau int32 [M]."""
    M, K = X.shape
    K2, N = W.shape
    if K2 != K:
        raise ValueError("X and W inner sizes differ")
    if X.dtype != W.dtype:
        raise TypeError("operands must share a dtype")
    _same_device(W, X, "W")
    _tau_check(tau, M, like=X)
    _check_out(Y, (M, N), X, "Y")
    _check("qalg_forward_noalloc", lib().qalg_forward_noalloc(
        _dev_ptr(X, "X"), _dev_ptr(W, "W"), _dev_ptr(tau, "tau"), q, M, K, N, _dev_ptr(Y, "Y"), _dtype_code(X),
        flags, _stream(stream)))
    return Y


def qalg_read_status(ws, q: int, M: int, E: int = 1, stream=None) -> int:
    """Rows with an out-of-range type seen by the last index build in ws (synchronises)."""
    out = _c_i64(0)
    _check("qalg_read_status", lib().qalg_read_status(
        _dev_ptr(ws, "ws"), E, q, M, _stream(stream), ctypes.byref(out)))
    return out.value
