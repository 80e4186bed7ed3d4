// C-ABI of libqalg: argument validation, path choice and launches.  See
// include/qalg.h for the contract of every entry point.
//
// Nothing here waits on the device except qalg_read_status.  Every argument
// error is detected before the first launch of a call.
#include "qalg.h"

#include <climits>
#include <cstdint>

#include "qalg_internal.h"

namespace {

using qalg::Op;
using qalg::ProblemDesc;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

qalg_status hip_status(hipError_t e) { return e == hipSuccess ? QALG_OK : QALG_ERR_HIP; }

constexpr uint32_t kTileFlags = QALG_FLAG_TILE_M64 | QALG_FLAG_TILE_M128 | QALG_FLAG_TILE_M256;

// forced tile height of the persistent forward: 0 (none), 64, 128, 256, or -1 (several flags)
int forced_tile_height(uint32_t flags) {
  const uint32_t t = flags & kTileFlags;
  if (t == 0) return 0;
  if (t == QALG_FLAG_TILE_M64) return 64;
  if (t == QALG_FLAG_TILE_M128) return 128;
  if (t == QALG_FLAG_TILE_M256) return 256;
  return -1;
}

// Shape, type and flag checks shared by the projection entry points.
qalg_status check_shape(int32_t E, int32_t q, int64_t M, int64_t K, int64_t N, int32_t dtype,
                        uint32_t flags) {
  if (dtype != QALG_F32 && dtype != QALG_BF16) return QALG_ERR_DTYPE;
  if (flags & ~uint32_t(QALG_FLAG_INDEX_READY | QALG_FLAG_FORCE_TILED | QALG_FLAG_FORCE_SMALL_M |
                       QALG_FLAG_LAW_TENSOR | kTileFlags | QALG_FLAG_TWO_STAGE | QALG_FLAG_MASKED))
    return QALG_ERR_ARG;
  if ((flags & QALG_FLAG_FORCE_TILED) && (flags & QALG_FLAG_FORCE_SMALL_M)) return QALG_ERR_ARG;
  if (E < 1 || M < 0 || K <= 0 || N <= 0) return QALG_ERR_DIM;
  if (M > INT32_MAX / 2 || K > INT32_MAX / 2 || N > INT32_MAX / 2) return QALG_ERR_DIM;
  if (q < 1 || q > QALG_MAX_Q || K % q || N % q) return QALG_ERR_Q;
  if (dtype == QALG_BF16 && ((K / q) % 8 || (N / q) % 8)) return QALG_ERR_ALIGN;
  if (dtype == QALG_F32 && ((K / q) % 4 || (N / q) % 4)) return QALG_ERR_ALIGN;
  return QALG_OK;
}

qalg_status check_ws(int32_t E, int32_t q, int64_t M, const void* ws, size_t ws_bytes) {
  if (ws == nullptr) return QALG_ERR_NULL;
  if (!aligned16(ws)) return QALG_ERR_WORKSPACE;
  const size_t need = size_t(E) * qalg_workspace_bytes(q, M);
  if (ws_bytes < need) return QALG_ERR_WORKSPACE;
  return QALG_OK;
}

int64_t ws_stride_ints(int32_t q, int64_t M) { return qalg::ws_layout(q, M).total_ints; }

// L of the recursive law Q_2^(x)L for q = 2^L, or -1 when q is not a power of two.
int tensor_levels(int32_t q) {
  if (q < 1 || (q & (q - 1))) return -1;
  int L = 0;
  while ((1 << L) < q) ++L;
  return L;
}


// Shared driver of qalg_forward / qalg_backward_dx / qalg_backward_dw / batched forward.
qalg_status run_projection(Op op, int32_t E, const void* A, const void* B, const int32_t* tau,
                           int32_t q, int64_t M, int64_t K, int64_t N, void* C, int32_t dtype,
                           void* ws, size_t ws_bytes, uint32_t flags, void* stream) {
  qalg_status st = check_shape(E, q, M, K, N, dtype, flags);
  if (st != QALG_OK) return st;
  if ((flags & QALG_FLAG_FORCE_SMALL_M) && (op != Op::Fwd || dtype != QALG_BF16)) return QALG_ERR_ARG;
  const int forced_bm = forced_tile_height(flags);
  if (forced_bm != 0) {
    if (forced_bm < 0 || op != Op::Fwd || E != 1 || dtype != QALG_BF16 ||
        (flags & (QALG_FLAG_FORCE_TILED | QALG_FLAG_FORCE_SMALL_M)))
      return QALG_ERR_ARG;
  }
  const bool tensor = (flags & QALG_FLAG_LAW_TENSOR) != 0;
  const bool two_stage = (flags & QALG_FLAG_TWO_STAGE) != 0;
  const bool masked = (flags & QALG_FLAG_MASKED) != 0;
  if (masked) {
    if (op != Op::Fwd || dtype != QALG_BF16 || tensor || two_stage ||
        (flags & (QALG_FLAG_FORCE_TILED | QALG_FLAG_FORCE_SMALL_M | kTileFlags)))
      return QALG_ERR_ARG;
  }
  if (two_stage) {
    // section 5.3's second schedule: bf16 forward of the complete law, its own kernels
    if (op != Op::Fwd || dtype != QALG_BF16 || tensor ||
        (flags & (QALG_FLAG_FORCE_TILED | QALG_FLAG_FORCE_SMALL_M | kTileFlags)))
      return QALG_ERR_ARG;
    if (M * N >= (int64_t(1) << 31)) return QALG_ERR_DIM;
  }
  if (tensor) {
    // the recursive law: persistent forward, register-staged dX and dW, one bank, bf16
    if (E != 1 || dtype != QALG_BF16 || (flags & (QALG_FLAG_FORCE_TILED | QALG_FLAG_FORCE_SMALL_M)))
      return QALG_ERR_ARG;
    if (tensor_levels(q) < 0) return QALG_ERR_Q;
  }
  // with no rows only dW's output is touched (it is zero-filled)
  if (M > 0 && (A == nullptr || B == nullptr || C == nullptr || tau == nullptr)) return QALG_ERR_NULL;
  if (M == 0 && op == Op::Dw && C == nullptr) return QALG_ERR_NULL;
  if ((A && !aligned16(A)) || (B && !aligned16(B)) || (C && !aligned16(C)) ||
      (tau && (reinterpret_cast<uintptr_t>(tau) & 3u)))
    return QALG_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int elem = dtype == QALG_BF16 ? 2 : 4;

  if (M == 0) {
    if (op != Op::Dw) return QALG_OK;
    // no rows: every weight-gradient block is zero
    return hip_status(qalg::launch_fill_zero(C, size_t(E) * size_t(K) * size_t(N) * elem, s));
  }

  ProblemDesc p{};
  p.op = op;
  p.A = A;
  p.B = B;
  p.C = C;
  p.tau = tau;
  p.q = q;
  p.M = M;
  p.K = K;
  p.N = N;
  p.E = E;
  p.law_L = tensor ? tensor_levels(q) : 0;
  // dW: a workspace of qalg_workspace_bytes_dw lets the register-staged path split its contraction
  if (op == Op::Dw && E == 1 && ws != nullptr && ws_bytes >= qalg_workspace_bytes_dw(q, M, K, N))
    p.dw_part = static_cast<char*>(ws) + qalg_workspace_bytes(q, M);

  // the workspace contract is the same on every path, used or not
  st = check_ws(E, q, M, ws, ws_bytes);
  if (st != QALG_OK) return st;

  if (masked) {
    // rows of an out-of-range type come out as zeros from the kernel itself; the
    // index is built only to honour the workspace contract (its count of such rows)
    if (!(flags & QALG_FLAG_INDEX_READY)) {
      if (qalg::launch_build_index(tau, q, M, E, static_cast<int32_t*>(ws), ws_stride_ints(q, M), s) != hipSuccess)
        return QALG_ERR_HIP;
    }
    p.ws = static_cast<int32_t*>(ws);
    p.ws_stride = ws_stride_ints(q, M);
    return hip_status(qalg::launch_tiled_masked_bf16(p, s));
  }
  if (two_stage) {
    if (ws_bytes < size_t(E) * qalg_workspace_bytes_two_stage(q, M, N)) return QALG_ERR_WORKSPACE;
    const int64_t stride = ws_stride_ints(q, M);
    int32_t* wsi = static_cast<int32_t*>(ws);
    p.ws = wsi;
    p.ws_stride = stride;
    // the diagonal maps of the E problems follow their E indices
    p.fwd_diag = static_cast<char*>(ws) + size_t(E) * qalg_workspace_bytes(q, M);
    hipError_t e;
    if (!(flags & QALG_FLAG_INDEX_READY))
      e = qalg::launch_build_index_zeroing(tau, q, M, E, wsi, stride, C, N, 2, M * N * 2, s);
    else
      e = qalg::launch_zero_bad_rows(wsi, q, M, E, stride, C, N, 2, M * N * 2, s);
    if (e != hipSuccess) return QALG_ERR_HIP;
    return hip_status(qalg::launch_tiled_two_stage_bf16(p, s));
  }

  if ((p.law_L > 0 && op == Op::Fwd) || forced_bm != 0) {
    if (!qalg::fwd_persistent_shape_ok(p)) {
      const int64_t lim = int64_t(1) << 31;
      if (M * K >= lim || K * N >= lim || M * N >= lim) return QALG_ERR_DIM;
      return forced_bm ? QALG_ERR_ARG : QALG_ERR_ALIGN;
    }
    if (forced_bm != 0 && qalg::fwd_tile_height(p, forced_bm) == 0) return QALG_ERR_ARG;
    int32_t* wsl = static_cast<int32_t*>(ws);
    p.ws = wsl;
    p.ws_stride = ws_stride_ints(q, M);
    if (!(flags & QALG_FLAG_INDEX_READY)) {
      if (qalg::launch_build_index(tau, q, M, 1, wsl, p.ws_stride, s) != hipSuccess) return QALG_ERR_HIP;
    }
    return hip_status(qalg::launch_fwd_persistent_bf16(p, s, forced_bm));
  }

  // small-M weight-streaming forward: reads the types directly, no index
  const bool small_ok = dtype == QALG_BF16 && qalg::small_m_supported(p);
  if (flags & QALG_FLAG_FORCE_SMALL_M) {
    if (!small_ok) return QALG_ERR_ARG;
  }
  const bool use_small = small_ok && !(flags & QALG_FLAG_FORCE_TILED);
  if (use_small) return hip_status(qalg::launch_small_m_bf16(p, s));
  const int64_t stride = ws_stride_ints(q, M);
  int32_t* wsi = static_cast<int32_t*>(ws);
  p.ws = wsi;
  p.ws_stride = stride;

  hipError_t e;
  if (dtype == QALG_BF16 && !(flags & QALG_FLAG_FORCE_TILED) && qalg::fwd_persistent_supported(p)) {
    // the persistent forward zeroes the rows of an out-of-range type itself
    if (!(flags & QALG_FLAG_INDEX_READY)) {
      e = qalg::launch_build_index(tau, q, M, E, wsi, stride, s);
      if (e != hipSuccess) return QALG_ERR_HIP;
    }
    return hip_status(qalg::launch_fwd_persistent_bf16(p, s));
  }

  // A handful of rows per type (and more than the weight-streaming kernel
  // takes): one tile over all rows reads every weight block once (the masked
  // schedule), where per-type tiles would read W_jj once per type.  Measured on
  // 64 experts at 8 and 16 rows per type: 0.99-1.06x of the plain product,
  // against 0.72-0.85x for per-type tiles.
  if (dtype == QALG_BF16 && op == Op::Fwd && p.law_L == 0 && !(flags & QALG_FLAG_FORCE_TILED) &&
      (M + q - 1) / q <= 16 && q > 1) {
    if (!(flags & QALG_FLAG_INDEX_READY)) {
      e = qalg::launch_build_index(tau, q, M, E, wsi, stride, s);
      if (e != hipSuccess) return QALG_ERR_HIP;
    }
    return hip_status(qalg::launch_tiled_masked_bf16(p, s));
  }

  if (dtype == QALG_BF16 && qalg::grad_persistent_supported(p)) {
    // the persistent gradients read the index on the device (closed-form rows
    // for a cyclic schedule, the row list otherwise); dX zeroes the rows of an
    // out-of-range type itself, dW ignores them
    if (!(flags & QALG_FLAG_INDEX_READY)) {
      e = qalg::launch_build_index(tau, q, M, E, wsi, stride, s);
      if (e != hipSuccess) return QALG_ERR_HIP;
    }
    return hip_status(qalg::launch_grad_persistent_bf16(p, s));
  }

  // rows of an out-of-range type get zero Y / dX rows; dW ignores them
  void* zero_out = op == Op::Dw ? nullptr : C;
  const int64_t zero_ld = op == Op::Fwd ? N : K;
  const int64_t zero_stride = M * zero_ld * elem;
  if (!(flags & QALG_FLAG_INDEX_READY)) {
    e = qalg::launch_build_index_zeroing(tau, q, M, E, wsi, stride, zero_out, zero_ld, elem,
                                         zero_stride, s);
  } else if (zero_out != nullptr) {
    e = qalg::launch_zero_bad_rows(wsi, q, M, E, stride, zero_out, zero_ld, elem, zero_stride, s);
  } else {
    e = hipSuccess;
  }
  if (e != hipSuccess) return QALG_ERR_HIP;

  e = dtype == QALG_BF16 ? qalg::launch_tiled_bf16(p, s) : qalg::launch_tiled_f32(p, s);
  return hip_status(e);
}

// Shared driver of the graph-law entry points (bf16, q <= 64, one 64-bit
// out-edge mask per type).  Where their shapes allow, the forward takes the
// persistent kernel (absent-edge blocks zeroed by a pass first) and dX and dW
// the persistent gradient kernels (tiles of absent edges have no k-steps and
// store zeros); every other case runs the register-staged kernels, whose
// tiles of absent edges store zeros.
qalg_status run_graph(Op op, const void* A, const void* B, const int32_t* tau, int32_t q, const uint64_t* adj,
                      int64_t M, int64_t K, int64_t N, void* C, int32_t dtype, void* ws, size_t ws_bytes,
                      uint32_t flags, void* stream) {
  if (dtype != QALG_BF16) return QALG_ERR_DTYPE;
  if (flags & ~uint32_t(QALG_FLAG_INDEX_READY)) return QALG_ERR_ARG;
  if (M < 0 || K <= 0 || N <= 0 || M > INT32_MAX / 2 || K > INT32_MAX / 2 || N > INT32_MAX / 2) return QALG_ERR_DIM;
  const int64_t lim = int64_t(1) << 31;
  if (M * K >= lim || K * N >= lim || M * N >= lim) return QALG_ERR_DIM;
  if (q < 1 || q > 64 || K % q || N % q) return QALG_ERR_Q;
  if ((K / q) % 8 || (N / q) % 8) return QALG_ERR_ALIGN;
  if (M > 0 && (A == nullptr || B == nullptr || C == nullptr || tau == nullptr || adj == nullptr))
    return QALG_ERR_NULL;
  if (M == 0 && op == Op::Dw && C == nullptr) return QALG_ERR_NULL;
  if ((A && !aligned16(A)) || (B && !aligned16(B)) || (C && !aligned16(C)) ||
      (tau && (reinterpret_cast<uintptr_t>(tau) & 3u)) || (adj && (reinterpret_cast<uintptr_t>(adj) & 7u)))
    return QALG_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (M == 0) {
    if (op != Op::Dw) return QALG_OK;
    return hip_status(qalg::launch_fill_zero(C, size_t(K) * size_t(N) * 2, s));
  }
  qalg_status st = check_ws(1, q, M, ws, ws_bytes);
  if (st != QALG_OK) return st;
  ProblemDesc p{};
  p.op = op;
  p.A = A;
  p.B = B;
  p.C = C;
  p.tau = tau;
  p.q = q;
  p.M = M;
  p.K = K;
  p.N = N;
  p.E = 1;
  p.graph_adj = adj;
  if (op == Op::Dw && ws_bytes >= qalg_workspace_bytes_dw(q, M, K, N))
    p.dw_part = static_cast<char*>(ws) + qalg_workspace_bytes(q, M);
  int32_t* wsi = static_cast<int32_t*>(ws);
  p.ws = wsi;
  p.ws_stride = ws_stride_ints(q, M);
  const bool ready = (flags & QALG_FLAG_INDEX_READY) != 0;
  if (op == Op::Fwd && qalg::fwd_persistent_shape_ok(p)) {
    if (!ready && qalg::launch_build_index(tau, q, M, 1, wsi, p.ws_stride, s) != hipSuccess) return QALG_ERR_HIP;
    if (qalg::launch_graph_zero_bf16(tau, adj, q, M, N, C, s) != hipSuccess) return QALG_ERR_HIP;
    return hip_status(qalg::launch_fwd_persistent_bf16(p, s));
  }
  hipError_t e;
  if (qalg::grad_persistent_supported(p)) {
    // dX zeroes the rows of an out-of-range type itself
    if (!ready && qalg::launch_build_index(tau, q, M, 1, wsi, p.ws_stride, s) != hipSuccess) return QALG_ERR_HIP;
    return hip_status(qalg::launch_grad_persistent_bf16(p, s));
  }
  // rows of an out-of-range type get zero Y / dX rows; dW ignores them
  void* zero_out = op == Op::Dw ? nullptr : C;
  const int64_t zero_ld = op == Op::Fwd ? N : K;
  if (!ready)
    e = qalg::launch_build_index_zeroing(tau, q, M, 1, wsi, p.ws_stride, zero_out, zero_ld, 2, M * zero_ld * 2, s);
  else if (zero_out != nullptr)
    e = qalg::launch_zero_bad_rows(wsi, q, M, 1, p.ws_stride, zero_out, zero_ld, 2, M * zero_ld * 2, s);
  else
    e = hipSuccess;
  if (e != hipSuccess) return QALG_ERR_HIP;
  return hip_status(qalg::launch_tiled_bf16(p, s));
}

// Shared driver of the unequal-width entry points (the complete-graph law on
// groups of widths in_widths / out_widths, eq 18; bf16, q <= 64): index, zero
// rows of out-of-range types, then the register-staged kernels.
qalg_status run_widths(Op op, const void* A, const void* B, const int32_t* tau, int32_t q, const int64_t* in_w,
                       const int64_t* out_w, int64_t M, int64_t K, int64_t N, void* C, int32_t dtype, void* ws,
                       size_t ws_bytes, uint32_t flags, void* stream) {
  if (dtype != QALG_BF16) return QALG_ERR_DTYPE;
  if (flags & ~uint32_t(QALG_FLAG_INDEX_READY)) return QALG_ERR_ARG;
  if (M < 0 || K <= 0 || N <= 0 || M > INT32_MAX / 2 || K > INT32_MAX / 2 || N > INT32_MAX / 2) return QALG_ERR_DIM;
  const int64_t lim = int64_t(1) << 31;
  if (M * K >= lim || K * N >= lim || M * N >= lim) return QALG_ERR_DIM;
  if (q < 1 || q > qalg::kMaxWidthGroups) return QALG_ERR_Q;
  if (in_w == nullptr || out_w == nullptr) return QALG_ERR_NULL;
  int64_t sk = 0, sn = 0;
  for (int g = 0; g < q; ++g) {
    if (in_w[g] <= 0 || out_w[g] <= 0) return QALG_ERR_DIM;
    if (in_w[g] % 8 || out_w[g] % 8) return QALG_ERR_ALIGN;
    sk += in_w[g];
    sn += out_w[g];
  }
  if (sk != K || sn != N) return QALG_ERR_DIM;
  if (M > 0 && (A == nullptr || B == nullptr || C == nullptr || tau == nullptr)) return QALG_ERR_NULL;
  if (M == 0 && op == Op::Dw && C == nullptr) return QALG_ERR_NULL;
  if ((A && !aligned16(A)) || (B && !aligned16(B)) || (C && !aligned16(C)) ||
      (tau && (reinterpret_cast<uintptr_t>(tau) & 3u)))
    return QALG_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (M == 0) {
    if (op != Op::Dw) return QALG_OK;
    return hip_status(qalg::launch_fill_zero(C, size_t(K) * size_t(N) * 2, s));
  }
  qalg_status st = check_ws(1, q, M, ws, ws_bytes);
  if (st != QALG_OK) return st;
  ProblemDesc p{};
  p.op = op;
  p.A = A;
  p.B = B;
  p.C = C;
  p.tau = tau;
  p.q = q;
  p.M = M;
  p.K = K;
  p.N = N;
  p.E = 1;
  p.in_widths = in_w;
  p.out_widths = out_w;
  if (op == Op::Dw && ws_bytes >= qalg_workspace_bytes_dw(q, M, K, N))
    p.dw_part = static_cast<char*>(ws) + qalg_workspace_bytes(q, M);
  int32_t* wsi = static_cast<int32_t*>(ws);
  p.ws = wsi;
  p.ws_stride = ws_stride_ints(q, M);
  hipError_t e;
  if (op == Op::Fwd && qalg::fwd_widths_persistent_ok(p)) {
    // the persistent forward zeroes the rows of an out-of-range type itself
    if (!(flags & QALG_FLAG_INDEX_READY) && qalg::launch_build_index(tau, q, M, 1, wsi, p.ws_stride, s) != hipSuccess)
      return QALG_ERR_HIP;
    return hip_status(qalg::launch_fwd_widths_bf16(p, s));
  }
  if (qalg::grad_persistent_supported(p)) {
    // dX zeroes the rows of an out-of-range type itself
    if (!(flags & QALG_FLAG_INDEX_READY) && qalg::launch_build_index(tau, q, M, 1, wsi, p.ws_stride, s) != hipSuccess)
      return QALG_ERR_HIP;
    return hip_status(qalg::launch_grad_persistent_bf16(p, s));
  }
  void* zero_out = op == Op::Dw ? nullptr : C;
  const int64_t zero_ld = op == Op::Fwd ? N : K;
  if (!(flags & QALG_FLAG_INDEX_READY))
    e = qalg::launch_build_index_zeroing(tau, q, M, 1, wsi, p.ws_stride, zero_out, zero_ld, 2, M * zero_ld * 2, s);
  else if (zero_out != nullptr)
    e = qalg::launch_zero_bad_rows(wsi, q, M, 1, p.ws_stride, zero_out, zero_ld, 2, M * zero_ld * 2, s);
  else
    e = hipSuccess;
  if (e != hipSuccess) return QALG_ERR_HIP;
  return hip_status(qalg::launch_tiled_bf16(p, s));
}

}  // namespace

extern "C" {

const char* qalg_status_string(int status) {
  switch (status) {
    case QALG_OK: return "QALG_OK";
    case QALG_ERR_NULL: return "QALG_ERR_NULL: a required pointer is NULL";
    case QALG_ERR_DIM: return "QALG_ERR_DIM: a size is negative, zero or too large";
    case QALG_ERR_Q: return "QALG_ERR_Q: q < 1, q > QALG_MAX_Q, or q does not divide K and N";
    case QALG_ERR_ALIGN: return "QALG_ERR_ALIGN: pointer or group width misaligned";
    case QALG_ERR_DTYPE: return "QALG_ERR_DTYPE: unknown element type";
    case QALG_ERR_WORKSPACE: return "QALG_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case QALG_ERR_HIP: return "QALG_ERR_HIP: a HIP launch or copy failed";
    case QALG_ERR_ARG: return "QALG_ERR_ARG: unknown flag, schedule or unsupported forced path";
    default: return "unknown qalg status";
  }
}

int qalg_version(void) { return QALG_VERSION; }

size_t qalg_workspace_bytes(int32_t q, int64_t M) {
  if (q < 1 || q > QALG_MAX_Q || M < 0 || M > INT32_MAX / 2) return 0;
  return size_t(qalg::ws_layout(q, M).total_ints) * sizeof(int32_t);
}

size_t qalg_workspace_bytes_two_stage(int32_t q, int64_t M, int64_t N) {
  const size_t base = qalg_workspace_bytes(q, M);
  if (base == 0 || N <= 0 || N > INT32_MAX / 2) return 0;
  return base + (size_t(M) * size_t(N) * sizeof(float) + 255) / 256 * 256;
}

size_t qalg_workspace_bytes_dw(int32_t q, int64_t M, int64_t K, int64_t N) {
  const size_t base = qalg_workspace_bytes(q, M);
  if (base == 0 || K <= 0 || N <= 0 || K > INT32_MAX / 2 || N > INT32_MAX / 2) return 0;
  return base + size_t(qalg::kDwMaxSplits) * size_t(K) * size_t(N) * sizeof(float);
}

qalg_status qalg_index_layout(int32_t q, int64_t M, int64_t out_offsets[4]) {
  if (q < 1 || q > QALG_MAX_Q) return QALG_ERR_Q;
  if (M < 0 || M > INT32_MAX / 2) return QALG_ERR_DIM;
  if (out_offsets == nullptr) return QALG_ERR_NULL;
  const qalg::WsLayout L = qalg::ws_layout(q, M);
  out_offsets[0] = 0;
  out_offsets[1] = L.counts;
  out_offsets[2] = L.offsets;
  out_offsets[3] = L.rows;
  return QALG_OK;
}

qalg_status qalg_type_schedule(const int64_t* positions, int64_t M, int32_t q, int32_t kind,
                               int64_t period, int32_t* tau, void* stream) {
  if (q < 1 || q > QALG_MAX_Q) return QALG_ERR_Q;
  if (M < 0 || M > INT32_MAX / 2) return QALG_ERR_DIM;
  if (kind != QALG_SCHEDULE_CYCLIC && kind != QALG_SCHEDULE_INTERVAL) return QALG_ERR_ARG;
  if (kind == QALG_SCHEDULE_INTERVAL && (period <= 0 || period % q)) return QALG_ERR_ARG;
  if (M == 0) return QALG_OK;
  if (positions == nullptr || tau == nullptr) return QALG_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(positions) & 7u) || (reinterpret_cast<uintptr_t>(tau) & 3u))
    return QALG_ERR_ALIGN;
  return hip_status(qalg::launch_type_schedule(positions, M, q, kind, period, tau,
                                               static_cast<hipStream_t>(stream)));
}

qalg_status qalg_build_index_batched(int32_t E, const int32_t* tau, int32_t q, int64_t M, void* ws,
                                     size_t ws_bytes, void* stream) {
  if (E < 1) return QALG_ERR_DIM;
  if (q < 1 || q > QALG_MAX_Q) return QALG_ERR_Q;
  if (M < 0 || M > INT32_MAX / 2) return QALG_ERR_DIM;
  if (M > 0 && tau == nullptr) return QALG_ERR_NULL;
  if (tau && (reinterpret_cast<uintptr_t>(tau) & 3u)) return QALG_ERR_ALIGN;
  const qalg_status st = check_ws(E, q, M, ws, ws_bytes);
  if (st != QALG_OK) return st;
  return hip_status(qalg::launch_build_index(tau, q, M, E, static_cast<int32_t*>(ws),
                                             ws_stride_ints(q, M), static_cast<hipStream_t>(stream)));
}

qalg_status qalg_build_index(const int32_t* tau, int32_t q, int64_t M, void* ws, size_t ws_bytes,
                             void* stream) {
  return qalg_build_index_batched(1, tau, q, M, ws, ws_bytes, stream);
}

qalg_status qalg_forward(const void* X, const void* W, const int32_t* tau, int32_t q, int64_t M,
                         int64_t K, int64_t N, void* Y, int32_t dtype, void* ws, size_t ws_bytes,
                         uint32_t flags, void* stream) {
  return run_projection(Op::Fwd, 1, X, W, tau, q, M, K, N, Y, dtype, ws, ws_bytes, flags, stream);
}

qalg_status qalg_forward_graph(const void* X, const void* W, const int32_t* tau, int32_t q,
                               const uint64_t* adjacency, int64_t M, int64_t K, int64_t N, void* Y,
                               int32_t dtype, void* ws, size_t ws_bytes, uint32_t flags, void* stream) {
  return run_graph(Op::Fwd, X, W, tau, q, adjacency, M, K, N, Y, dtype, ws, ws_bytes, flags, stream);
}

qalg_status qalg_backward_dx_graph(const void* dY, const void* W, const int32_t* tau, int32_t q,
                                   const uint64_t* adjacency, int64_t M, int64_t K, int64_t N, void* dX,
                                   int32_t dtype, void* ws, size_t ws_bytes, uint32_t flags, void* stream) {
  return run_graph(Op::Dx, dY, W, tau, q, adjacency, M, K, N, dX, dtype, ws, ws_bytes, flags, stream);
}

qalg_status qalg_backward_dw_graph(const void* X, const void* dY, const int32_t* tau, int32_t q,
                                   const uint64_t* adjacency, int64_t M, int64_t K, int64_t N, void* dW,
                                   int32_t dtype, void* ws, size_t ws_bytes, uint32_t flags, void* stream) {
  return run_graph(Op::Dw, X, dY, tau, q, adjacency, M, K, N, dW, dtype, ws, ws_bytes, flags, stream);
}

qalg_status qalg_forward_widths(const void* X, const void* W, const int32_t* tau, int32_t q,
                                const int64_t* in_widths, const int64_t* out_widths, int64_t M, int64_t K,
                                int64_t N, void* Y, int32_t dtype, void* ws, size_t ws_bytes, uint32_t flags,
                                void* stream) {
  return run_widths(Op::Fwd, X, W, tau, q, in_widths, out_widths, M, K, N, Y, dtype, ws, ws_bytes, flags, stream);
}

qalg_status qalg_backward_dx_widths(const void* dY, const void* W, const int32_t* tau, int32_t q,
                                    const int64_t* in_widths, const int64_t* out_widths, int64_t M, int64_t K,
                                    int64_t N, void* dX, int32_t dtype, void* ws, size_t ws_bytes, uint32_t flags,
                                    void* stream) {
  return run_widths(Op::Dx, dY, W, tau, q, in_widths, out_widths, M, K, N, dX, dtype, ws, ws_bytes, flags, stream);
}

qalg_status qalg_backward_dw_widths(const void* X, const void* dY, const int32_t* tau, int32_t q,
                                    const int64_t* in_widths, const int64_t* out_widths, int64_t M, int64_t K,
                                    int64_t N, void* dW, int32_t dtype, void* ws, size_t ws_bytes, uint32_t flags,
                                    void* stream) {
  return run_widths(Op::Dw, X, dY, tau, q, in_widths, out_widths, M, K, N, dW, dtype, ws, ws_bytes, flags, stream);
}

qalg_status qalg_backward_dx(const void* dY, const void* W, const int32_t* tau, int32_t q,
                             int64_t M, int64_t K, int64_t N, void* dX, int32_t dtype, void* ws,
                             size_t ws_bytes, uint32_t flags, void* stream) {
  if (flags & QALG_FLAG_FORCE_SMALL_M) return QALG_ERR_ARG;
  return run_projection(Op::Dx, 1, dY, W, tau, q, M, K, N, dX, dtype, ws, ws_bytes, flags, stream);
}

qalg_status qalg_backward_dw(const void* X, const void* dY, const int32_t* tau, int32_t q,
                             int64_t M, int64_t K, int64_t N, void* dW, int32_t dtype, void* ws,
                             size_t ws_bytes, uint32_t flags, void* stream) {
  if (flags & QALG_FLAG_FORCE_SMALL_M) return QALG_ERR_ARG;
  return run_projection(Op::Dw, 1, X, dY, tau, q, M, K, N, dW, dtype, ws, ws_bytes, flags, stream);
}

qalg_status qalg_forward_batched(int32_t E, const void* X, const void* W, const int32_t* tau,
                                 int32_t q, int64_t M, int64_t K, int64_t N, void* Y,
                                 int32_t dtype, void* ws, size_t ws_bytes, uint32_t flags,
                                 void* stream) {
  return run_projection(Op::Fwd, E, X, W, tau, q, M, K, N, Y, dtype, ws, ws_bytes, flags, stream);
}

namespace {
// shared by the gated forward and its variant that keeps the pre-activations (GU may be null)
qalg_status run_gated(const void* X, const void* Wgu, const int32_t* tau, int32_t q, int64_t M, int64_t K,
                      int64_t F, void* H, void* GU, int32_t dtype, void* ws, size_t ws_bytes, uint32_t flags,
                      void* stream);
}  // namespace

qalg_status qalg_gated_forward(const void* X, const void* Wgu, const int32_t* tau, int32_t q, int64_t M,
                               int64_t K, int64_t F, void* H, int32_t dtype, void* ws, size_t ws_bytes,
                               uint32_t flags, void* stream) {
  return run_gated(X, Wgu, tau, q, M, K, F, H, nullptr, dtype, ws, ws_bytes, flags, stream);
}

qalg_status qalg_gated_forward_keep(const void* X, const void* Wgu, const int32_t* tau, int32_t q, int64_t M,
                                    int64_t K, int64_t F, void* H, void* GU, int32_t dtype, void* ws,
                                    size_t ws_bytes, uint32_t flags, void* stream) {
  if (M > 0 && GU == nullptr) return QALG_ERR_NULL;
  if (GU != nullptr && !aligned16(GU)) return QALG_ERR_ALIGN;
  return run_gated(X, Wgu, tau, q, M, K, F, H, GU, dtype, ws, ws_bytes, flags, stream);
}

namespace {
qalg_status run_gated(const void* X, const void* Wgu, const int32_t* tau, int32_t q, int64_t M, int64_t K,
                      int64_t F, void* H, void* GU, int32_t dtype, void* ws, size_t ws_bytes, uint32_t flags,
                      void* stream) {
  if (dtype != QALG_BF16) return QALG_ERR_DTYPE;
  if (flags & ~uint32_t(QALG_FLAG_INDEX_READY | QALG_FLAG_LAW_TENSOR)) return QALG_ERR_ARG;
  if (M < 0 || K <= 0 || F <= 0 || M > INT32_MAX / 2 || K > INT32_MAX / 2 || F > INT32_MAX / 4)
    return QALG_ERR_DIM;
  if (q < 1 || q > QALG_MAX_Q || K % q || F % q) return QALG_ERR_Q;
  if ((flags & QALG_FLAG_LAW_TENSOR) && tensor_levels(q) < 0) return QALG_ERR_Q;
  if ((F / q) % 128 || (K / q) % 64) return QALG_ERR_ALIGN;
  if (M == 0) return QALG_OK;
  if (X == nullptr || Wgu == nullptr || tau == nullptr || H == nullptr) return QALG_ERR_NULL;
  if (!aligned16(X) || !aligned16(Wgu) || !aligned16(H) || (reinterpret_cast<uintptr_t>(tau) & 3u))
    return QALG_ERR_ALIGN;
  qalg_status st = check_ws(1, q, M, ws, ws_bytes);
  if (st != QALG_OK) return st;
  ProblemDesc p{};
  p.op = Op::Fwd;
  p.A = X;
  p.B = Wgu;
  p.C = H;
  p.tau = tau;
  p.q = q;
  p.M = M;
  p.K = K;
  p.N = 2 * F;  // the merged bank's width
  p.E = 1;
  p.law_L = (flags & QALG_FLAG_LAW_TENSOR) ? tensor_levels(q) : 0;
  if (!qalg::fwd_gated_supported(p)) return QALG_ERR_DIM;
  int32_t* wsi = static_cast<int32_t*>(ws);
  p.ws = wsi;
  p.ws_stride = ws_stride_ints(q, M);
  hipStream_t s = static_cast<hipStream_t>(stream);
  p.gu = GU;
  if (!(flags & QALG_FLAG_INDEX_READY)) {
    const hipError_t e = qalg::launch_build_index(tau, q, M, 1, wsi, p.ws_stride, s);
    if (e != hipSuccess) return QALG_ERR_HIP;
  }
  return hip_status(qalg::launch_fwd_gated_bf16(p, s));
}
}  // namespace

qalg_status qalg_merge_gate_up(const void* Wg, const void* Wu, int32_t q, int64_t K, int64_t F, void* Wgu,
                               int32_t dtype, void* stream) {
  if (dtype != QALG_BF16) return QALG_ERR_DTYPE;
  if (K <= 0 || F <= 0 || K > INT32_MAX / 2 || F > INT32_MAX / 4) return QALG_ERR_DIM;
  if (q < 1 || q > QALG_MAX_Q || F % q) return QALG_ERR_Q;
  if ((F / q) % 128) return QALG_ERR_ALIGN;
  if (Wg == nullptr || Wu == nullptr || Wgu == nullptr) return QALG_ERR_NULL;
  if (!aligned16(Wg) || !aligned16(Wu) || !aligned16(Wgu)) return QALG_ERR_ALIGN;
  return hip_status(qalg::launch_merge_gate_up_bf16(Wg, Wu, Wgu, K, F, q, static_cast<hipStream_t>(stream)));
}

qalg_status qalg_split_gate_up(const void* Wgu, int32_t q, int64_t K, int64_t F, void* Wg, void* Wu,
                               int32_t dtype, void* stream) {
  if (dtype != QALG_BF16) return QALG_ERR_DTYPE;
  if (K <= 0 || F <= 0 || K > INT32_MAX / 2 || F > INT32_MAX / 4) return QALG_ERR_DIM;
  if (q < 1 || q > QALG_MAX_Q || F % q) return QALG_ERR_Q;
  if ((F / q) % 128) return QALG_ERR_ALIGN;
  if (Wgu == nullptr || Wg == nullptr || Wu == nullptr) return QALG_ERR_NULL;
  if (!aligned16(Wgu) || !aligned16(Wg) || !aligned16(Wu)) return QALG_ERR_ALIGN;
  return hip_status(qalg::launch_split_gate_up_bf16(Wgu, Wg, Wu, K, F, q, static_cast<hipStream_t>(stream)));
}

// shared checks of the two pointwise SwiGLU entry points
static qalg_status check_swiglu(int32_t q, int64_t M, int64_t F, int32_t dtype) {
  if (dtype != QALG_BF16) return QALG_ERR_DTYPE;
  if (M < 0 || F <= 0 || F > INT32_MAX / 4) return QALG_ERR_DIM;
  if (q < 1 || q > QALG_MAX_Q || F % q) return QALG_ERR_Q;
  if ((F / q) % 128) return QALG_ERR_ALIGN;
  return QALG_OK;
}

qalg_status qalg_swiglu_forward(const void* GU, int32_t q, int64_t M, int64_t F, void* H, int32_t dtype,
                                void* stream) {
  if (qalg_status st = check_swiglu(q, M, F, dtype)) return st;
  if (M == 0) return QALG_OK;
  if (GU == nullptr || H == nullptr) return QALG_ERR_NULL;
  if (!aligned16(GU) || !aligned16(H)) return QALG_ERR_ALIGN;
  return hip_status(qalg::launch_swiglu_fwd_bf16(GU, H, M, F, q, static_cast<hipStream_t>(stream)));
}

qalg_status qalg_swiglu_backward(const void* GU, const void* dH, int32_t q, int64_t M, int64_t F, void* dGU,
                                 int32_t dtype, void* stream) {
  if (qalg_status st = check_swiglu(q, M, F, dtype)) return st;
  if (M == 0) return QALG_OK;
  if (GU == nullptr || dH == nullptr || dGU == nullptr) return QALG_ERR_NULL;
  if (!aligned16(GU) || !aligned16(dH) || !aligned16(dGU)) return QALG_ERR_ALIGN;
  return hip_status(qalg::launch_swiglu_bwd_bf16(GU, dH, dGU, M, F, q, static_cast<hipStream_t>(stream)));
}

qalg_status qalg_attention_forward(const void* Q, const void* K, const void* V, int32_t Hq, int32_t Hkv,
                                   int64_t S, int32_t d, int32_t q, void* O, int32_t dtype, uint32_t flags,
                                   void* stream) {
  return qalg_attention_forward_at(Q, K, V, Hq, Hkv, S, d, q, 0, O, dtype, flags, stream);
}

qalg_status qalg_attention_forward_at(const void* Q, const void* K, const void* V, int32_t Hq, int32_t Hkv,
                                      int64_t S, int32_t d, int32_t q, int64_t first_position, void* O,
                                      int32_t dtype, uint32_t flags, void* stream) {
  if (first_position < 0) return QALG_ERR_DIM;
  if (dtype != QALG_BF16) return QALG_ERR_DTYPE;
  if (flags & ~uint32_t(QALG_FLAG_LAW_TENSOR)) return QALG_ERR_ARG;
  if (Hq < 1 || Hkv < 1 || Hq % Hkv || S < 0 || (d != 64 && d != 128)) return QALG_ERR_DIM;
  if (S * int64_t(d) * 2 >= (int64_t(1) << 31)) return QALG_ERR_DIM;  // a head's rows: 32-bit byte offsets
  if (q < 1 || q > QALG_MAX_Q || d % q) return QALG_ERR_Q;
  const int L = (flags & QALG_FLAG_LAW_TENSOR) ? tensor_levels(q) : 0;
  if (L < 0) return QALG_ERR_Q;
  if (!qalg::attn_supported(d, q)) return QALG_ERR_ALIGN;
  if (S == 0) return QALG_OK;
  if (Q == nullptr || K == nullptr || V == nullptr || O == nullptr) return QALG_ERR_NULL;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return QALG_ERR_ALIGN;
  return hip_status(
      qalg::launch_attn_fwd_bf16(Q, K, V, O, Hq, Hkv, S, d, q, L, first_position, static_cast<hipStream_t>(stream)));
}

// the checks every attention entry shares; L receives the law's level count
static qalg_status attn_check(int32_t Hq, int32_t Hkv, int64_t S, int32_t d, int32_t q, int64_t first_position,
                              int32_t dtype, uint32_t flags, int* L) {
  if (first_position < 0) return QALG_ERR_DIM;
  if (dtype != QALG_BF16) return QALG_ERR_DTYPE;
  if (flags & ~uint32_t(QALG_FLAG_LAW_TENSOR)) return QALG_ERR_ARG;
  if (Hq < 1 || Hkv < 1 || Hq % Hkv || S < 0 || (d != 64 && d != 128)) return QALG_ERR_DIM;
  if (S * int64_t(d) * 2 >= (int64_t(1) << 31)) return QALG_ERR_DIM;  // a head's rows: 32-bit byte offsets
  if (q < 1 || q > QALG_MAX_Q || d % q) return QALG_ERR_Q;
  *L = (flags & QALG_FLAG_LAW_TENSOR) ? tensor_levels(q) : 0;
  if (*L < 0) return QALG_ERR_Q;
  if (!qalg::attn_supported(d, q)) return QALG_ERR_ALIGN;
  return QALG_OK;
}

qalg_status qalg_attention_forward_train(const void* Q, const void* K, const void* V, int32_t Hq, int32_t Hkv,
                                         int64_t S, int32_t d, int32_t q, int64_t first_position, void* O, float* lse,
                                         int32_t dtype, uint32_t flags, void* stream) {
  int L = 0;
  const qalg_status st = attn_check(Hq, Hkv, S, d, q, first_position, dtype, flags, &L);
  if (st != QALG_OK) return st;
  if (S == 0) return QALG_OK;
  if (Q == nullptr || K == nullptr || V == nullptr || O == nullptr || lse == nullptr) return QALG_ERR_NULL;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || reinterpret_cast<uintptr_t>(lse) % 4)
    return QALG_ERR_ALIGN;
  return hip_status(qalg::launch_attn_fwd_lse_bf16(Q, K, V, O, lse, Hq, Hkv, S, d, q, L, first_position,
                                                   static_cast<hipStream_t>(stream)));
}

size_t qalg_attention_backward_workspace_bytes(int32_t Hq, int32_t Hkv, int64_t S, int32_t d, int32_t q) {
  if (Hq < 1 || Hkv < 1 || Hq % Hkv || S < 0 || (d != 64 && d != 128) || q < 1 || q > QALG_MAX_Q) return 0;
  const size_t n = qalg::attn_bwd_ws_bytes(Hq, Hkv, S, d, q);
  return (n + 255) / 256 * 256;
}

qalg_status qalg_attention_backward(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                                    const float* lse, int32_t Hq, int32_t Hkv, int64_t S, int32_t d, int32_t q,
                                    int64_t first_position, void* dQ, void* dK, void* dV, int32_t dtype, void* ws,
                                    size_t ws_bytes, uint32_t flags, void* stream) {
  int L = 0;
  const qalg_status st = attn_check(Hq, Hkv, S, d, q, first_position, dtype, flags, &L);
  if (st != QALG_OK) return st;
  if (S == 0) return QALG_OK;
  if (Q == nullptr || K == nullptr || V == nullptr || O == nullptr || dO == nullptr || lse == nullptr ||
      dQ == nullptr || dK == nullptr || dV == nullptr || ws == nullptr)
    return QALG_ERR_NULL;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(dO) || !aligned16(dQ) ||
      !aligned16(dK) || !aligned16(dV) || reinterpret_cast<uintptr_t>(lse) % 4)
    return QALG_ERR_ALIGN;
  if (!aligned16(ws) || ws_bytes < qalg_attention_backward_workspace_bytes(Hq, Hkv, S, d, q)) return QALG_ERR_WORKSPACE;
  return hip_status(qalg::launch_attn_bwd_bf16(Q, K, V, O, dO, lse, dQ, dK, dV, ws, Hq, Hkv, S, d, q, L,
                                               first_position, static_cast<hipStream_t>(stream)));
}

size_t qalg_attention_decode_workspace_bytes(int32_t B, int32_t Hq, int64_t N, int32_t d) {
  if (B < 0 || Hq < 1 || N < 1 || (d != 64 && d != 128)) return 0;
  const size_t n = qalg::attn_decode_part_bytes(B, Hq, N, d);
  return (n + 255) / 256 * 256;
}

qalg_status qalg_attention_decode(const void* Qn, const void* Kc, const void* Vc, const int64_t* q_pos,
                                  const int64_t* key_pos, int32_t B, int32_t Hq, int32_t Hkv, int64_t N, int32_t d,
                                  int32_t q, int32_t kind, int64_t period, void* O, int32_t dtype, void* ws,
                                  size_t ws_bytes, uint32_t flags, void* stream) {
  if (dtype != QALG_BF16) return QALG_ERR_DTYPE;
  if (flags & ~uint32_t(QALG_FLAG_LAW_TENSOR)) return QALG_ERR_ARG;
  if (B < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv || Hq / Hkv > 8 || N < 1 || (d != 64 && d != 128)) return QALG_ERR_DIM;
  if (B > 65535 || Hkv > 65535 || int64_t(B) * Hq > INT32_MAX || N > qalg::attn_decode_max_slots()) return QALG_ERR_DIM;
  if (q < 1 || q > QALG_MAX_Q || d % q) return QALG_ERR_Q;
  const int L = (flags & QALG_FLAG_LAW_TENSOR) ? tensor_levels(q) : 0;
  if (L < 0) return QALG_ERR_Q;
  if (!qalg::attn_decode_supported(d, q)) return QALG_ERR_ALIGN;
  if (kind != QALG_SCHEDULE_CYCLIC && kind != QALG_SCHEDULE_INTERVAL) return QALG_ERR_ARG;
  if (kind == QALG_SCHEDULE_INTERVAL && (period <= 0 || period % q)) return QALG_ERR_ARG;
  if (B == 0) return QALG_OK;
  if (Qn == nullptr || Kc == nullptr || Vc == nullptr || q_pos == nullptr || key_pos == nullptr || O == nullptr)
    return QALG_ERR_NULL;
  if (!aligned16(Qn) || !aligned16(Kc) || !aligned16(Vc) || !aligned16(O) ||
      (reinterpret_cast<uintptr_t>(q_pos) & 7u) || (reinterpret_cast<uintptr_t>(key_pos) & 7u))
    return QALG_ERR_ALIGN;
  if (ws == nullptr) return QALG_ERR_NULL;
  if (!aligned16(ws) || ws_bytes < qalg_attention_decode_workspace_bytes(B, Hq, N, d)) return QALG_ERR_WORKSPACE;
  return hip_status(qalg::launch_attn_decode_bf16(Qn, Kc, Vc, q_pos, key_pos, O, B, Hq, Hkv, N, d, q, L, kind, period,
                                                  ws, static_cast<hipStream_t>(stream)));
}

qalg_status qalg_read_status(const void* ws, int32_t E, int32_t q, int64_t M, void* stream,
                             int64_t* bad_tau_rows) {
  if (ws == nullptr || bad_tau_rows == nullptr) return QALG_ERR_NULL;
  if (E < 1 || M < 0 || M > INT32_MAX / 2) return QALG_ERR_DIM;
  if (q < 1 || q > QALG_MAX_Q) return QALG_ERR_Q;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t pitch = size_t(ws_stride_ints(q, M)) * sizeof(int32_t);
  int64_t total = 0;
  for (int32_t e = 0; e < E; ++e) {
    int32_t v = 0;
    if (hipMemcpyAsync(&v, static_cast<const char*>(ws) + e * pitch, sizeof(v),
                       hipMemcpyDeviceToHost, s) != hipSuccess)
      return QALG_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return QALG_ERR_HIP;
    total += v;
  }
  *bad_tau_rows = total;
  return QALG_OK;
}

}  // extern "C"
