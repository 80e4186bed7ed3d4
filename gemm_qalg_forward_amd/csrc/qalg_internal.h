// Internal declarations shared by the libqalg translation units: the workspace
// layout of the type index and the host-side launchers each kernel file exports.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qalg {

// Row-tile heights the index precomputes prefix sums for (tiled kernels pick one).
constexpr int kNumTileHeights = 5;
constexpr int kTileHeights[kNumTileHeights] = {16, 32, 64, 128, 256};
constexpr int tile_height_slot(int bm) {
  return bm == 16 ? 0 : bm == 32 ? 1 : bm == 64 ? 2 : bm == 128 ? 3 : bm == 256 ? 4 : -1;
}

// Workspace of one problem, in int32 elements:
//   [0]            rows with an out-of-range type
//   [1]            magic (kIndexMagic) once an index was written
//   [2], [3]       q and M of that index
//   [4]            o >= 0 if the schedule is cyclic, tau[m] = (o + m) mod q for
//                  every row (then the k-th row of type i is (i - o) mod q + k q);
//                  -1 otherwise
//   [16, 16+q)     counts[q]                 (M_i)
//   [.., +q+1)     offsets[q+1]              (running sums of counts)
//   [.., +5(q+1))  tile_off[5][q+1]          (running sums of ceil(M_i / BM))
//   [rows, +M)     rows[M]                   (rows of type 0, 1, ..., then bad rows)
//   then at least 64 spare ints, so that kernels may read row ids in whole
//   groups of up to 64 past the end of the list (the extra ids are never used)
constexpr int32_t kIndexMagic = 0x51414c47;  // "QALG"

struct WsLayout {
  int64_t counts, offsets, tile_off, rows, total_ints;
};

inline WsLayout ws_layout(int q, int64_t M) {
  WsLayout L;
  L.counts = 16;
  L.offsets = L.counts + q;
  L.tile_off = L.offsets + (q + 1);
  int64_t end = L.tile_off + int64_t(kNumTileHeights) * (q + 1);
  L.rows = (end + 15) / 16 * 16;
  L.total_ints = (L.rows + M + 64 + 63) / 64 * 64;
  return L;
}

// ---- launchers (return hipError_t of the launch) ----

hipError_t launch_type_schedule(const int64_t* pos, int64_t M, int q, int kind, int64_t period,
                                int32_t* tau, hipStream_t s);
hipError_t launch_build_index(const int32_t* tau, int q, int64_t M, int E, int32_t* ws,
                              int64_t ws_stride_ints, hipStream_t s);
// Same, and zero the output rows (row length zero_ld elements of zero_elem_bytes)
// whose type is out of range, in each problem's output (zero_stride_bytes apart).
hipError_t launch_build_index_zeroing(const int32_t* tau, int q, int64_t M, int E, int32_t* ws,
                                      int64_t ws_stride_ints, void* zero_out, int64_t zero_ld,
                                      int zero_elem_bytes, int64_t zero_stride_bytes,
                                      hipStream_t s);
// Zero `bytes` bytes (a multiple of 4) at p with a kernel (no memset node in captured graphs).
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
// Zero those rows from an index built earlier.
hipError_t launch_zero_bad_rows(const int32_t* ws, int q, int64_t M, int E, int64_t ws_stride_ints,
                                void* out, int64_t ld, int elem_bytes, int64_t stride_bytes,
                                hipStream_t s);

enum class Op { Fwd = 0, Dx = 1, Dw = 2 };

struct ProblemDesc {
  Op op;
  const void* A;      // fwd: X;  dx: dY;  dw: X
  const void* B;      // fwd: W;  dx: W;   dw: dY
  void* C;            // fwd: Y;  dx: dX;  dw: dW
  const int32_t* tau; // types of problem 0 (small-M path reads them directly)
  const int32_t* ws;  // index of problem 0
  int64_t ws_stride;  // int32 elements between the indices of consecutive problems
  int q;
  int64_t M, K, N;
  int E;              // problems (experts); operands packed back to back
  int law_L = 0;      // 0: the complete-graph law Q_q; L >= 1: the recursive law Q_2^(x)L, q = 2^L
  void* dw_part = nullptr;  // dW on the register-staged path: fp32 scratch for a split contraction
  const uint64_t* graph_adj = nullptr;  // graph law Q_G: per-type out-edge masks (device; q <= 64)
  const int64_t* in_widths = nullptr;   // unequal group widths (host arrays of q; sums K and N)
  const int64_t* out_widths = nullptr;
  void* gu = nullptr;                   // gated forward: also store the merged pre-activations here
  void* fwd_diag = nullptr;             // two-stage forward: fp32 diagonal maps, M x N per problem
};

// dW's split contraction (register-staged path): at most this many partial tiles per output tile
constexpr int kDwMaxSplits = 16;
// unequal group widths: at most this many groups (the tables ride in the kernel arguments)
constexpr int kMaxWidthGroups = 64;

hipError_t launch_tiled_bf16(const ProblemDesc& p, hipStream_t s);
hipError_t launch_tiled_f32(const ProblemDesc& p, hipStream_t s);
// the two-stage forward (diagonal maps over all rows into p.fwd_diag, then the strips); bf16, complete law
hipError_t launch_tiled_two_stage_bf16(const ProblemDesc& p, hipStream_t s);
// the masked forward (one tile over all rows, every block once, masked per row); bf16, complete law
hipError_t launch_tiled_masked_bf16(const ProblemDesc& p, hipStream_t s);
hipError_t launch_small_m_bf16(const ProblemDesc& p, hipStream_t s);
bool small_m_supported(const ProblemDesc& p);
// Persistent 256x256-tile forward (bf16, one problem); zeroes rows of out-of-range type itself.
bool fwd_persistent_supported(const ProblemDesc& p);
// unequal group widths on the persistent forward (256x256 tiles; see the shape rule there)
bool fwd_widths_persistent_ok(const ProblemDesc& p);
hipError_t launch_fwd_widths_bf16(const ProblemDesc& p, hipStream_t s);
// the shapes the persistent forward can run at all (the only path of the recursive law)
bool fwd_persistent_shape_ok(const ProblemDesc& p);
// forced_bm: 0 picks the tile height from the rows per type; 256, 128 or 64 forces it
hipError_t launch_fwd_persistent_bf16(const ProblemDesc& p, hipStream_t s, int forced_bm = 0);
// tile height the persistent forward uses (forced_bm as above); 0 if the forced one cannot run
int fwd_tile_height(const ProblemDesc& p, int forced_bm);
// Gated (SwiGLU gate/up) forward over a merged bank; p.N is the merged width 2F.
bool fwd_gated_supported(const ProblemDesc& p);
hipError_t launch_fwd_gated_bf16(const ProblemDesc& p, hipStream_t s);
// graph law: zero the output blocks of absent edges (before the forward)
hipError_t launch_graph_zero_bf16(const int32_t* tau, const uint64_t* adj, int q, int64_t M, int64_t out_n,
                                  void* Y, hipStream_t s);
hipError_t launch_merge_gate_up_bf16(const void* Wg, const void* Wu, void* Wgu, int64_t K, int64_t F, int q,
                                     hipStream_t s);
// pointwise SwiGLU pieces on the merged gate/up layout (qalg_act.hip)
hipError_t launch_swiglu_fwd_bf16(const void* GU, void* H, int64_t M, int64_t F, int q, hipStream_t s);
hipError_t launch_swiglu_bwd_bf16(const void* GU, const void* dH, void* dGU, int64_t M, int64_t F, int q,
                                  hipStream_t s);
hipError_t launch_split_gate_up_bf16(const void* Wgu, void* Wg, void* Wu, int64_t K, int64_t F, int q,
                                     hipStream_t s);

// causal attention with the algebraic score, forward (qalg_attn.hip)
bool attn_supported(int d, int q);
hipError_t launch_attn_fwd_bf16(const void* Q, const void* K, const void* V, void* O, int Hq, int Hkv, int64_t S,
                                int d, int q, int L, int64_t first_pos, hipStream_t s);
// the forward that also stores each query's log-sum-exp (Hq x S fp32), for the backward
hipError_t launch_attn_fwd_lse_bf16(const void* Q, const void* K, const void* V, void* O, float* lse, int Hq,
                                    int Hkv, int64_t S, int d, int q, int L, int64_t first_pos, hipStream_t s);
// the backward's per-query (lse, D) scratch, and the two backward kernels
size_t attn_bwd_stat_bytes(int64_t Hq, int64_t S, int q);
size_t attn_bwd_ws_bytes(int64_t Hq, int64_t Hkv, int64_t S, int d, int q);  // the stat pairs and the head-share sums
hipError_t launch_attn_bwd_bf16(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                                const float* lse, void* dQ, void* dK, void* dV, void* stat, int Hq, int Hkv,
                                int64_t S, int d, int q, int L, int64_t first_pos, hipStream_t s);
// cached decoding (Algorithm 3): per-chunk partials in `part`, then their ordered combination into O
bool attn_decode_supported(int d, int q);
int64_t attn_decode_max_slots();  // cache slots per sequence the decode kernels take
size_t attn_decode_part_bytes(int64_t B, int64_t Hq, int64_t N, int d);
hipError_t launch_attn_decode_bf16(const void* Q, const void* K, const void* V, const int64_t* q_pos,
                                   const int64_t* key_pos, void* O, int B, int Hq, int Hkv, int64_t N, int d, int q,
                                   int L, int kind, int64_t period, void* part, hipStream_t s);
// Persistent 256-row-tile dX / dW (bf16, one problem) for cyclic schedules; a
// launch on any other schedule returns at once.
bool grad_persistent_supported(const ProblemDesc& p);
hipError_t launch_grad_persistent_bf16(const ProblemDesc& p, hipStream_t s);

}  // namespace qalg
