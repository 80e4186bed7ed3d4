// Tiled matrix-core kernels of the row-typed Q_q projection (bf16 in, fp32
// accumulate, bf16 out) for gfx950.
//
// Paper: arXiv 2609.32814.  Forward: section 4, eq 16-17, and Algorithm 1
// (section 6.1): a row of type i gets y_i = x_i W_ii and y_j = x_i W_ij +
// x_j W_jj.  Section 5.3 describes the fused schedule used here: an output
// tile sums both endpoint products in registers and is stored once.  Gradients:
// appendix B, eq 31-35, with one owner per output element (section 5.3).
//
// Every output tile is an ordinary GEMM tile whose contraction runs over at
// most two segments of the feature axis:
//   forward  Y[I_i, cols of group j]  : X[I_i, g_i] W[g_i, .] (+ X[I_i, g_j] W[g_j, .] if j != i)
//   dX       dX[I_i, cols of group k] : dY[I_i, all N] W[g_i, :]^T if k == i,
//                                       dY[I_i, group k] W[g_k, g_k]^T otherwise
//   dW       dW[g_b, g_j]             : X[R, g_b]^T dY[R, g_j], R = all typed rows if b == j,
//                                       else the rows of type b
// Absent block products are never visited: they are simply not in a tile's
// segment list.  Rows of a type are addressed through the index's row list
// (a gather for arbitrary types; for a cyclic schedule the list is the
// arithmetic progression start + k*q, i.e. strided rows).
//
// Data movement.  Operands go global -> registers -> LDS (double buffered,
// one barrier per k-step) -> MFMA.  Both LDS tiles are stored
// contraction-contiguous in 16-byte chunks so that each lane fetches one
// 8-element MFMA operand with a single 128-bit LDS read; chunk positions are
// XOR-swizzled by row to spread a wave's reads over the LDS banks.  Operands
// whose contraction axis is the slow axis in memory (W in the forward, X and
// dY in dW) are loaded as 8x8 blocks and transposed in registers on the way
// into LDS.  The MFMA is v_mfma_f32_32x32x16_bf16 with the operands swapped
// (the weight-side tile as the first operand) so that each lane ends with
// four consecutive output columns of one row; the lane halves exchange pieces
// (v_permlane32_swap) so that each lane stores 16 contiguous bytes.
#include <type_traits>

#include "qalg_device.h"
#include "qalg_internal.h"

namespace qalg {

namespace {

using dev::law_member;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <int BM_, int BN_, int BK_, int WGM_, int WGN_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WGM = WGM_, WGN = WGN_;
  static constexpr int THREADS = 64 * WGM * WGN;
  static constexpr int WTM = BM / WGM, WTN = BN / WGN;  // wave tile
  static constexpr int FM = WTM / 32, FN = WTN / 32;    // 32x32 MFMA tiles per wave
  static constexpr int KCH = BK / 8;                    // 16-byte chunks per LDS row
  static_assert(FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  static_assert(BK == 32 || BK == 64 || BK == 128, "BK");
  static constexpr int A_CHUNKS = BM * KCH;             // 16-byte chunks of a K-major A tile
  static constexpr int B_CHUNKS = BN * KCH;
  static constexpr int A_BLOCKS = (BM / 8) * KCH;       // 8x8 blocks of an MN-major tile
  static constexpr int B_BLOCKS = (BN / 8) * KCH;
  static constexpr int STAGE = (BM + BN) * BK;          // bf16 elements per LDS stage
};

struct Args {
  const uint16_t* A;
  const uint16_t* B;
  uint16_t* C;
  const int32_t* ws;
  int64_t ws_stride;                 // int32 elements between problems' indices
  int64_t strideA, strideB, strideC; // elements between problems' operands
  int64_t off_offsets, off_tiles, off_rows;
  int q, M, K, N, s, r;
  int ct_per_group;                  // column tiles per output group
  int n_ct;                          // all column tiles (q * ct_per_group)
  int tm_dw, tn_dw;                  // dW: tiles per block along rows / columns
  int L;                             // recursive law Q_2^(x)L (TENSOR kernels); 0 otherwise
  const uint64_t* adj;               // graph law Q_G (GRAPH kernels): out-edge mask of each type
  // unequal group widths (WIDTHS kernels, q <= kMaxWidthGroups): group starts
  // along K (gk) and N (gn), and prefix counts of the tiles of each group along
  // the tiled output axes (rows of dW: tk; columns of Y, dW: tn; columns of dX: tk)
  int gk[kMaxWidthGroups + 1], gn[kMaxWidthGroups + 1];
  int tk[kMaxWidthGroups + 1], tn[kMaxWidthGroups + 1];
  float* part;                       // dW split contraction: fp32 partial tiles [splits][K][N]
  int splits;                        // dW: workgroups per output tile (1: no split)
  float* D;                          // two-stage forward: the diagonal maps of every row, fp32 [M][N]
  const int32_t* tau;                // kMasked forward: the row types (E x M)
  int64_t strideD;                   // elements between problems' D
};

// Recursive law Q_2^(x)L (appendix C, eq 36): b is in the support of (i, j)
// when every bit of b equals i's or j's.  Hence, transposed for the VJPs:
//   dX[I_i, g_b] sums over the output groups j that agree with b wherever b
//     differs from i (2^(L - |i ^ b|) groups);
//   dW[g_b, g_j] sums over the rows of the types i that agree with b wherever
//     b differs from j (2^(L - |b ^ j|) types).
// In both, segment n fixes the free bits (the bits where the two given indices
// agree) to n's bits in order (law_member).

// Graph law Q_G (section 3.1, eq 9-12): B(i, i) = {i}, B(i, j) = {i, j} when
// (i, j) is an edge and empty otherwise.  Transposed for the VJPs:
//   dX[I_i, g_i] sums over the output groups {i} and the out-neighbours of i;
//   dX[I_i, g_k] (k != i) is dY[I_i, g_k] W_kk^T on an edge (i, k), else 0;
//   dW[g_j, g_j] sums over the rows of type j and of the in-neighbours of j;
//   dW[g_b, g_j] (b != j) sums over the rows of type b on an edge (b, j), else 0.
__device__ __forceinline__ bool graph_edge(const uint64_t* adj, int i, int j) { return (adj[i] >> j) & 1ull; }

__device__ __forceinline__ uint64_t graph_in_mask(const uint64_t* adj, int q, int j) {
  uint64_t m = 1ull << j;
  for (int i = 0; i < q; ++i) m |= ((adj[i] >> j) & 1ull) << i;
  return m;
}

__device__ __forceinline__ int swz(int row, int chunk, int kch) {
  return chunk ^ (((row & 7) ^ ((row >> 3) & 1)) & (kch - 1));
}

// 8x8 transpose of 16-bit elements held as 8 rows of 4 dwords: out[c] holds
// column c of the input as 8 elements (pairs of consecutive rows per dword).
__device__ __forceinline__ void transpose8x8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int d = c >> 1;
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const unsigned lo = in[2 * e][d], hi = in[2 * e + 1][d];
      o[e] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
    out[c] = o;
  }
}

__device__ __forceinline__ u32x2 pack4_bf16(float a, float b, float c, float d) {
  const bf16x2 lo = __builtin_convertvector((f32x2){a, b}, bf16x2);
  const bf16x2 hi = __builtin_convertvector((f32x2){c, d}, bf16x2);
  return (u32x2){__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
}

// XCD-aware order: workgroup w runs on XCD w mod 8.  Logical tiles come in
// groups of gs that share operand rows (the column tiles of one row tile, or
// the tiles of one dW block); each group goes whole to one XCD, and the groups
// go round robin over the XCDs, so that a group's tiles share an L2 while the
// costly and the cheap groups still spread over all XCDs.  Workgroups past
// the last whole round of 8 groups keep their index.
__device__ __forceinline__ int xcd_remap(int w, int G, int gs) {
  const int span = 8 * gs;
  if (gs < 1 || w >= (G / span) * span) return w;
  const int x = w % 8, i = w / 8;
  const int gi = i / gs, o = i - gi * gs;
  return (gi * 8 + x) * gs + o;
}

// Position of a row tile among the per-type row tiles: largest i with tile_off[i] <= rt.
__device__ __forceinline__ int find_type(const int32_t* tile_off, int q, int rt) {
  int lo = 0, hi = q;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tile_off[mid] <= rt)
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

// kLawWidths: the complete-graph law Q_q on groups of unequal widths (eq 18)
constexpr int kLawComplete = 0, kLawTensor = 1, kLawGraph = 2, kLawWidths = 3;

// Forward schedules (section 5.3): kFused sums both endpoint products of an
// output tile in registers.  The two-stage schedule computes the diagonal maps
// over all rows first (kDiag: D[m, g_j] = X[m, g_j] W_jj for every typed row m,
// row tiles across types, so each W_jj tile is read once for all rows; fp32
// into D), then the type-dependent maps (kStrip: for a type-i row tile and
// output group j != i, X[I_i, g_i] W_ij; each off-diagonal block is read once,
// by the one type that uses it), whose epilogue adds D and rounds once.
//
// kMasked (few rows per type): one tile over all M rows in their own order and
// the whole contraction, the weight column tile read once, block by block; the
// activations of block b reach only the rows that use it (type b, or all rows
// when b is the output group j: eq 17's x_i W_ij + x_j W_jj), the others are
// zeroed in registers.  Every weight block is read once per column tile, as in
// the plain product, and nothing is re-read per type.
constexpr int kFused = 0, kDiag = 1, kStrip = 2, kMasked = 3;

template <Op OP, class C, int LAW = kLawComplete, int SCHED = kFused>
__global__ __launch_bounds__(C::THREADS) void tiled_bf16_kernel(Args a) {
  constexpr bool TENSOR = LAW == kLawTensor, GRAPH = LAW == kLawGraph, WIDTHS = LAW == kLawWidths;
  static_assert(SCHED == kFused || (OP == Op::Fwd && LAW == kLawComplete), "two-stage: complete-law forward");
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, KCH = C::KCH, T = C::THREADS;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * C::STAGE];

  const int e = blockIdx.y;
  const int32_t* ws = a.ws + int64_t(e) * a.ws_stride;
  const uint16_t* Ag = a.A + int64_t(e) * a.strideA;
  const uint16_t* Bg = a.B + int64_t(e) * a.strideB;
  uint16_t* Cg = a.C + int64_t(e) * a.strideC;
  const int32_t* offsets = ws + a.off_offsets;
  const int32_t* rows = ws + a.off_rows;
  const int q = a.q;

  // an index of another (q, M) is never trusted: no row id is read from it
  if (ws[1] != kIndexMagic || ws[2] != q || ws[3] != a.M) return;
  // cyclic schedules are handled by the persistent kernel launched beside this one

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / C::WGN, wn = wid % C::WGN;

  // ---------------- tile decode ----------------
  int out_first;        // fwd/dx: first slot in `rows`;  dw: first output row
  int m_cnt;            // valid output rows in the tile
  int n0, n_cnt;        // output columns [n0, n0 + n_cnt)
  int nseg, seg_len;    // contraction: nseg segments of seg_len each
  int segA0 = 0, segA1 = 0, segB0 = 0, segB1 = 0;
  int tb_b = 0, tb_j = 0;  // recursive law: the tile's (dX: column group, row type; dW: b, j)
  const int32_t* krows = nullptr;  // dw: contraction rows

  int seg_len1 = 0;  // unequal widths: the second forward segment's length
  int split = 0;  // dW: this workgroup's share of the tile's contraction
  if constexpr (OP == Op::Dw && WIDTHS) {
    // tiles: (row tile over all K features) x (column tile over all N columns).
    // dW tiles differ widely in cost (diagonal blocks contract over all rows),
    // so consecutive workgroups, which the hardware deals round robin over the
    // XCDs, take the splits of one tile: each tile's work spreads over all XCDs.
    const int n_tn = a.tn[q];
    const int tix = blockIdx.x / a.splits;
    split = blockIdx.x - tix * a.splits;
    const int rt = tix / n_tn, ct = tix - rt * n_tn;
    const int b = find_type(a.tk, q, rt), j = find_type(a.tn, q, ct);
    out_first = a.gk[b] + (rt - a.tk[b]) * BM;
    m_cnt = min(BM, a.gk[b + 1] - out_first);
    n0 = a.gn[j] + (ct - a.tn[j]) * BN;
    n_cnt = min(BN, a.gn[j + 1] - n0);
    const int k_first = (b == j) ? 0 : offsets[b];
    const int k_last = (b == j) ? offsets[q] : offsets[b + 1];
    krows = rows + k_first;
    nseg = 1;
    seg_len = k_last - k_first;
    segA0 = out_first;
    segB0 = n0;
  } else if constexpr (OP == Op::Dw) {
    const int per_block = a.tm_dw * a.tn_dw;
    // consecutive workgroups take the splits of one tile (see the widths case)
    const int tix = blockIdx.x / a.splits;
    split = blockIdx.x - tix * a.splits;
    const int bid = tix / per_block;
    const int t = tix - bid * per_block;
    int b, j;
    if (bid < q) {
      b = j = bid;                         // diagonal blocks first: longest contraction
    } else {
      const int x = bid - q;
      b = x / (q - 1);
      const int jj = x - b * (q - 1);
      j = jj < b ? jj : jj + 1;
    }
    const int rm = t / a.tn_dw, rn = t - rm * a.tn_dw;
    out_first = b * a.s + rm * BM;
    m_cnt = min(BM, a.s - rm * BM);
    n0 = j * a.r + rn * BN;
    n_cnt = min(BN, a.r - rn * BN);
    const int k_first = (b == j) ? 0 : offsets[b];
    const int k_last = (b == j) ? offsets[q] : offsets[b + 1];
    krows = rows + k_first;
    nseg = 1;
    seg_len = k_last - k_first;
    segA0 = b * a.s + rm * BM;  // X column of output row 0
    segB0 = n0;                 // dY column of output column 0
    if constexpr (TENSOR || GRAPH) {
      tb_b = b;
      tb_j = j;
    }
    if constexpr (GRAPH) {
      if (b != j && !graph_edge(a.adj, b, j)) nseg = 0;  // absent edge: a zero block
    }
  } else {
    const int32_t* tile_off = ws + a.off_tiles + tile_height_slot(BM) * (q + 1);
    const int w = xcd_remap(blockIdx.x, gridDim.x, a.n_ct);
    const int rt = w / a.n_ct;
    const int ct = w - rt * a.n_ct;
    int i;
    if constexpr (SCHED == kMasked) {
      // row tiles over all M rows in order (no index gather)
      out_first = rt * BM;
      if (out_first >= a.M) return;
      m_cnt = min(BM, a.M - out_first);
      i = 0;
    } else if constexpr (SCHED == kDiag) {
      // row tiles over all typed rows (the index lists them type by type)
      out_first = rt * BM;
      if (out_first >= offsets[q]) return;
      m_cnt = min(BM, offsets[q] - out_first);
      i = 0;
    } else {
      if (rt >= tile_off[q]) return;
      i = find_type(tile_off, q, rt);
      out_first = offsets[i] + (rt - tile_off[i]) * BM;
      m_cnt = min(BM, offsets[i + 1] - out_first);
    }
    if constexpr (WIDTHS) {
      if constexpr (OP == Op::Fwd) {
        // output group j of widths r_j; segments X[., g_i] W[g_i, .] (s_i) and X[., g_j] W[g_j, .] (s_j)
        const int j = find_type(a.tn, q, ct);
        n0 = a.gn[j] + (ct - a.tn[j]) * BN;
        n_cnt = min(BN, a.gn[j + 1] - n0);
        nseg = (j == i) ? 1 : 2;
        seg_len = a.gk[i + 1] - a.gk[i];
        seg_len1 = a.gk[j + 1] - a.gk[j];
        segA0 = segB0 = a.gk[i];
        segA1 = segB1 = a.gk[j];
      } else {
        // dX column group k of width s_k; contraction all N (k == i) or output group k (r_k)
        const int k = find_type(a.tk, q, ct);
        n0 = a.gk[k] + (ct - a.tk[k]) * BN;
        n_cnt = min(BN, a.gk[k + 1] - n0);
        nseg = 1;
        seg_len = (k == i) ? a.N : a.gn[k + 1] - a.gn[k];
        segA0 = (k == i) ? 0 : a.gn[k];
      }
    } else {
    const int j = ct / a.ct_per_group, cc = ct - j * a.ct_per_group;
    const int gw = (OP == Op::Fwd) ? a.r : a.s;
    n0 = j * gw + cc * BN;
    n_cnt = min(BN, gw - cc * BN);
    if constexpr (OP == Op::Fwd) {
      seg_len = a.s;
      nseg = (j == i) ? 1 : 2;
      segA0 = segB0 = i * a.s;   // X columns / W rows of group i
      segA1 = segB1 = j * a.s;   // X columns / W rows of group j
      if constexpr (SCHED == kMasked) {
        nseg = q;                // every block b = 0 .. q-1, masked per row
        tb_j = j;
      } else if constexpr (SCHED == kDiag) {
        nseg = 1;                // X[., g_j] W_jj
        segA0 = segB0 = j * a.s;
      } else if constexpr (SCHED == kStrip) {
        nseg = (j == i) ? 0 : 1; // X[I_i, g_i] W_ij (the diagonal term is in D)
      }
      if constexpr (GRAPH) {
        if (j != i && !graph_edge(a.adj, i, j)) nseg = 0;  // absent edge: zero output block
      }
    } else if constexpr (GRAPH) {
      seg_len = a.r;
      tb_b = j;
      tb_j = i;
      if (j == i) {
        // contraction over the output groups {i} and the out-neighbours of i
        nseg = __builtin_popcountll(a.adj[i] | (1ull << i));
      } else {
        nseg = graph_edge(a.adj, i, j) ? 1 : 0;
        segA0 = j * a.r;
      }
    } else if constexpr (TENSOR) {
      // dX column group j of a type-i row: contraction over the output groups
      // agreeing with j where j differs from i, r columns each
      nseg = 1 << (a.L - __builtin_popcount(i ^ j));
      seg_len = a.r;
      tb_b = j;
      tb_j = i;
    } else {
      nseg = 1;
      seg_len = (j == i) ? a.N : a.r;
      segA0 = (j == i) ? 0 : j * a.r;  // dY columns (= W columns) of the contraction
    }
    }
  }
  const int kts = (seg_len + BK - 1) / BK;  // k-steps per segment (the first, for unequal widths)
  const int this_seg_len = seg_len;
  const int this_seg_len1 = WIDTHS ? seg_len1 : seg_len;
  int nk = nseg * kts;
  if constexpr (WIDTHS && OP == Op::Fwd) {
    if (nseg == 2) nk = kts + (seg_len1 + BK - 1) / BK;
  }
  // recursive-law dW: the segment (type) the copy steps are in, its first
  // k-step, row range and k-steps (loads call it with increasing k-steps)
  int w_n = 0, w_k0 = 0, w_lo = 0, w_len = 0, w_kn = 0;
  if constexpr (TENSOR && OP == Op::Dw) {
    // dW block (b, j): the rows of each type agreeing with b where b differs from j
    const int fm_ = tb_b ^ tb_j;
    nseg = 1 << (a.L - __builtin_popcount(fm_));
    nk = 0;
    for (int n = 0; n < nseg; ++n) {
      const int t = law_member(tb_b, fm_, n, a.L);
      nk += (offsets[t + 1] - offsets[t] + BK - 1) / BK;
    }
    const int t0 = law_member(tb_b, fm_, 0, a.L);
    w_lo = offsets[t0];
    w_len = offsets[t0 + 1] - w_lo;
    w_kn = (w_len + BK - 1) / BK;
  }
  // graph-law walkers: the member (type for dW, output group for dX) of the
  // segment the copy steps are in, and the members still to come
  uint64_t g_rest = 0;
  int g_cur = 0;
  if constexpr (GRAPH && OP == Op::Dw) {
    if (tb_b == tb_j) {
      // dW block (j, j): the rows of type j and of its in-neighbours
      const uint64_t mem = graph_in_mask(a.adj, q, tb_j);
      nseg = __builtin_popcountll(mem);
      nk = 0;
      for (uint64_t m = mem; m != 0; m &= m - 1) {
        const int t = __builtin_ctzll(m);
        nk += (offsets[t + 1] - offsets[t] + BK - 1) / BK;
      }
      g_cur = __builtin_ctzll(mem);
      g_rest = mem & (mem - 1);
      w_lo = offsets[g_cur];
      w_len = offsets[g_cur + 1] - w_lo;
      w_kn = (w_len + BK - 1) / BK;
    } else if (nseg > 0) {
      nk = kts;  // the rows of type b: one segment (krows, seg_len above)
    }
  }
  if constexpr (GRAPH && OP == Op::Dx) {
    if (tb_b == tb_j) {
      const uint64_t mem = a.adj[tb_j] | (1ull << tb_j);
      g_cur = __builtin_ctzll(mem);
      g_rest = mem & (mem - 1);
    }
  }

  // ---------------- loaders ----------------
  // A tile: BM output rows x BK contraction; B tile: BN output columns x BK.
  constexpr bool A_KMAJOR = (OP != Op::Dw);
  constexpr bool B_KMAJOR = (OP == Op::Dx);
  constexpr int A_PER = A_KMAJOR ? (C::A_CHUNKS + T - 1) / T : (C::A_BLOCKS + T - 1) / T;
  constexpr int B_PER = B_KMAJOR ? (C::B_CHUNKS + T - 1) / T : (C::B_BLOCKS + T - 1) / T;
  constexpr int A_REGS = A_KMAJOR ? 1 : 8;
  constexpr int B_REGS = B_KMAJOR ? 1 : 8;
  // dW with both operands' 8x8 blocks fitting the workgroup once: the X blocks
  // go to the first threads and the dY blocks to the last, so that each thread
  // gathers 8 rows of one operand, and the row ids are fetched a k-step ahead
  constexpr bool DW_SPLIT = OP == Op::Dw && C::A_BLOCKS + C::B_BLOCKS <= T;
  constexpr int B_BASE = DW_SPLIT ? T - C::B_BLOCKS : 0;  // first thread of the dY blocks

  const uint16_t* a_ptr[A_PER];  // K-major: row base (contraction offset added per step)
  int a_typ[A_PER];              // kMasked: the row's type (-1: padding row or out of range)
  bool a_use[A_PER];             // kMasked: whether the loaded step reaches the row
  int a_kc[A_PER];               // K-major: chunk; MN-major: block's k-chunk
  int a_mn[A_PER];               // K-major: local row; MN-major: local first column (x8)
  bool a_on[A_PER];
  const uint16_t* b_ptr[B_PER];
  int b_kc[B_PER];
  int b_mn[B_PER];
  bool b_on[B_PER];

#pragma unroll
  for (int u = 0; u < A_PER; ++u) {
    const int c = tid + u * T;
    if constexpr (A_KMAJOR) {
      a_on[u] = c < C::A_CHUNKS;
      const int rl = c / KCH, kc = c % KCH;
      a_mn[u] = rl;
      a_kc[u] = kc;
      const int slot = out_first + min(rl, m_cnt - 1);
      const int grow = SCHED == kMasked ? slot : rows[slot];
      if constexpr (SCHED == kMasked) {
        const int t = (rl < m_cnt) ? a.tau[int64_t(e) * a.M + grow] : -1;
        a_typ[u] = (t >= 0 && t < q) ? t : -1;  // an out-of-range row takes no block: a zero output row
      }
      const int64_t ld = (OP == Op::Fwd) ? a.K : a.N;
      a_ptr[u] = Ag + int64_t(grow) * ld;  // + segment column + k offset per step
    } else {
      a_on[u] = c < C::A_BLOCKS;
      const int kb = c % KCH, mb = c / KCH;
      a_kc[u] = kb;
      a_mn[u] = mb * 8;
      a_ptr[u] = Ag + segA0 + mb * 8;  // row offset added per step (gathered)
    }
  }
#pragma unroll
  for (int u = 0; u < B_PER; ++u) {
    const int c = tid + u * T;
    if constexpr (B_KMAJOR) {
      b_on[u] = c < C::B_CHUNKS;
      const int nl = c / KCH, kc = c % KCH;
      b_mn[u] = nl;
      b_kc[u] = kc;
      b_ptr[u] = Bg + int64_t(n0 + min(nl, n_cnt - 1)) * a.N;  // W row = dX column
    } else {
      const int cb = c - B_BASE;
      b_on[u] = cb >= 0 && cb < C::B_BLOCKS;
      const int kb = max(cb, 0) % KCH, nb = max(cb, 0) / KCH;
      b_kc[u] = kb;
      b_mn[u] = nb * 8;
      b_ptr[u] = Bg + n0 + nb * 8;
    }
  }

  u32x4 ra[A_PER][A_REGS];
  u32x4 rb[B_PER][B_REGS];

  // segment of k-step kt: segment index sg (0/1, two-segment forwards), offset
  // k0 inside it, its length, dW's contraction rows and the A column offset.
  // The walks of the recursive and graph laws only move forward: calls come
  // with increasing kt.
  auto seg_at = [&](int kt, int& sg, int& k0, int& seg_len, const int32_t*& krows_s,
                    int& segA0_s) __attribute__((always_inline)) {
    sg = kt >= kts ? 1 : 0;
    k0 = (kt - sg * kts) * BK;
    seg_len = sg ? this_seg_len1 : this_seg_len;
    krows_s = krows;
    segA0_s = segA0;
    if constexpr (SCHED == kMasked) {
      // block n = kt / kts; sg carries n (the segment column is n s)
      sg = kt / kts;
      k0 = (kt - sg * kts) * BK;
      segA0_s = sg * a.s;
    }
    if constexpr (GRAPH) {
      if constexpr (OP == Op::Dx) {
        if (tb_b == tb_j) {  // member groups visited in increasing order as kt grows
          const int n = kt / kts;
          while (w_n < n) {
            g_cur = __builtin_ctzll(g_rest);
            g_rest &= g_rest - 1;
            ++w_n;
          }
          k0 = (kt - n * kts) * BK;
          segA0_s = g_cur * a.r;
          sg = 0;
        }
      } else if constexpr (OP == Op::Dw) {
        if (tb_b == tb_j) {  // diagonal block: the member types' row ranges
          while (kt >= w_k0 + w_kn && g_rest != 0) {
            w_k0 += w_kn;
            g_cur = __builtin_ctzll(g_rest);
            g_rest &= g_rest - 1;
            w_lo = offsets[g_cur];
            w_len = offsets[g_cur + 1] - w_lo;
            w_kn = (w_len + BK - 1) / BK;
          }
          krows_s = rows + w_lo;
          seg_len = w_len;
          k0 = (kt - w_k0) * BK;
        }
      }
    }
    if constexpr (TENSOR) {
      if constexpr (OP == Op::Dx) {
        const int n = kt / kts;
        k0 = (kt - n * kts) * BK;
        segA0_s = law_member(tb_b, tb_b ^ tb_j, n, a.L) * a.r;
        sg = 0;
      } else {  // Dw: the types' row ranges, walked forward as kt grows
        while (kt >= w_k0 + w_kn && w_n + 1 < nseg) {
          w_k0 += w_kn;
          ++w_n;
          const int t = law_member(tb_b, tb_b ^ tb_j, w_n, a.L);
          w_lo = offsets[t];
          w_len = offsets[t + 1] - w_lo;
          w_kn = (w_len + BK - 1) / BK;
        }
        krows_s = rows + w_lo;
        seg_len = w_len;
        k0 = (kt - w_k0) * BK;
      }
    }
  };

  auto load_step = [&](int kt) __attribute__((always_inline)) {
    int sg, k0, seg_len, segA0_s;
    const int32_t* krows_s;
    seg_at(kt, sg, k0, seg_len, krows_s, segA0_s);
#pragma unroll
    for (int u = 0; u < A_PER; ++u) {
      if constexpr (A_KMAJOR) {
        const int kk = k0 + a_kc[u] * 8;
        const int col = SCHED == kMasked ? segA0_s + kk : (sg ? segA1 : segA0_s) + kk;
        if (a_on[u] && kk < seg_len)
          ra[u][0] = *reinterpret_cast<const u32x4*>(a_ptr[u] + col);
        else
          ra[u][0] = (u32x4){0u, 0u, 0u, 0u};
        if constexpr (SCHED == kMasked) {
          // block sg reaches rows of type sg, and every row when sg is the output
          // group; the others are zeroed when the step is stored to LDS (using
          // the loaded value here would wait for the load at once)
          a_use[u] = a_typ[u] >= 0 && (a_typ[u] == sg || sg == tb_j);
        }
      } else {  // dW: 8 gathered contraction rows x 8 output rows
        const int kk = k0 + a_kc[u] * 8;
        const bool on = a_on[u] && a_mn[u] < m_cnt;
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          if (on && kk + rr < seg_len) {
            const int grow = krows_s[kk + rr];
            ra[u][rr] = *reinterpret_cast<const u32x4*>(a_ptr[u] + int64_t(grow) * a.K);
          } else {
            ra[u][rr] = (u32x4){0u, 0u, 0u, 0u};
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < B_PER; ++u) {
      if constexpr (B_KMAJOR) {  // dX: W row (output column), contraction along W's columns
        const int kk = k0 + b_kc[u] * 8;
        if (b_on[u] && kk < seg_len)
          rb[u][0] = *reinterpret_cast<const u32x4*>(b_ptr[u] + segA0_s + kk);
        else
          rb[u][0] = (u32x4){0u, 0u, 0u, 0u};
      } else if constexpr (OP == Op::Fwd) {  // W rows of the segment, 8 output columns
        const int kk = k0 + b_kc[u] * 8;
        const int wrow = SCHED == kMasked ? sg * a.s + kk : (sg ? segB1 : segB0) + kk;
        const bool on = b_on[u] && b_mn[u] < n_cnt;
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          if (on && kk + rr < seg_len)
            rb[u][rr] = *reinterpret_cast<const u32x4*>(b_ptr[u] + int64_t(wrow + rr) * a.N);
          else
            rb[u][rr] = (u32x4){0u, 0u, 0u, 0u};
        }
      } else {  // dW: dY rows gathered, 8 output columns
        const int kk = k0 + b_kc[u] * 8;
        const bool on = b_on[u] && b_mn[u] < n_cnt;
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          if (on && kk + rr < seg_len) {
            const int grow = krows_s[kk + rr];
            rb[u][rr] = *reinterpret_cast<const u32x4*>(b_ptr[u] + int64_t(grow) * a.N);
          } else {
            rb[u][rr] = (u32x4){0u, 0u, 0u, 0u};
          }
        }
      }
    }
  };

  // DW_SPLIT: this thread's block (X features or dY columns: 8 of them, at
  // contraction chunk dw_kc), computed from scalars so that no selection
  // between the per-operand arrays is needed, and the row ids of the block's
  // 8 contraction rows for the next gathered load (-1: padding)
  const bool dw_isA = tid < C::A_BLOCKS;
  const int dw_c = dw_isA ? tid : max(tid - B_BASE, 0);
  const int dw_kc = dw_c % KCH, dw_mn = (dw_c / KCH) * 8;
  const bool dw_on = dw_isA ? dw_mn < m_cnt : (tid >= B_BASE && dw_mn < n_cnt);
  const uint16_t* dw_ptr = dw_isA ? Ag + segA0 + dw_mn : Bg + n0 + dw_mn;
  const int64_t dw_ld = dw_isA ? a.K : a.N;
  int nid[8];
  auto fetch_ids = [&](int kt) __attribute__((always_inline)) {
    int sg, k0, seg_len, segA0_s;
    const int32_t* krows_s;
    seg_at(kt, sg, k0, seg_len, krows_s, segA0_s);
    const int kk = k0 + dw_kc * 8;
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) nid[rr] = (dw_on && kk + rr < seg_len) ? krows_s[kk + rr] : -1;
  };
  auto load_ids = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      u32x4 v = (u32x4){0u, 0u, 0u, 0u};
      if (nid[rr] >= 0) v = *reinterpret_cast<const u32x4*>(dw_ptr + int64_t(nid[rr]) * dw_ld);
      ra[0][rr] = v;  // store_step takes ra on the X threads, rb on the dY threads
      rb[0][rr] = v;
    }
  };

  auto store_step = [&](int stage) {
    uint16_t* As = smem + stage * C::STAGE;
    uint16_t* Bs = As + BM * BK;
#pragma unroll
    for (int u = 0; u < A_PER; ++u) {
      if (!a_on[u]) continue;
      if constexpr (A_KMAJOR) {
        const int rl = a_mn[u];
        u32x4 v = ra[u][0];
        if constexpr (SCHED == kMasked) v = a_use[u] ? v : (u32x4){0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(As + rl * BK + swz(rl, a_kc[u], KCH) * 8) = v;
      } else {
        u32x4 t8[8];
        transpose8x8(ra[u], t8);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int rl = a_mn[u] + c;
          *reinterpret_cast<u32x4*>(As + rl * BK + swz(rl, a_kc[u], KCH) * 8) = t8[c];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < B_PER; ++u) {
      if (!b_on[u]) continue;
      if constexpr (B_KMAJOR) {
        const int nl = b_mn[u];
        *reinterpret_cast<u32x4*>(Bs + nl * BK + swz(nl, b_kc[u], KCH) * 8) = rb[u][0];
      } else {
        u32x4 t8[8];
        transpose8x8(rb[u], t8);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int nl = b_mn[u] + c;
          *reinterpret_cast<u32x4*>(Bs + nl * BK + swz(nl, b_kc[u], KCH) * 8) = t8[c];
        }
      }
    }
  };

  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) acc[fm][fn] = (f32x16){};

  const int l32 = lane & 31, lhi = lane >> 5;
  auto compute_step = [&](int stage) {
    const uint16_t* As = smem + stage * C::STAGE;
    const uint16_t* Bs = As + BM * BK;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int ch = ks * 2 + lhi;
      bf16x8 af[C::FM], bfr[C::FN];
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm) {
        const int rl = wm * C::WTM + fm * 32 + l32;
        af[fm] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(As + rl * BK + swz(rl, ch, KCH) * 8));
      }
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) {
        const int nl = wn * C::WTN + fn * 32 + l32;
        bfr[fn] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(Bs + nl * BK + swz(nl, ch, KCH) * 8));
      }
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[fn], af[fm], acc[fm][fn], 0, 0, 0);
    }
  };

  // ---------------- main loop ----------------
  // (dW with a split contraction: this workgroup's contiguous range of k-steps)
  int k_lo = 0, k_hi = nk;
  if constexpr (OP == Op::Dw) {
    const int chunk = (nk + a.splits - 1) / a.splits;
    k_lo = min(nk, split * chunk);
    k_hi = min(nk, k_lo + chunk);
  }
  if constexpr (DW_SPLIT) {
    if (k_hi > k_lo) {
      fetch_ids(k_lo);
      load_ids();
      if (k_lo + 1 < k_hi) fetch_ids(k_lo + 1);
      store_step(0);
      __syncthreads();
      for (int kt = k_lo; kt < k_hi; ++kt) {
        const bool more = kt + 1 < k_hi;
        if (more) {
          load_ids();                            // k-step kt + 1 (ids fetched a step ago)
          if (kt + 2 < k_hi) fetch_ids(kt + 2);  // in flight during this k-step's MFMAs
        }
        compute_step((kt - k_lo) & 1);
        if (more) store_step((kt - k_lo + 1) & 1);
        __syncthreads();
      }
    }
  } else if (k_hi > k_lo) {
    load_step(k_lo);
    store_step(0);
    __syncthreads();
    for (int kt = k_lo; kt < k_hi; ++kt) {
      const bool more = kt + 1 < k_hi;
      if (more) load_step(kt + 1);
      compute_step((kt - k_lo) & 1);
      if (more) store_step((kt - k_lo + 1) & 1);
      __syncthreads();
    }
  }

  // ---------------- epilogue: one RNE rounding per output ----------------
  const int64_t ldc = (OP == Op::Fwd) ? a.N : (OP == Op::Dx ? a.K : a.N);
  if constexpr (OP == Op::Dw) {
    if (a.splits > 1) {
      // fp32 partial tile; the reduction sums the splits in order and rounds once
      float* prow0 = a.part + int64_t(split) * a.K * a.N;
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm) {
        const int ml = wm * C::WTM + fm * 32 + l32;
        if (ml >= m_cnt) continue;
        float* prow = prow0 + int64_t(out_first + ml) * a.N + n0;
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int nl = wn * C::WTN + fn * 32 + g * 8 + lhi * 4;
            if (nl < n_cnt) {
              const f32x16& v = acc[fm][fn];
              *reinterpret_cast<float4*>(prow + nl) = make_float4(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]);
            }
          }
      }
      return;
    }
  }
  if constexpr (SCHED == kDiag) {
    // fp32 diagonal maps into D (rows at their own positions)
    float* Dg = a.D + int64_t(e) * a.strideD;
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
      const int ml = wm * C::WTM + fm * 32 + l32;
      if (ml >= m_cnt) continue;
      float* drow = Dg + int64_t(rows[out_first + ml]) * a.N + n0;
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int nl = wn * C::WTN + fn * 32 + g * 8 + lhi * 4;
          if (nl < n_cnt) {
            const f32x16& v = acc[fm][fn];
            *reinterpret_cast<float4*>(drow + nl) = make_float4(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]);
          }
        }
    }
    return;
  }
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
    const int ml = wm * C::WTM + fm * 32 + l32;
    if (ml >= m_cnt) continue;
    int64_t grow;
    if constexpr (OP == Op::Dw || SCHED == kMasked)
      grow = out_first + ml;
    else
      grow = rows[out_first + ml];
    uint16_t* crow = Cg + grow * ldc + n0;
    if constexpr (SCHED == kStrip) {
      // add the row's diagonal map from D: the output is the sum of both
      // endpoint products, rounded once below
      const float* drow = a.D + int64_t(e) * a.strideD + grow * a.N + n0;
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int nl = wn * C::WTN + fn * 32 + g * 8 + lhi * 4;
          if (nl < n_cnt) {
            const float4 d = *reinterpret_cast<const float4*>(drow + nl);
            acc[fm][fn][4 * g] += d.x;
            acc[fm][fn][4 * g + 1] += d.y;
            acc[fm][fn][4 * g + 2] += d.z;
            acc[fm][fn][4 * g + 3] += d.w;
          }
        }
    }
    // lane (l32, lhi) holds columns g*8 + lhi*4 .. +3 of each 32-column block;
    // v_permlane32_swap on the packed pieces of groups 2gp and 2gp + 1 (lanes
    // 32-63 of the first exchanged with lanes 0-31 of the second; both lanes of
    // a pair hold the same row) leaves half 0 with columns 16gp + 0..7 and half
    // 1 with 16gp + 8..15: one 16-byte store per lane (column counts are whole
    // 8-column pieces)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        const f32x16& v = acc[fm][fn];
        const u32x2 x = pack4_bf16(v[8 * gp], v[8 * gp + 1], v[8 * gp + 2], v[8 * gp + 3]);
        const u32x2 y = pack4_bf16(v[8 * gp + 4], v[8 * gp + 5], v[8 * gp + 6], v[8 * gp + 7]);
        const auto s0 = __builtin_amdgcn_permlane32_swap(x[0], y[0], false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(x[1], y[1], false, false);
        const int nl = wn * C::WTN + fn * 32 + gp * 16 + lhi * 8;
        if (nl < n_cnt) *reinterpret_cast<u32x4*>(crow + nl) = (u32x4){s0[0], s1[0], s0[1], s1[1]};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 path: the same tiles and segments, scalar FMA, 64x64 tiles.
// ---------------------------------------------------------------------------
constexpr int F_BM = 64, F_BN = 64, F_BK = 16, F_T = 256;

template <Op OP>
__global__ __launch_bounds__(F_T) void tiled_f32_kernel(Args a, const float* A32, const float* B32, float* C32) {
  __shared__ float As[F_BK][F_BM + 4];
  __shared__ float Bs[F_BK][F_BN + 4];
  const int e = blockIdx.y;
  const int32_t* ws = a.ws + int64_t(e) * a.ws_stride;
  const float* Ag = A32 + int64_t(e) * a.strideA;
  const float* Bg = B32 + int64_t(e) * a.strideB;
  float* Cg = C32 + int64_t(e) * a.strideC;
  const int32_t* offsets = ws + a.off_offsets;
  const int32_t* rows = ws + a.off_rows;
  const int q = a.q;
  const int tid = threadIdx.x;
  if (ws[1] != kIndexMagic || ws[2] != q || ws[3] != a.M) return;

  int out_first, m_cnt, n0, n_cnt, nseg, seg_len;
  int segA0 = 0, segA1 = 0, segB0 = 0, segB1 = 0;
  const int32_t* krows = nullptr;
  if constexpr (OP == Op::Dw) {
    const int per_block = a.tm_dw * a.tn_dw;
    const int bid = blockIdx.x / per_block;
    const int t = blockIdx.x - bid * per_block;
    int b, j;
    if (bid < q) {
      b = j = bid;
    } else {
      const int x = bid - q;
      b = x / (q - 1);
      const int jj = x - b * (q - 1);
      j = jj < b ? jj : jj + 1;
    }
    const int rm = t / a.tn_dw, rn = t - rm * a.tn_dw;
    out_first = b * a.s + rm * F_BM;
    m_cnt = min(F_BM, a.s - rm * F_BM);
    n0 = j * a.r + rn * F_BN;
    n_cnt = min(F_BN, a.r - rn * F_BN);
    const int k_first = (b == j) ? 0 : offsets[b];
    const int k_last = (b == j) ? offsets[q] : offsets[b + 1];
    krows = rows + k_first;
    nseg = 1;
    seg_len = k_last - k_first;
  } else {
    const int32_t* tile_off = ws + a.off_tiles + tile_height_slot(F_BM) * (q + 1);
    const int rt = blockIdx.x / a.n_ct;
    const int ct = blockIdx.x - rt * a.n_ct;
    if (rt >= tile_off[q]) return;
    const int i = find_type(tile_off, q, rt);
    out_first = offsets[i] + (rt - tile_off[i]) * F_BM;
    m_cnt = min(F_BM, offsets[i + 1] - out_first);
    const int j = ct / a.ct_per_group, cc = ct - j * a.ct_per_group;
    const int gw = (OP == Op::Fwd) ? a.r : a.s;
    n0 = j * gw + cc * F_BN;
    n_cnt = min(F_BN, gw - cc * F_BN);
    if constexpr (OP == Op::Fwd) {
      seg_len = a.s;
      nseg = (j == i) ? 1 : 2;
      segA0 = segB0 = i * a.s;
      segA1 = segB1 = j * a.s;
    } else {
      nseg = 1;
      seg_len = (j == i) ? a.N : a.r;
      segA0 = (j == i) ? 0 : j * a.r;
    }
  }

  const int tx = tid % 16, ty = tid / 16;  // thread owns rows ty*4.., columns tx*4..
  float acc[4][4] = {};
  for (int sg = 0; sg < nseg; ++sg) {
    for (int k0 = 0; k0 < seg_len; k0 += F_BK) {
      // A tile element (m, k): 64 x 16 = 1024 values, 4 per thread
      for (int x = tid; x < F_BM * F_BK; x += F_T) {
        int ml, kk;
        if constexpr (OP == Op::Dw) { ml = x % F_BM; kk = x / F_BM; } else { kk = x % F_BK; ml = x / F_BK; }
        const int k = k0 + kk;
        float v = 0.f;
        if (ml < m_cnt && k < seg_len) {
          if constexpr (OP == Op::Fwd) v = Ag[int64_t(rows[out_first + ml]) * a.K + (sg ? segA1 : segA0) + k];
          else if constexpr (OP == Op::Dx) v = Ag[int64_t(rows[out_first + ml]) * a.N + segA0 + k];
          else v = Ag[int64_t(krows[k]) * a.K + out_first + ml];
        }
        As[kk][ml] = v;
      }
      for (int x = tid; x < F_BN * F_BK; x += F_T) {
        int nl, kk;
        if constexpr (OP == Op::Dx) { kk = x % F_BK; nl = x / F_BK; } else { nl = x % F_BN; kk = x / F_BN; }
        const int k = k0 + kk;
        float v = 0.f;
        if (nl < n_cnt && k < seg_len) {
          if constexpr (OP == Op::Fwd) v = Bg[int64_t((sg ? segB1 : segB0) + k) * a.N + n0 + nl];
          else if constexpr (OP == Op::Dx) v = Bg[int64_t(n0 + nl) * a.N + segA0 + k];
          else v = Bg[int64_t(krows[k]) * a.N + n0 + nl];
        }
        Bs[kk][nl] = v;
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < F_BK; ++kk) {
        float av[4], bv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) { av[u] = As[kk][ty * 4 + u]; bv[u] = Bs[kk][tx * 4 + u]; }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[u][v] = fmaf(av[u], bv[v], acc[u][v]);
      }
      __syncthreads();
    }
  }
  const int64_t ldc = (OP == Op::Dx) ? a.K : a.N;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int ml = ty * 4 + u;
    if (ml >= m_cnt) continue;
    const int64_t grow = (OP == Op::Dw) ? int64_t(out_first + ml) : int64_t(rows[out_first + ml]);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int nl = tx * 4 + v;
      if (nl < n_cnt) Cg[grow * ldc + n0 + nl] = acc[u][v];
    }
  }
}

inline int cdiv(int64_t a, int64_t b) { return int((a + b - 1) / b); }

// dW = bf16(sum over splits of the fp32 partial tiles), in split order: one
// rounding per element, the same bits on every run.  4 elements per thread.
// It checks the index like the tile kernel that wrote the partials: when that
// kernel returned at once (an index of another q or M), dW is left untouched
// instead of being overwritten from stale partials.
__global__ __launch_bounds__(256) void dw_reduce_kernel(const float* __restrict__ part, int splits, int64_t n,
                                                        uint16_t* __restrict__ out, const int32_t* __restrict__ ws,
                                                        int q, int M) {
  if (ws[1] != kIndexMagic || ws[2] != q || ws[3] != M) return;
  const int64_t i = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  float4 acc = *reinterpret_cast<const float4*>(part + i);
  for (int p = 1; p < splits; ++p) {
    const float4 v = *reinterpret_cast<const float4*>(part + int64_t(p) * n + i);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  *reinterpret_cast<u32x2*>(out + i) = pack4_bf16(acc.x, acc.y, acc.z, acc.w);
}

hipError_t launch_dw_reduce(const Args& a, int64_t n, uint16_t* out, hipStream_t s) {
  const int64_t threads = n / 4;
  hipLaunchKernelGGL(dw_reduce_kernel, dim3(unsigned((threads + 255) / 256)), dim3(256), 0, s, a.part, a.splits, n,
                     out, a.ws, a.q, a.M);
  return hipGetLastError();
}

Args make_args(const ProblemDesc& p, int bm, int bn) {
  Args a{};
  a.splits = 1;
  a.A = static_cast<const uint16_t*>(p.A);
  a.B = static_cast<const uint16_t*>(p.B);
  a.C = static_cast<uint16_t*>(p.C);
  a.ws = p.ws;
  a.ws_stride = p.ws_stride;
  a.q = p.q;
  a.M = int(p.M);
  a.K = int(p.K);
  a.N = int(p.N);
  a.s = int(p.K / p.q);
  a.r = int(p.N / p.q);
  const WsLayout L = ws_layout(p.q, p.M);
  a.off_offsets = L.offsets;
  a.off_tiles = L.tile_off;
  a.off_rows = L.rows;
  if (p.op == Op::Fwd) {
    a.strideA = p.M * p.K; a.strideB = p.K * p.N; a.strideC = p.M * p.N;
    a.ct_per_group = cdiv(a.r, bn);
  } else if (p.op == Op::Dx) {
    a.strideA = p.M * p.N; a.strideB = p.K * p.N; a.strideC = p.M * p.K;
    a.ct_per_group = cdiv(a.s, bn);
  } else {
    a.strideA = p.M * p.K; a.strideB = p.M * p.N; a.strideC = p.K * p.N;
    a.ct_per_group = 0;
    a.tm_dw = cdiv(a.s, bm);
    a.tn_dw = cdiv(a.r, bn);
  }
  a.n_ct = p.q * a.ct_per_group;
  if (p.in_widths != nullptr) {
    // group starts, and per-group tile counts along the tiled output axes
    const int tile_k = p.op == Op::Dw ? bm : bn;  // dW rows / dX columns run along K
    a.gk[0] = a.gn[0] = a.tk[0] = a.tn[0] = 0;
    for (int g = 0; g < p.q; ++g) {
      a.gk[g + 1] = a.gk[g] + int(p.in_widths[g]);
      a.gn[g + 1] = a.gn[g] + int(p.out_widths[g]);
      a.tk[g + 1] = a.tk[g] + cdiv(p.in_widths[g], tile_k);
      a.tn[g + 1] = a.tn[g] + cdiv(p.out_widths[g], bn);
    }
    a.n_ct = p.op == Op::Fwd ? a.tn[p.q] : a.tk[p.q];
  }
  return a;
}

// dW tiles of a launch
int64_t dw_tiles(const ProblemDesc& p, const Args& a) {
  return p.in_widths != nullptr ? int64_t(a.tk[p.q]) * a.tn[p.q] : int64_t(p.q) * p.q * a.tm_dw * a.tn_dw;
}

dim3 grid_for(const ProblemDesc& p, const Args& a, int bm, int sched = kFused) {
  if (p.op == Op::Dw) return dim3(unsigned(dw_tiles(p, a) * (a.splits > 1 ? a.splits : 1)), unsigned(p.E));
  // row tiles over all rows (masked and diagonal schedules): exactly ceil(M / BM);
  // tiles of one type each: at most sum_i ceil(M_i / BM) <= ceil(M / BM) + q - 1.
  // (Sizing the former like the latter would leave most workgroups idle, and
  // the XCD remap would put all the busy ones on one XCD.)
  const int64_t rt = (p.M + bm - 1) / bm + (sched == kMasked || sched == kDiag ? 0 : p.q - 1);
  return dim3(unsigned(rt * a.n_ct), unsigned(p.E));
}

template <Op OP, class C, int SCHED = kFused>
hipError_t launch_cfg(const ProblemDesc& p, hipStream_t s) {
  Args a = make_args(p, C::BM, C::BN);
  a.L = p.law_L;
  // (not beside the persistent kernel: there this launch may return at once)
  if (OP == Op::Dw && p.dw_part != nullptr && p.E == 1) {
    // enough workgroups to cover the CUs about four times, at most kDwMaxSplits per tile
    const int64_t tiles = dw_tiles(p, a);
    int64_t sp = (4 * 256 + tiles - 1) / tiles;
    sp = sp < 1 ? 1 : (sp > kDwMaxSplits ? kDwMaxSplits : sp);
    a.splits = int(sp);
    a.part = static_cast<float*>(p.dw_part);
  }
  a.adj = p.graph_adj;
  const dim3 g = grid_for(p, a, C::BM, SCHED);
  if (g.x == 0) return hipSuccess;
  if constexpr (SCHED != kFused) {
    a.D = static_cast<float*>(p.fwd_diag);
    a.strideD = p.M * p.N;
    a.tau = p.tau;
    hipLaunchKernelGGL((tiled_bf16_kernel<Op::Fwd, C, kLawComplete, SCHED>), g, dim3(C::THREADS), 0, s, a);
    return hipGetLastError();
  }
  if constexpr (OP != Op::Fwd) {
    if (p.law_L > 0) {
      hipLaunchKernelGGL((tiled_bf16_kernel<OP, C, kLawTensor>), g, dim3(C::THREADS), 0, s, a);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess || a.splits == 1) return e;
      return launch_dw_reduce(a, p.K * p.N, static_cast<uint16_t*>(p.C), s);
    }
  }
  if (p.in_widths != nullptr) {
    hipLaunchKernelGGL((tiled_bf16_kernel<OP, C, kLawWidths>), g, dim3(C::THREADS), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1) return e;
    return launch_dw_reduce(a, p.K * p.N, static_cast<uint16_t*>(p.C), s);
  }
  if (p.graph_adj != nullptr) {
    hipLaunchKernelGGL((tiled_bf16_kernel<OP, C, kLawGraph>), g, dim3(C::THREADS), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1) return e;
    return launch_dw_reduce(a, p.K * p.N, static_cast<uint16_t*>(p.C), s);
  }
  hipLaunchKernelGGL((tiled_bf16_kernel<OP, C>), g, dim3(C::THREADS), 0, s, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  return launch_dw_reduce(a, p.K * p.N, static_cast<uint16_t*>(p.C), s);
}

using Cfg128 = TileCfg<128, 128, 64, 2, 2>;
using Cfg64 = TileCfg<64, 64, 64, 2, 2>;
using Cfg32 = TileCfg<32, 64, 64, 1, 2>;
// few rows per type, wider column tiles: each weight row is read as 256 or 512
// contiguous bytes instead of 128, and a launch has 2-4x fewer tiles, each
// re-reading the diagonal block W_jj (measured on 64 experts, 7168 -> 2048,
// q = 4: M = 64 0.59 -> 0.48 ms, M = 256 0.99 -> 0.74 ms)
using CfgN32 = TileCfg<32, 256, 64, 1, 4>;
using CfgN64 = TileCfg<64, 256, 64, 1, 4>;
using CfgM32 = TileCfg<32, 128, 64, 1, 2>;
using CfgM64 = TileCfg<64, 128, 64, 2, 2>;
// dW on wide groups: 256- or 192-feature tiles with 32-deep k-steps (twice the
// MFMA work per loaded byte of the 128 x 128 tile, whose loads saturate the
// vector-memory path)
using CfgW256 = TileCfg<256, 256, 32, 2, 4>;
using CfgW192 = TileCfg<192, 256, 32, 2, 4>;
using CfgW192n = TileCfg<192, 192, 32, 2, 2>;

// whether every group along the output columns of Y (out widths) or dX (in widths) is a whole
// number of bn-wide tiles
bool cols_exact(const ProblemDesc& p, int bn) {
  for (int g = 0; g < p.q; ++g) {
    const int64_t w = p.op == Op::Fwd ? (p.out_widths ? p.out_widths[g] : p.N / p.q)
                                      : (p.in_widths ? p.in_widths[g] : p.K / p.q);
    if (w % bn) return false;
  }
  return true;
}

// whether every feature group (rows of dW) and output group (its columns) is a whole number of bm x bn tiles
bool dw_tiles_exact(const ProblemDesc& p, int bm, int bn) {
  for (int g = 0; g < p.q; ++g) {
    const int64_t s = p.in_widths ? p.in_widths[g] : p.K / p.q;
    const int64_t r = p.out_widths ? p.out_widths[g] : p.N / p.q;
    if (s % bm || r % bn) return false;
  }
  return true;
}

// Column-tile width of the forward's few-rows tiles (64, 128 or 256) for output
// groups of width r: the share of each tile's columns inside the group, times
// the relative streaming efficiency of the width (1, 0.9, 0.75: wider weight
// rows stream better), largest wins, ties to the wider tile
int fwd_small_bn(int64_t r) {
  int best = 64;
  double best_v = -1.0;
  for (int bn : {256, 128, 64}) {
    const double fill = double(r) / double(((r + bn - 1) / bn) * bn);
    const double v = fill * (bn == 256 ? 1.0 : bn == 128 ? 0.9 : 0.75);
    if (v > best_v + 1e-9) best = bn, best_v = v;
  }
  return best;
}

}  // namespace

hipError_t launch_tiled_bf16(const ProblemDesc& p, hipStream_t s) {
  // Row-tile height from the rows per type (tiles never straddle types).
  const int64_t per_type = p.op == Op::Dw ? p.K / p.q : (p.M + p.q - 1) / p.q;
  switch (p.op) {
    case Op::Fwd:
      // wide tiles where every type has rows for several and the output groups divide evenly
      if (per_type >= 512 && cols_exact(p, 256)) return launch_cfg<Op::Fwd, CfgW256>(p, s);
      if (per_type >= 128) return launch_cfg<Op::Fwd, Cfg128>(p, s);
      if (p.in_widths == nullptr) {
        const int bn = fwd_small_bn(p.N / p.q);
        if (bn == 256)
          return per_type >= 48 ? launch_cfg<Op::Fwd, CfgN64>(p, s)
                                : launch_cfg<Op::Fwd, CfgN32>(p, s);
        if (bn == 128)
          return per_type >= 48 ? launch_cfg<Op::Fwd, CfgM64>(p, s)
                                : launch_cfg<Op::Fwd, CfgM32>(p, s);
      }
      if (per_type >= 48) return launch_cfg<Op::Fwd, Cfg64>(p, s);
      return launch_cfg<Op::Fwd, Cfg32>(p, s);
    case Op::Dx:
      // (not for graph laws: their dX tiles range from no work to q segments, and the
      // smaller tiles balance that better)
      if (per_type >= 512 && cols_exact(p, 256) && p.graph_adj == nullptr)
        return launch_cfg<Op::Dx, CfgW256>(p, s);
      if (per_type >= 128) return launch_cfg<Op::Dx, Cfg128>(p, s);
      if (per_type >= 48) return launch_cfg<Op::Dx, Cfg64>(p, s);
      return launch_cfg<Op::Dx, Cfg32>(p, s);
    case Op::Dw:
      if (dw_tiles_exact(p, 256, 256)) return launch_cfg<Op::Dw, CfgW256>(p, s);
      if (dw_tiles_exact(p, 192, 256)) return launch_cfg<Op::Dw, CfgW192>(p, s);
      if (dw_tiles_exact(p, 192, 192)) return launch_cfg<Op::Dw, CfgW192n>(p, s);
      if (per_type >= 128) return launch_cfg<Op::Dw, Cfg128>(p, s);
      return launch_cfg<Op::Dw, Cfg64>(p, s);
  }
  return hipErrorInvalidValue;
}

// The two-stage forward (section 5.3's second schedule): the diagonal maps
// over all typed rows into p.fwd_diag (fp32, M x N per problem), then the
// type-dependent maps with the diagonal added in the epilogue.  Row tiles of
// the first stage span all rows (its height from M), the second stage's from
// the rows per type, each as in the fused forward.
hipError_t launch_tiled_two_stage_bf16(const ProblemDesc& p, hipStream_t s) {
  const int64_t per_type = (p.M + p.q - 1) / p.q;
  const int bn = fwd_small_bn(p.N / p.q);
  auto pick = [&](int64_t rows, auto sched) -> hipError_t {
    constexpr int SC = decltype(sched)::value;
    if (rows >= 128) return launch_cfg<Op::Fwd, Cfg128, SC>(p, s);
    if (bn == 256) return rows >= 48 ? launch_cfg<Op::Fwd, CfgN64, SC>(p, s)
                                     : launch_cfg<Op::Fwd, CfgN32, SC>(p, s);
    if (bn == 128) return rows >= 48 ? launch_cfg<Op::Fwd, CfgM64, SC>(p, s)
                                     : launch_cfg<Op::Fwd, CfgM32, SC>(p, s);
    return rows >= 48 ? launch_cfg<Op::Fwd, Cfg64, SC>(p, s) : launch_cfg<Op::Fwd, Cfg32, SC>(p, s);
  };
  const hipError_t e = pick(p.M, std::integral_constant<int, kDiag>{});
  if (e != hipSuccess) return e;
  return pick(per_type, std::integral_constant<int, kStrip>{});
}

// The masked forward for few rows per type (kMasked): one tile per (row tile
// of all rows, column tile), the whole contraction, blocks masked per row.
hipError_t launch_tiled_masked_bf16(const ProblemDesc& p, hipStream_t s) {
  const int bn = fwd_small_bn(p.N / p.q);
  const int64_t rows = p.M;
  constexpr int SC = kMasked;
  if (rows >= 128) return launch_cfg<Op::Fwd, Cfg128, SC>(p, s);
  if (bn == 256) return rows >= 48 ? launch_cfg<Op::Fwd, CfgN64, SC>(p, s)
                                   : launch_cfg<Op::Fwd, CfgN32, SC>(p, s);
  if (bn == 128) return rows >= 48 ? launch_cfg<Op::Fwd, CfgM64, SC>(p, s)
                                   : launch_cfg<Op::Fwd, CfgM32, SC>(p, s);
  return rows >= 48 ? launch_cfg<Op::Fwd, Cfg64, SC>(p, s) : launch_cfg<Op::Fwd, Cfg32, SC>(p, s);
}

hipError_t launch_tiled_f32(const ProblemDesc& p, hipStream_t s) {
  const Args a = make_args(p, F_BM, F_BN);
  const dim3 g = grid_for(p, a, F_BM);
  if (g.x == 0) return hipSuccess;
  const float* A = static_cast<const float*>(p.A);
  const float* B = static_cast<const float*>(p.B);
  float* Cp = static_cast<float*>(p.C);
  switch (p.op) {
    case Op::Fwd: hipLaunchKernelGGL((tiled_f32_kernel<Op::Fwd>), g, dim3(F_T), 0, s, a, A, B, Cp); break;
    case Op::Dx: hipLaunchKernelGGL((tiled_f32_kernel<Op::Dx>), g, dim3(F_T), 0, s, a, A, B, Cp); break;
    case Op::Dw: hipLaunchKernelGGL((tiled_f32_kernel<Op::Dw>), g, dim3(F_T), 0, s, a, A, B, Cp); break;
  }
  return hipGetLastError();
}

}  // namespace qalg
