// Persistent matrix-core forward of the row-typed Q_q projection (bf16 in,
// fp32 accumulate, bf16 out) for gfx950.
//
// Paper: arXiv 2609.32814.  Section 4, eq 16-17: a token row of type i gets
// y_i = x_i W_ii and y_j = x_i W_ij + x_j W_jj (j != i).  Section 6.1, eq 27
// and Algorithm 1: the support of output group j for type i is B(i, j) =
// {i, j}.  Section 5.3: in the fused forward the two endpoint products of an
// output are summed in registers and the output is stored once.
//
// Work decomposition.  The rows of each type (from the type index) are cut
// into row tiles of BM rows that never straddle types; the N columns into
// column tiles of BN columns that never straddle output groups.  Output tile
// (row tile of type i, column tile in group j) is one GEMM tile whose
// contraction runs over two K segments, X[rows, g_i] W[g_i, cols] and
// X[rows, g_j] W[g_j, cols], or over the single segment g_i when j == i.  The
// other q-2 weight blocks of that column tile never enter the tile: absent
// block products are skipped at tile granularity.
//
// Schedule.  One workgroup per compute unit loops over its tiles (persistent).
// The k-steps of all its tiles form one stream: operand loads for the next
// k-step, and across a tile boundary for the next tile's first k-step, are in
// flight while the current k-step runs on the matrix cores, so a tile costs
// no pipeline fill.  Long tiles (two contraction segments) and short ones
// (one) are ordered separately in groups of up to 4 row tiles by the class's
// column tiles (neighbouring tiles share operand rows or weight columns); each
// order is cut into one contiguous share per XCD (workgroup w runs on XCD
// w mod 8 when the grid is one workgroup per CU), and the workgroups of an XCD
// are dealt the longs round robin, then the shorts, balanced in k-steps, so
// concurrently running tiles of one XCD share their operands in its L2.
//
// Data movement.  Operands go from global memory straight into LDS with the
// gfx950 direct-to-LDS copy (global_load_lds_dwordx4: 16 bytes per lane, a
// wave moves 1 KB per copy, no registers involved).  A k-step covers 64
// contraction values, so each X row contributes one whole 128-byte line per
// k-step (32 values, half a line, measured 8-12 % slower).  Two LDS stages
// (64 KB each for 256x256 tiles): the copies of k-step step+1 run while
// k-step step is computed, four quarter steps of 16 contraction values.  The
// barrier that publishes the next stage sits after the third quarter, whose
// MFMAs cover the wait; the fourth quarter reads the next k-step's first
// fragments and issues the copies of k-step step+2 into the stage just
// consumed.  Inside each quarter the 16 MFMAs are interleaved one by one with
// the fragment reads and the copies (pinned by scheduling barriers), so that
// the matrix cores see a steady stream instead of bursts of other
// instructions.
//
// LDS layouts (the LDS serves 256 bytes, 64 banks, per pass; both layouts
// keep every pass of the reads used here on distinct banks):
//  * X tile: row r of the tile keeps its eight 16-byte pieces (8 contraction
//    values each) at piece c ^ ((r >> 1) & 7).  MFMA fragments are plain
//    128-bit reads (lane: row l % 32, piece 2*ks + l / 32 for quarter ks).
//  * W tile: contraction row k keeps the tile's BN columns in the weight
//    bank's own row-major order, its 64-byte groups (32 columns) permuted by
//    g ^ s(k) (swz_rm: k & 3 for BN 256 and 128, (k >> 1) & 1 for BN 192).  The
//    MFMA needs 8 consecutive contraction values per lane, so the fragment is
//    read with two ds_read_b64_tr_b16 (gfx950 transposing LDS read): in a
//    16-lane group, lane t's element e comes from element t % 4 of the
//    8-byte read issued by lane 4e + t / 4, so lanes that read 4 rows x 4
//    columns each receive one column x 4 rows.
// The MFMA is v_mfma_f32_32x32x16_bf16 with the weight fragment as the first
// operand, so each lane ends with four consecutive output columns of one row;
// the 256x256 tile runs on 8 waves, two per SIMD, each a 128x64 wave tile
// (4x2 MFMA tiles): the second wave's MFMAs issue while the first one reads
// fragments or copies (measured 1-4 % faster than 4 waves of 128x128 tiles,
// which held all 256 accumulator registers per lane); 128x256 tiles likewise
// (8 waves of 64x64, 2-3 % on the 768 -> 3072 projection); the other tile
// shapes and the gated epilogue keep 4 waves.
//
// Rows.  For a cyclic schedule (tau[m] = (o + m) mod q for all m, detected by
// the index) the rows of type i are the arithmetic progression
// (i - o) mod q + k q and are computed, never loaded; otherwise the index's
// row list is read one tile ahead of its use.
//
// Rows whose type is out of range (listed after all typed rows by the index)
// are written as zero by the same launch.
#include <type_traits>

#include "qalg.h"
#include "qalg_internal.h"
#include "qalg_device.h"

namespace qalg {

namespace {

using namespace dev;

constexpr int kBK = 64;       // contraction per k-step (128-byte X row segments)
constexpr int kStages = 2;    // LDS stages: the next k-step's operands arrive while one is computed
constexpr int kQ = kBK / 16;  // MFMA quarter steps per k-step

// GATED: the gate/up half of a gated FFN over a merged weight bank (see the
// gated entry point below): each wave's 128 accumulator columns are 64 gate
// and the matching 64 up columns, and the epilogue writes silu(gate) * up.
// WGM x WGN waves per workgroup (4 or 8); the low tile heights (for few rows
// per type) use 1 x 4 or 2 x 2 so that every wave still has at least 2 x 2
// MFMA blocks.
// KEEP_ (gated only): also store the merged pre-activations GU in bf16 and
// compute H from those rounded values (the training step keeps GU for the VJP).
template <int BM_, int BN_, bool GATED_ = false, int WGM_ = 2, int WGN_ = 2, bool KEEP_ = false>
struct FwdCfg {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_;
  static constexpr int NW = WGM * WGN;
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  static constexpr bool GATED = GATED_;
  static constexpr bool KEEP = KEEP_;
  static_assert(!KEEP || GATED, "pre-activations are kept by the gated forward only");
  static constexpr int THREADS = 64 * NW;
  static constexpr int WTM = BM / WGM, WTN = BN / WGN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0 && FM >= 1 && FN >= 1, "wave tile");
  // X tile: BM rows of 128 bytes (64 contraction values), 16-byte pieces swizzled
  static constexpr int A_BYTES = BM * kBK * 2;
  static constexpr int AROWB = kBK * 2;
  // W tile: 64 contraction rows of BN*2 bytes, 16-byte pieces swizzled
  static constexpr int ROWB = BN * 2;
  static constexpr int NCH = BN / 8;                // 16-byte pieces per W row
  static constexpr int B_BYTES = kBK * ROWB;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0, "whole 1 KB copies per wave");
  static constexpr int A_DMA = A_BYTES / (1024 * NW);  // 1 KB direct-to-LDS copies per wave and k-step
  static constexpr int B_DMA = B_BYTES / (1024 * NW);
  static constexpr int DMA = A_DMA + B_DMA;
  static_assert(kStages * DMA < 64, "vmcnt range");
  // epilogue: each wave restages 32 rows x WTN columns of bf16 at a time in
  // its own share of a buffer behind the stages
  static constexpr int OUT_WTN = GATED ? WTN / 2 : WTN;  // output columns per wave tile
  static_assert(!GATED || FN % 2 == 0, "gate and up halves of a wave tile");
  static constexpr int E_PITCH = OUT_WTN * 2;      // bytes per restaged row
  static constexpr int E_NP = OUT_WTN / 8;         // 16-byte pieces per row
  // gated: a 32-row slice of one half (gate or up) of the wave's columns in fp32
  static constexpr int E_BYTES = GATED ? 32 * OUT_WTN * 4 : 32 * E_PITCH;
  static constexpr int E_MASK = E_NP == 12 ? 3 : E_NP - 1;  // piece swizzle: p ^ (row & E_MASK)
  static_assert(E_NP % 2 == 0 && (E_NP == 12 || (E_NP & E_MASK) == 0), "epilogue buffer");
  static constexpr int E_OFF = kStages * STAGE;
  static constexpr int LDS_BYTES = E_OFF + NW * E_BYTES;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};


struct FwdArgs {
  const char* X;
  const char* W;
  char* Y;
  const int32_t* ws;
  int64_t off_offsets, off_tiles, off_rows;
  int q, M, K, N, s, r;
  int cpg;     // column tiles per output group
  int n_ct;    // column tiles in all (q * cpg)
  int kts;     // k-steps per contraction segment (s / kBK)
  int out_n;   // columns of an output row (N; N / 2 for the gated epilogue)
  int L;       // 0: the complete-graph law Q_q; L >= 1: the recursive law Q_2^(x)L (q = 2^L)
  const uint64_t* adj;  // graph law Q_G (complete-law kernels): out-edges of each type; null for Q_q
  char* GU;             // gated forward with kept pre-activations: M x N merged GU (bf16); else null
  // unequal group widths (eq 18), complete law: widths = 1; first K column of
  // input group g, first N column and first column tile of output group g
  int widths;
  int gk[kMaxWidthGroups + 1], gn[kMaxWidthGroups + 1], tn[kMaxWidthGroups + 1];
};

// One output tile, decoded from its position in the tile order.
struct Tile {
  int i;          // row type
  int rank0;      // rank of the tile's first row among the rows of its type
  int first;      // first slot of the tile's rows in the index's row list
  int m_cnt;      // rows in the tile
  int n0;         // first output column
  int seg0, seg1; // K offsets of the contraction segments (group i, group j)
  int nk;         // k-steps
  int kts0;       // k-steps of the first segment (group i)
  int fmask;      // recursive law: bits where i and j differ (free bits of the segments)
  int fbase;      // recursive law: i's bits elsewhere (segment n is fbase | pdep(n, fmask))
};

// The recursive law Q_2^(x)L (appendix C): types and groups are L-bit strings,
// and output group j of a type-i row sums x_b W_bj over every b whose bits each
// equal i's or j's (eq 36), i.e. b = (i & ~m) | (any subset of m), m = i ^ j:
// 2^popcount(m) segments.  Tiles fall in L + 1 classes by d = popcount(m), with
// C(L, d) output groups per type and 2^d segments each (binom_small and
// unrank_mask enumerate them).
// scatter the low bits of n into the set bits of m
__device__ __forceinline__ int deposit_bits(int n, int m, int L) {
  int b = 0;
  for (int k = 0; k < L; ++k)
    if ((m >> k) & 1) {
      if (n & 1) b |= 1 << k;
      n >>= 1;
    }
  return b;
}

// Tile list of a workgroup for the recursive law: each XCD takes a contiguous
// share of every class; its workgroups are dealt the concatenation of those
// shares, longest class first, round robin, so k-steps per workgroup end within
// one tile of each other.
struct ClassDeal {
  int L, n_rt, cpg, xcd, nx, g, G, k;
  __device__ void init(int L_, int n_rt_, int cpg_, int xcd_, int nx_, int slot, int per_x) {
    L = L_;
    n_rt = n_rt_;
    cpg = cpg_;
    xcd = xcd_;
    nx = nx_;
    g = slot;
    G = per_x;
    k = 0;
  }
  __device__ bool next(int* cls, int* idx) {
    int p = uni(g + k * G);
    k = uni(k + 1);
    for (int d = L; d >= 0; --d) {
      const int T = n_rt * binom_small(L, d) * cpg;
      const int x0 = T * xcd / nx, x1 = T * (xcd + 1) / nx;
      if (p < x1 - x0) {
        *cls = d;
        *idx = x0 + p;
        return true;
      }
      p -= x1 - x0;
    }
    return false;
  }
};

// the two-class deal of the complete law, with the class as an int (1: long)
struct TileDeal2 : TileDeal {
  __device__ bool next(int* cls, int* idx) {
    bool lg;
    const bool ok = TileDeal::next(&lg, idx);
    *cls = lg ? 1 : 0;
    return ok;
  }
};

// Tiles come in two lengths: "long" tiles (output group j != row type i, two
// contraction segments) and "short" ones (j == i, one segment).  Each class is
// ordered in groups of up to 4 row tiles x the class's column tiles, row tile
// fastest (measured against 2, 8 and 16 row tiles: the least L2 refetch for
// 256x256 tiles); idx is the tile's position in its class.
// Complete law: cls 1 is the long class, 0 the short one.  Recursive law: cls
// is d, the Hamming distance between row type and output group.
template <class C, bool TENSOR, class IX>
__device__ __forceinline__ Tile decode_tile(const FwdArgs& a, const IX& ix, int n_rt, int cls, int idx) {
  constexpr int G = 4;
  if constexpr (!TENSOR) {
    if (a.widths) {
      // unequal widths: one class, groups of 4 row tiles x all n_ct column
      // tiles (row tile fastest); the tile's output group j from the column
      // tile starts, its contraction over groups i and j (i alone if j == i)
      const int span = G * a.n_ct;
      const int g = idx / span;
      const int first_rt = g * G;
      const int gm = min(n_rt - first_rt, G);
      const int w = idx - g * span;
      const int rt = first_rt + w % gm;
      const int c2 = w / gm;
      const int i = ix.group_of_tile(rt);
      int j = 0;
      while (j + 1 < a.q && c2 >= a.tn[j + 1]) j = uni(j + 1);
      Tile t;
      t.i = i;
      t.rank0 = (rt - ix.tiles_before(i)) * C::BM;
      t.first = ix.offset(i) + t.rank0;
      t.m_cnt = min(C::BM, ix.count(i) - t.rank0);
      t.n0 = a.gn[j] + (c2 - a.tn[j]) * C::BN;
      t.seg0 = a.gk[i];
      t.seg1 = a.gk[j];
      t.kts0 = uni((a.gk[i + 1] - a.gk[i]) / kBK);
      t.nk = uni(t.kts0 + (j == i ? 0 : (a.gk[j + 1] - a.gk[j]) / kBK));
      t.fmask = t.fbase = 0;
      return t;
    }
  }
  const bool is_long = cls != 0;
  const int ngrp = TENSOR ? binom_small(a.L, cls) : (is_long ? a.q - 1 : 1);
  const int ncol = ngrp * a.cpg;  // column tiles of the class per row tile
  const int span = G * ncol;
  const int g = idx / span;
  const int first_rt = g * G;
  const int gm = min(n_rt - first_rt, G);
  const int w = idx - g * span;
  const int rt = first_rt + w % gm;
  const int c2 = w / gm;
  const int i = ix.group_of_tile(rt);
  int ct;
  Tile t;
  if constexpr (TENSOR) {
    const int jj = c2 / a.cpg, cc = c2 - jj * a.cpg;
    const int m = unrank_mask(jj, cls, a.L);
    ct = (i ^ m) * a.cpg + cc;
    t.fmask = m;
    t.fbase = i & ~m;
  } else if (is_long) {
    const int jj = c2 / a.cpg, cc = c2 - jj * a.cpg;
    ct = (jj < i ? jj : jj + 1) * a.cpg + cc;  // output groups other than i
    t.fmask = t.fbase = 0;
  } else {
    ct = i * a.cpg + c2;
    t.fmask = t.fbase = 0;
  }
  t.i = i;
  t.rank0 = (rt - ix.tiles_before(i)) * C::BM;
  t.first = ix.offset(i) + t.rank0;
  t.m_cnt = min(C::BM, ix.count(i) - t.rank0);
  const int j = ct / a.cpg, cc = ct - j * a.cpg;
  t.n0 = j * a.r + cc * C::BN;
  if constexpr (TENSOR) {
    t.seg0 = t.fbase * a.s;  // segment 0: no free bit set
    t.seg1 = 0;
    t.nk = uni(a.kts << cls);
  } else {
    t.seg0 = i * a.s;
    t.seg1 = j * a.s;
    t.kts0 = a.kts;
    t.nk = uni((j == i) ? a.kts : 2 * a.kts);
    if (a.adj != nullptr && j != i) {
      // graph law Q_G: without the edge (i, j) the output block has no term
      // (eq 9: edge * edge and unmatched slots vanish); its zeros are written
      // before the launch, and the tile does no work
      const cint_ptr e = to_const(reinterpret_cast<const int32_t*>(a.adj));
      const int word = uni(e[2 * i + (j >> 5)]);
      if (!((word >> (j & 31)) & 1)) t.nk = 0;
    }
  }
  return t;
}

template <class C, bool CYC, bool TENSOR>
__device__ __forceinline__ void fwd_body(const FwdArgs& a, char* smem) {
  constexpr int BM = C::BM, T = C::THREADS;
  const int32_t* ws = a.ws;
  const int32_t* rows = ws + a.off_rows;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);

  // per-type row offsets and row-tile offsets, read through the scalar data
  // cache (tile decoding then never waits on the vector-memory counter, which
  // also counts the copies in flight, and the LDS is left to the stages)
  const cint_ptr s_off = to_const(ws + a.off_offsets);
  const cint_ptr s_toff = to_const(ws + a.off_tiles + tile_height_slot(BM) * (a.q + 1));
  // tile decoding: closed form for a cyclic schedule (no memory access on the
  // way to the next tile), the index tables otherwise
  using IX = std::conditional_t<CYC, CycIndex, MemIndex>;
  IX ix;
  if constexpr (CYC)
    ix = CycIndex::make(a.q, uni(ws[4]), a.M, BM);
  else
    ix = MemIndex{s_off, s_toff, a.q};

  // rows of an out-of-range type: zero output rows (rare)
  {
    const int typed = uni(s_off[a.q]);
    const int nbad = a.M - typed;
    const int row_u4 = a.out_n / 8;  // 16-byte pieces per output row
    for (int b = blockIdx.x; b < nbad; b += gridDim.x) {
      u32x4* yr = reinterpret_cast<u32x4*>(a.Y + int64_t(rows[typed + b]) * a.out_n * 2);
      for (int x = tid; x < row_u4; x += T) yr[x] = (u32x4){0u, 0u, 0u, 0u};
      if constexpr (C::KEEP) {
        u32x4* gr = reinterpret_cast<u32x4*>(a.GU + int64_t(rows[typed + b]) * a.N * 2);
        for (int x = tid; x < a.N / 8; x += T) gr[x] = (u32x4){0u, 0u, 0u, 0u};
      }
    }
  }

  // this workgroup's tiles: contiguous shares of the long and of the short
  // tiles per XCD (workgroup w runs on XCD w mod 8 when the grid is one
  // workgroup per CU), dealt so that k-steps per workgroup are balanced
  const int n_rt = ix.tiles_before(a.q);
  const int n_long = n_rt * (a.q - 1) * a.cpg, n_short = n_rt * a.cpg;
  const int nx = gridDim.x >= 8 ? 8 : 1;
  const int per_x = gridDim.x / nx;
  const int xcd = blockIdx.x % nx, slot = blockIdx.x / nx;
  if (slot >= per_x) return;  // grid not a multiple of 8: the remainder idles
  using Deal = std::conditional_t<TENSOR, ClassDeal, TileDeal2>;
  Deal dcopy, dcomp;
  if constexpr (TENSOR)
    dcopy.init(a.L, n_rt, a.cpg, xcd, nx, slot, per_x);
  else if (a.widths)
    dcopy.init(n_rt * a.n_ct, 0, 2 * a.kts, a.kts, xcd, nx, slot, per_x);  // one class, all tiles
  else
    dcopy.init(n_long, n_short, 2 * a.kts, a.kts, xcd, nx, slot, per_x);
  dcomp = dcopy;
  int l_long;  // class of the copy cursor's next tile
  int l_idx;
  // the next tile with work (graph-law tiles of absent edges have none and are
  // skipped by both cursors alike)
  auto next_work = [&](Deal& d, int* cls, int* idx, Tile* t) -> bool {
    for (;;) {
      if (!d.next(cls, idx)) return false;
      *t = decode_tile<C, TENSOR>(a, ix, n_rt, *cls, uni(*idx));
      if (t->nk > 0) return true;
    }
  };
  Tile lt0;
  if (!next_work(dcopy, &l_long, &l_idx, &lt0)) return;

  const uint32_t n_bytes = uint32_t(a.N) * 2u;      // bytes per weight row
  const uint32_t y_bytes = uint32_t(a.out_n) * 2u;  // bytes per output row
  const uint32_t k_bytes = uint32_t(a.K) * 2u;
  // cyclic schedule: the k-th row of type i is (i - cyc) mod q + k q, no row list needed
  const int cyc = ws[4];
  auto row_of = [&](const Tile& t, int r) -> int {
    if constexpr (CYC) {
      const int start = t.i >= cyc ? t.i - cyc : t.i - cyc + a.q;
      return start + (t.rank0 + r) * a.q;
    }
    return rows[t.first + r];
  };

  // ---------------- copy cursor: direct global -> LDS copies, 3 k-steps ahead ----------------
  // copy u of this wave moves 1 KB: lane l carries 16-byte slot (wid * DMA_x + u) * 64 + l
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>(smem)));
  uint32_t b_src[C::B_DMA];  // byte offset of the lane's W piece relative to (k-step row 0, n0)
#pragma unroll
  for (int u = 0; u < C::B_DMA; ++u) {
    const int sl = (wid * C::B_DMA + u) * 64 + lane;
    const int k = sl / C::NCH, p = sl - (sl / C::NCH) * C::NCH;
    const int c = p ^ swz_rm<C::ROWB>(k);
    b_src[u] = uint32_t(k) * n_bytes + uint32_t(c) * 16u;
  }
  int a_row[C::A_DMA];   // tile-local row of each X copy slot, and its swizzled piece
  uint32_t a_pc[C::A_DMA];
#pragma unroll
  for (int u = 0; u < C::A_DMA; ++u) {
    const int sl = (wid * C::A_DMA + u) * 64 + lane;
    a_row[u] = sl >> 3;
    a_pc[u] = uint32_t((sl & 7) ^ swz_x128(sl >> 3)) * 16u;
  }
  // row ids are fetched one tile ahead of their use (listed schedules only),
  // so that the wait for them overlaps a whole tile
  int pre_row[C::A_DMA];
  auto prefetch_rows = [&](const Tile& t) {
#pragma unroll
    for (int u = 0; u < C::A_DMA; ++u) pre_row[u] = row_of(t, min(a_row[u], t.m_cnt - 1));
  };
  uint32_t a_src[C::A_DMA];
  auto take_rows = [&]() {
#pragma unroll
    for (int u = 0; u < C::A_DMA; ++u) a_src[u] = uint32_t(pre_row[u]) * k_bytes + a_pc[u];
  };

  // copy cursor: tile lt at k-step lk; the tile after it is decoded ahead so
  // that a listed schedule's row ids are fetched a whole tile before use
  Tile lt = lt0;
  int lk = 0;
  Tile nt = lt;
  bool have_next = next_work(dcopy, &l_long, &l_idx, &nt);
  if (!have_next) nt = lt;
  prefetch_rows(lt);
  take_rows();
  if (have_next) prefetch_rows(nt);
  bool more = true;  // the copy cursor has not passed the last k-step
  // copy cursor split in three so that the copies can be interleaved with MFMAs
  uint32_t cp_x = 0, cp_w = 0;  // per-step byte offsets of the X and W pieces
  // recursive law: k-step within the current segment, segment number, its K offset
  int lks = 0, lseg = 0, lcol = lt.seg0;
  auto prep_copies = [&]() {
    int kcol;
    if constexpr (TENSOR) {
      kcol = lcol + lks * kBK;
    } else {
      const int sg = lk >= lt.kts0 ? 1 : 0;
      kcol = (sg ? lt.seg1 : lt.seg0) + (lk - sg * lt.kts0) * kBK;
    }
    cp_x = uint32_t(kcol) * 2u;
    cp_w = uint32_t(kcol) * n_bytes + uint32_t(lt.n0) * 2u;
  };
  auto copy_u = [&](int stage, int u) {
    const uint32_t S = lds0 + uint32_t(stage * C::STAGE);
    if (u < C::A_DMA)
      copy16_to_lds(a.X, a_src[u] + cp_x, S + uint32_t((wid * C::A_DMA + u) * 1024));
    else
      copy16_to_lds(a.W, cp_w + b_src[u - C::A_DMA], S + uint32_t(C::A_BYTES + (wid * C::B_DMA + (u - C::A_DMA)) * 1024));
  };
  // After the last k-step the cursor stays on it: the copies issued for the
  // k-steps past the end repeat it into a stage that is never read, so
  // that the pipeline needs no conditions (they are drained before exit).
  auto advance_copies = [&]() {
    if constexpr (TENSOR) {
      if (!more) return;
      if (uni(lk + 1) < lt.nk) {
        lk = uni(lk + 1);
        if (uni(lks + 1) == a.kts) {
          lks = 0;
          lseg = uni(lseg + 1);
          lcol = uni((lt.fbase | deposit_bits(lseg, lt.fmask, a.L)) * a.s);
        } else {
          lks = uni(lks + 1);
        }
        return;
      }
      if (!have_next) {
        more = false;  // the cursor stays on the last k-step
        return;
      }
      lt = nt;
      lk = 0;
      lks = 0;
      lseg = 0;
      lcol = lt.seg0;
      take_rows();
      have_next = next_work(dcopy, &l_long, &l_idx, &nt);
      if (have_next) prefetch_rows(nt);
      return;
    }
    if (more && (lk = uni(lk + 1)) >= lt.nk) {
      if (!have_next) {
        more = false;
        lk = uni(lt.nk - 1);
      } else {
        lt = nt;
        lk = 0;
        take_rows();
        have_next = next_work(dcopy, &l_long, &l_idx, &nt);
        if (have_next) prefetch_rows(nt);
      }
    }
  };
  auto issue_copies = [&](int stage) {
    prep_copies();
#pragma unroll
    for (int u = 0; u < C::DMA; ++u) copy_u(stage, u);
    advance_copies();
  };

  // ---------------- fragment reads ----------------
  const int wm = wid / C::WGN, wn = wid % C::WGN;
  const int l32 = lane & 31, lhi = lane >> 5;
  // X fragment (32 rows x 16 contraction): lane reads row l32, piece 2*ks + lhi
  int a_rd[kQ];
#pragma unroll
  for (int ks = 0; ks < kQ; ++ks)
    a_rd[ks] = (wm * C::WTM + l32) * C::AROWB + (((2 * ks + lhi) ^ swz_x128(l32)) << 4);
  // W fragment (32 columns x 16 contraction) as two transposing 8-byte reads per lane:
  // in a 16-lane group (g = lane / 16, t = lane % 16) lane t reads row 8*(g/2) + t/4 (+4),
  // columns 16*(g%2) + 4*(t%4) of the fragment; the transpose hands lane t column t, 4 rows.
  // b_rd[fn]: the lane's offset for the wave's fragment fn (32-column block m0 + fn,
  // stored as group (m0 + fn) ^ s(row)); a row 4 or 16 further has the same s.
  const int m0 = wn * (C::WTN / 32);  // block index of the wave's first 32-column block
  int b_rd[C::FN];
  {
    const int g = lane >> 4, t = lane & 15;
    const int k_l = 8 * (g >> 1) + (t >> 2);
    const int r2 = 2 * (g & 1) + ((t & 3) >> 1);
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
      b_rd[fn] = C::A_BYTES + k_l * C::ROWB + ((((m0 + fn) * 4) ^ swz_rm<C::ROWB>(k_l)) + r2) * 16 + 8 * (t & 1);
  }

  f32x16 acc[C::FM][C::FN];
  // fragments of the two 16-wide halves of a k-step (registers double buffered)
  bf16x8 fa0[C::FM], fb0[C::FN], fa1[C::FM], fb1[C::FN];
  auto read_a = [&](int stage, int ks, int fm) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(smem + stage * C::STAGE + a_rd[ks] + fm * 32 * C::AROWB);
  };
  auto read_b = [&](int stage, int ks, int fn) -> bf16x8 {
    const char* p = smem + stage * C::STAGE + b_rd[fn] + 16 * ks * C::ROWB;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(p));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(p + 4 * C::ROWB));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // fragment read j of a half k-step, in the order the MFMAs (x = fm * FN + fn)
  // first need them: a[0], b[0..FN-1], a[1..FM-1]
  auto read_slot = [&](int j, int stage, int ks, bf16x8 (&fa)[C::FM], bf16x8 (&fb)[C::FN]) {
    if (j == 0)
      fa[0] = read_a(stage, ks, 0);
    else if (j <= C::FN)
      fb[j - 1] = read_b(stage, ks, j - 1);
    else
      fa[j - C::FN] = read_a(stage, ks, j - C::FN);
  };
  auto load_frags = [&](int stage, int ks, bf16x8 (&fa)[C::FM], bf16x8 (&fb)[C::FN]) {
    const char* S = smem + stage * C::STAGE;
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
      fa[fm] = *reinterpret_cast<const bf16x8*>(S + a_rd[ks] + fm * 32 * C::AROWB);
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      const char* p = S + b_rd[fn] + 16 * ks * C::ROWB;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(p));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(p + 4 * C::ROWB));
      fb[fn] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  auto mfmas = [&](const bf16x8 (&fa)[C::FM], const bf16x8 (&fb)[C::FN]) {
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[fn], fa[fm], acc[fm][fn], 0, 0, 0);
  };

  // ---------------- pipeline ----------------
  // Two stages: while k-step `step` is computed from one, the copies of
  // k-step step+1 land in the other.  A k-step is four quarter steps of 16
  // contraction values; fragments are double buffered in registers, each
  // quarter's MFMAs interleaved with the reads of the next quarter's
  // fragments.  The barrier sits after the third quarter: by then every wave
  // has issued (and the barrier's fence completed) all its reads of the
  // current stage, so the fourth quarter reads the next k-step's first
  // fragments from the other stage and copies k-step step+2 into this one.
  issue_copies(0);
  issue_copies(1);
  wait_vmcnt<C::DMA>();
  lds_barrier();
  load_frags(0, 0, fa0, fb0);

  int c_long;
  int c_idx;
  Tile ct = lt0;
  next_work(dcomp, &c_long, &c_idx, &ct);
  int stage = 0;  // LDS stage of the current k-step (k-step mod 2)
  static_assert(C::FM + C::FN <= C::FM * C::FN, "fragment reads fit a quarter step");
  // one quarter step: MFMAs on fragments (fa, fb) of quarter ks, each followed
  // by one read of quarter ks + 1's fragments into (ga, gb)
  auto quarter = [&](int ks, const bf16x8 (&fa)[C::FM], const bf16x8 (&fb)[C::FN], bf16x8 (&ga)[C::FM],
                     bf16x8 (&gb)[C::FN]) {
#pragma unroll
    for (int x = 0; x < C::FM * C::FN; ++x) {
      const int fm = x / C::FN, fn = x % C::FN;
      acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[fn], fa[fm], acc[fm][fn], 0, 0, 0);
      if (x < C::FM + C::FN) read_slot(x, stage, ks + 1, ga, gb);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (;;) {
    // output rows of this tile, loaded now and used after its last k-step
    int out_row[C::FM];
    if constexpr (!CYC) {
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm) out_row[fm] = row_of(ct, min(wm * C::WTM + fm * 32 + l32, ct.m_cnt - 1));
    }
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) acc[fm][fn] = (f32x16){};

    for (int ck = 0; ck < ct.nk; ++ck) {
      quarter(0, fa0, fb0, fa1, fb1);
      quarter(1, fa1, fb1, fa0, fb0);
      quarter(2, fa0, fb0, fa1, fb1);
      // the copies of k-step step+1 (the only ones in flight) are complete
      wait_vmcnt<0>();
      lds_barrier();
      prep_copies();
      const int nstage = stage ^ 1;
      // last quarter: MFMAs on fragments 1 interleaved with the reads of the
      // next k-step's first fragments (stale past the last k-step, never used)
      // and the copies of k-step step+2 into this k-step's stage; narrow tiles
      // have fewer MFMAs than copies, the slots past the last MFMA carry the rest
      constexpr int kSlots = C::FM * C::FN > C::DMA ? C::FM * C::FN : C::DMA;
#pragma unroll
      for (int x = 0; x < kSlots; ++x) {
        if (x < C::FM * C::FN) {
          const int fm = x / C::FN, fn = x % C::FN;
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb1[fn], fa1[fm], acc[fm][fn], 0, 0, 0);
        }
        if (x < C::FM + C::FN) read_slot(x, nstage, 0, fa0, fb0);
        if (x < C::DMA) copy_u(stage, x);
        __builtin_amdgcn_sched_barrier(0);
      }
      advance_copies();
      stage = uni(nstage);
    }

    // epilogue: one rounding of each fp32 sum.  The MFMA layout leaves each
    // lane with pieces of one row, so a direct store would touch 32 rows per
    // instruction; instead each 32-row slice of the wave tile is written to
    // the wave's share of the LDS behind the stages and read back
    // row-contiguous, so that a store instruction writes whole rows of
    // 16-byte pieces.
    {
      char* ebuf = smem + C::E_OFF + wid * C::E_BYTES;
      // first output column of the wave (gated: the tile's 256 merged columns
      // hold 128 output columns, 64 per wave)
      const uint32_t col0 = uint32_t((C::GATED ? ct.n0 / 2 : ct.n0) + wn * C::OUT_WTN) * 2u;
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm) {
        if constexpr (C::GATED) {
          // h = silu(gate) * up in fp32, one rounding.  Gate column c sits in
          // block fn, its up column in block fn + FN/2 (same lane and
          // register).  Reading the two blocks together makes the register
          // allocator spill the accumulators, so each half goes through the
          // wave's LDS share in fp32 on its own: the gate half is written and
          // read back row-contiguous, then the up half at the same positions.
          // Slice layout: row l32 of 64 fp32 in 16-byte pieces, piece p kept
          // at p ^ (row & 15) (conflict-free for both the writes and the reads).
          constexpr int HN = C::FN / 2;  // 32-column blocks per half
          static_assert(HN * 32 == C::OUT_WTN && C::OUT_WTN == 64, "gated slice layout");
          auto write_half = [&](int fb) {
#pragma unroll
            for (int fn = 0; fn < HN; ++fn)
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                const f32x16& v = acc[fm][fb + fn];
                const int pc = (fn * 8 + g * 2 + lhi) ^ (l32 & 15);
                *reinterpret_cast<u32x4*>(ebuf + l32 * 256 + pc * 16) =
                    (u32x4){__float_as_uint(v[4 * g]), __float_as_uint(v[4 * g + 1]),
                            __float_as_uint(v[4 * g + 2]), __float_as_uint(v[4 * g + 3])};
              }
          };
          // lane: row it * 8 + lane / 8, output piece lane % 8 (8 columns)
          auto read_piece = [&](int it, float (&x)[8]) {
            const int row = it * 8 + (lane >> 3), p8 = lane & 7;
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              const u32x4 w = *reinterpret_cast<const u32x4*>(ebuf + row * 256 + (((2 * p8 + h2) ^ (row & 15)) << 4));
#pragma unroll
              for (int e = 0; e < 4; ++e) x[4 * h2 + e] = __uint_as_float(w[e]);
            }
          };
          float gate[4][8];
          write_half(0);
#pragma unroll
          for (int it = 0; it < 4; ++it) read_piece(it, gate[it]);
          write_half(HN);
#pragma unroll
          for (int it = 0; it < 4; ++it) {
            float up[8], h[8];
            read_piece(it, up);
            const int row = it * 8 + (lane >> 3), p8 = lane & 7;
            const int ml = wm * C::WTM + fm * 32 + row;
            int orow;
            if constexpr (CYC)
              orow = row_of(ct, ml);
            else
              orow = __shfl(out_row[fm], row);
            if constexpr (C::KEEP) {
              // the pre-activations in bf16 (the wave's 128 merged columns are
              // 64 gate then the matching 64 up), and H from those rounded values
              const u32x2 g0 = pack4_bf16(gate[it][0], gate[it][1], gate[it][2], gate[it][3]);
              const u32x2 g1 = pack4_bf16(gate[it][4], gate[it][5], gate[it][6], gate[it][7]);
              const u32x2 u0 = pack4_bf16(up[0], up[1], up[2], up[3]), u1 = pack4_bf16(up[4], up[5], up[6], up[7]);
              const u32x4 gq = {g0[0], g0[1], g1[0], g1[1]}, uq = {u0[0], u0[1], u1[0], u1[1]};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                gate[it][2 * e] = __uint_as_float(gq[e] << 16);
                gate[it][2 * e + 1] = __uint_as_float(gq[e] & 0xffff0000u);
                up[2 * e] = __uint_as_float(uq[e] << 16);
                up[2 * e + 1] = __uint_as_float(uq[e] & 0xffff0000u);
              }
              if (ml < ct.m_cnt) {
                char* gr = a.GU + (uint32_t(orow) * n_bytes + uint32_t(ct.n0 + wn * 128 + p8 * 8) * 2u);
                __builtin_nontemporal_store(gq, reinterpret_cast<u32x4*>(gr));
                __builtin_nontemporal_store(uq, reinterpret_cast<u32x4*>(gr + 128));
              }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float gv = gate[it][e];
              // sigmoid through the hardware reciprocal (about 1 ulp; the
              // result is rounded to bf16 next)
              h[e] = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * up[e];
            }
            const u32x2 lo = pack4_bf16(h[0], h[1], h[2], h[3]), hi = pack4_bf16(h[4], h[5], h[6], h[7]);
            const u32x4 val = {lo[0], lo[1], hi[0], hi[1]};
            // a store instruction writes 8 whole 128-byte output rows
            if (ml < ct.m_cnt)
              __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(a.Y + (uint32_t(orow) * y_bytes + col0 + uint32_t(p8) * 16u)));
          }
          continue;
        }
        // lane (l32, lhi) holds row l32, columns fn*32 + g*8 + lhi*4 .. +3
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x16& v = acc[fm][fn];
            const int pc = (fn * 4 + g) ^ (l32 & C::E_MASK);
            const u32x2 packed = pack4_bf16(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]);
            *reinterpret_cast<u32x2*>(ebuf + l32 * C::E_PITCH + pc * 16 + lhi * 8) = packed;
          }
        }
        // read back: 64 lanes take 64 consecutive (row, piece) slots per instruction
#pragma unroll
        for (int it = 0; it < C::E_NP / 2; ++it) {
          const int sl = it * 64 + lane;
          const int row = sl / C::E_NP, pc = sl - row * C::E_NP;
          const u32x4 val = *reinterpret_cast<const u32x4*>(ebuf + row * C::E_PITCH + ((pc ^ (row & C::E_MASK)) << 4));
          const int ml = wm * C::WTM + fm * 32 + row;
          int orow;
          if constexpr (CYC)
            orow = row_of(ct, ml);
          else
            orow = __shfl(out_row[fm], row);
          // non-temporal: the output is read much later, and keeping it out
          // of L2 leaves the cache to the operand tiles (measured 11 % on the
          // 4096 -> 12288 projection against plain stores)
          if (ml < ct.m_cnt)
            __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(a.Y + (uint32_t(orow) * y_bytes + col0 + uint32_t(pc) * 16u)));
        }
      }
    }
    if (!next_work(dcomp, &c_long, &c_idx, &ct)) break;
  }
  // the repeated copies past the last k-step land in LDS: drain them before
  // the workgroup's LDS can be handed to another workgroup
  wait_vmcnt<0>();
}

// one kernel per law: the recursive law's cursor state stays out of the
// complete law's register allocation
template <class C, bool TENSOR>
__global__ __launch_bounds__(C::THREADS, 1) void fwd_persistent_kernel(FwdArgs a) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int32_t* ws = a.ws;
  if (ws[1] != kIndexMagic || ws[2] != a.q || ws[3] != a.M) return;
  // two instantiations: the cyclic one never reads the row list, so it has no
  // global loads for the compiler to wait on inside the pipeline
  if (ws[4] >= 0)
    fwd_body<C, true, TENSOR>(a, smem);
  else
    fwd_body<C, false, TENSOR>(a, smem);
}

using Fwd256x256 = FwdCfg<256, 256, false, 2, 4>;
using Fwd256x256Gated = FwdCfg<256, 256, true>;
using Fwd256x256GatedKeep = FwdCfg<256, 256, true, 2, 2, true>;
using Fwd256x192 = FwdCfg<256, 192>;
using Fwd256x128 = FwdCfg<256, 128>;
// few rows per type: 128- and 64-row tiles (64 x 64 and 64 x 128 wave tiles)
using Fwd128x256 = FwdCfg<128, 256, false, 2, 4>;
using Fwd128x128 = FwdCfg<128, 128>;
using Fwd128x192 = FwdCfg<128, 192>;
using Fwd64x256 = FwdCfg<64, 256, false, 1, 4>;

int cu_count() {
  static int n = 0;
  if (n == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
  }
  return n;
}

template <class C, bool TENSOR>
hipError_t set_lds_limit() {
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&fwd_persistent_kernel<C, TENSOR>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  return hipSuccess;
}

template <class C>
hipError_t launch_fwd(const ProblemDesc& p, hipStream_t s) {
  const bool tensor = p.law_L > 0;
  const hipError_t e = tensor ? set_lds_limit<C, true>() : set_lds_limit<C, false>();
  if (e != hipSuccess) return e;
  FwdArgs a{};
  a.X = static_cast<const char*>(p.A);
  a.W = static_cast<const char*>(p.B);
  a.Y = static_cast<char*>(p.C);
  a.ws = p.ws;
  const WsLayout L = ws_layout(p.q, p.M);
  a.off_offsets = L.offsets;
  a.off_tiles = L.tile_off;
  a.off_rows = L.rows;
  a.q = p.q;
  a.M = int(p.M);
  a.K = int(p.K);
  a.N = int(p.N);
  a.s = int(p.K / p.q);
  a.r = int(p.N / p.q);
  a.kts = a.s / kBK;
  a.out_n = C::GATED ? a.N / 2 : a.N;
  a.L = p.law_L;
  a.adj = p.graph_adj;
  a.GU = static_cast<char*>(p.gu);
  a.cpg = a.r / C::BN;
  a.n_ct = p.q * a.cpg;
  if (p.in_widths != nullptr) {
    // unequal widths: group starts and column-tile starts from the widths
    a.widths = 1;
    a.gk[0] = a.gn[0] = a.tn[0] = 0;
    for (int g = 0; g < p.q; ++g) {
      a.gk[g + 1] = a.gk[g] + int(p.in_widths[g]);
      a.gn[g + 1] = a.gn[g] + int(p.out_widths[g]);
      a.tn[g + 1] = a.tn[g] + int(p.out_widths[g] / C::BN);
    }
    a.n_ct = a.tn[p.q];
    a.cpg = 0;
  }
  const int64_t max_tiles = ((p.M + C::BM - 1) / C::BM + p.q - 1) * int64_t(a.n_ct);
  int grid = cu_count();
  if (max_tiles < grid) grid = max_tiles < 8 ? int(max_tiles) : int(max_tiles / 8 * 8);
  if (grid < 1) grid = 1;
  const size_t lds = C::LDS_BYTES;
  if (tensor)
    hipLaunchKernelGGL((fwd_persistent_kernel<C, true>), dim3(grid), dim3(C::THREADS), lds, s, a);
  else
    hipLaunchKernelGGL((fwd_persistent_kernel<C, false>), dim3(grid), dim3(C::THREADS), lds, s, a);
  return hipGetLastError();
}

}  // namespace

bool fwd_persistent_shape_ok(const ProblemDesc& p) {
  if (p.op != Op::Fwd || p.E != 1) return false;
  const int64_t s = p.K / p.q, r = p.N / p.q;
  // byte offsets of every operand fit in 32 bits
  const int64_t lim = int64_t(1) << 31;
  if (p.M * p.K >= lim || p.K * p.N >= lim || p.M * p.N >= lim) return false;
  if (s % kBK != 0) return false;
  return r % 256 == 0 || r % 192 == 0 || r % 128 == 0;
}

// Unequal group widths on the persistent forward (complete law): 256x256
// tiles, so every output width a multiple of 256 and every input width of
// 64 (whole k-steps), and at least 128 rows per type on average.
bool fwd_widths_persistent_ok(const ProblemDesc& p) {
  if (p.op != Op::Fwd || p.E != 1 || p.law_L != 0 || p.graph_adj != nullptr) return false;
  if (p.in_widths == nullptr || p.out_widths == nullptr || p.q < 1 || p.q > kMaxWidthGroups) return false;
  const int64_t lim = int64_t(1) << 31;
  if (p.M * p.K >= lim || p.K * p.N >= lim || p.M * p.N >= lim) return false;
  for (int g = 0; g < p.q; ++g)
    if (p.in_widths[g] % kBK != 0 || p.out_widths[g] % 256 != 0) return false;
  return (p.M + p.q - 1) / p.q >= 128;
}

hipError_t launch_fwd_widths_bf16(const ProblemDesc& p, hipStream_t s) { return launch_fwd<Fwd256x256>(p, s); }

bool fwd_persistent_supported(const ProblemDesc& p) {
  // with only 256-row tiles available, below about 128 rows per type the
  // register-staged kernel's 128-row tiles waste less
  if (!fwd_persistent_shape_ok(p)) return false;
  return fwd_tile_height(p, 0) < 256 || (p.M + p.q - 1) / p.q >= 128;
}

// Gated: N is the merged bank's width 2F.  Output group j's 2r merged columns
// come in 256-column pieces, each [gate 64 | up 64 | gate 64 | up 64] of 128
// consecutive output columns, so r = F / q must be a multiple of 128.
bool fwd_gated_supported(const ProblemDesc& p) {
  if (p.op != Op::Fwd || p.E != 1) return false;
  const int64_t s = p.K / p.q, r2 = p.N / p.q;
  const int64_t lim = int64_t(1) << 31;
  if (p.M * p.K >= lim || p.K * p.N >= lim || p.M * p.N >= lim) return false;
  return s % kBK == 0 && r2 % 256 == 0;
}

hipError_t launch_fwd_gated_bf16(const ProblemDesc& p, hipStream_t s) {
  return p.gu != nullptr ? launch_fwd<Fwd256x256GatedKeep>(p, s) : launch_fwd<Fwd256x256Gated>(p, s);
}

namespace {

// Merged gate/up bank: for output group j and its piece t (output columns
// j r + 128 t .. +127), merged columns j 2r + 256 t + [0, 256) hold gate
// columns +0..63, up +0..63, gate +64..127, up +64..127.  One thread per
// 16-byte piece (8 columns) of the merged bank.
__global__ void merge_gate_up_kernel(const uint16_t* Wg, const uint16_t* Wu, uint16_t* Wgu, int64_t K, int F,
                                     int r) {
  const int64_t pieces_per_row = int64_t(2) * F / 8;
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= K * pieces_per_row) return;
  const int64_t k = i / pieces_per_row;
  const int c = int(i - k * pieces_per_row) * 8;  // merged column of the piece
  const int j = c / (2 * r), w = c - j * 2 * r;
  const int t = w / 256, x = w - t * 256;
  const int blk = x / 64;
  const int h = j * r + t * 128 + (blk >> 1) * 64 + (x & 63);
  const uint16_t* src = (blk & 1) ? Wu : Wg;
  *reinterpret_cast<uint4*>(Wgu + k * 2 * F + c) = *reinterpret_cast<const uint4*>(src + k * F + h);
}

}  // namespace

namespace {

// Graph law: zero the output blocks (rows of type i, columns of group j != i)
// that no edge (i, j) reaches.  One thread per 16-byte piece of an output row.
__global__ __launch_bounds__(256) void graph_zero_kernel(const int32_t* __restrict__ tau,
                                                         const uint64_t* __restrict__ adj, int q, int64_t M,
                                                         int out_n, int r, uint16_t* __restrict__ Y) {
  const int pc = blockIdx.x * 256 + threadIdx.x;
  if (pc * 8 >= out_n) return;
  const int j = (pc * 8) / r;
  for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
    const int i = tau[m];
    if (i < 0 || i >= q || i == j || ((adj[i] >> j) & 1ull)) continue;
    *reinterpret_cast<u32x4*>(Y + m * out_n + pc * 8) = (u32x4){0u, 0u, 0u, 0u};
  }
}

}  // namespace

hipError_t launch_graph_zero_bf16(const int32_t* tau, const uint64_t* adj, int q, int64_t M, int64_t out_n,
                                  void* Y, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const int64_t bx = (out_n / 8 + 255) / 256;
  int64_t by = (2048 + bx - 1) / bx;
  if (by > M) by = M;
  if (by > 65535) by = 65535;
  hipLaunchKernelGGL(graph_zero_kernel, dim3(unsigned(bx), unsigned(by)), dim3(256), 0, s, tau, adj, q, M,
                     int(out_n), int(out_n / q), static_cast<uint16_t*>(Y));
  return hipGetLastError();
}

hipError_t launch_merge_gate_up_bf16(const void* Wg, const void* Wu, void* Wgu, int64_t K, int64_t F, int q,
                                     hipStream_t s) {
  const int64_t n = K * (2 * F / 8);
  if (n == 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (n + threads - 1) / threads;
  hipLaunchKernelGGL(merge_gate_up_kernel, dim3(unsigned(blocks)), dim3(threads), 0, s,
                     static_cast<const uint16_t*>(Wg), static_cast<const uint16_t*>(Wu), static_cast<uint16_t*>(Wgu),
                     K, int(F), int(F / q));
  return hipGetLastError();
}

// Tile height from a cost model calibrated with the sweep of calibrate.py on
// 4096 <-> 12288 at M = 2048 .. 16384, q = 8 .. 64 (128-row tiles are 256,
// 192 or 128 columns wide, whichever the group width takes first): (waves of tiles over the
// CUs) x (tile area) / (relative per-area efficiency of the height: 1, 0.85
// and 0.6 for 256, 128 and 64 rows).  Few rows per type favour low tiles (a
// 256-row tile of a 64-row type is 3/4 padding); few tiles in all favour low
// tiles too (more workgroups busy); many rows favour the most efficient tile.
int fwd_tile_height(const ProblemDesc& p, int forced) {
  const int64_t r = p.N / p.q;
  const bool ok64 = r % 256 == 0, ok128 = r % 128 == 0 || r % 192 == 0;
  if (forced) {
    if (forced == 256) return 256;
    if (forced == 128 && ok128) return 128;
    if (forced == 64 && ok64) return 64;
    return 0;
  }
  const int64_t rows = (p.M + p.q - 1) / p.q;  // per type (cyclic estimate)
  const int64_t cus = cu_count();
  auto cost = [&](int bm, int bn, double eff) {
    const int64_t tiles = int64_t(p.q) * ((rows + bm - 1) / bm) * (p.N / bn);
    return double((tiles + cus - 1) / cus) * bm * bn / eff;
  };
  int best = 256;
  double c_best = cost(256, r % 256 == 0 ? 256 : (r % 192 == 0 ? 192 : 128), 1.0);
  if (ok128) {
    const double c = cost(128, ok64 ? 256 : (r % 192 == 0 ? 192 : 128), 0.85);
    if (c < c_best) best = 128, c_best = c;
  }
  if (ok64) {
    const double c = cost(64, 256, 0.6);
    if (c < c_best) best = 64, c_best = c;
  }
  return best;
}

hipError_t launch_fwd_persistent_bf16(const ProblemDesc& p, hipStream_t s, int forced_bm) {
  const int64_t r = p.N / p.q;
  const int bm = fwd_tile_height(p, forced_bm);
  if (bm == 64) return launch_fwd<Fwd64x256>(p, s);
  if (bm == 128) {
    if (r % 256 == 0) return launch_fwd<Fwd128x256>(p, s);
    if (r % 192 == 0) return launch_fwd<Fwd128x192>(p, s);
    return launch_fwd<Fwd128x128>(p, s);
  }
  if (bm != 256) return hipErrorInvalidValue;
  if (r % 256 == 0) return launch_fwd<Fwd256x256>(p, s);
  if (r % 192 == 0) return launch_fwd<Fwd256x192>(p, s);
  return launch_fwd<Fwd256x128>(p, s);
}

}  // namespace qalg
