// Persistent matrix-core gradients of the row-typed projection (bf16 in, fp32
// accumulate, bf16 out) for gfx950: the complete law Q_q and the recursive law
// Q_2^(x)L, on any schedule.
//
// Paper: arXiv 2609.32814, appendix B (eq 31-35) and appendix C (eq 36).  For
// the complete law and a row of type i:
//   dx_i = sum_j dy_j W_ij^T,   dx_k = dy_k W_kk^T (k != i)             (eq 31-32)
//   dW_jj += x_j^T dy_j (every row),  dW_ij += x_i^T dy_j (rows of type i)  (eq 33-35)
// Under the recursive law, b feeds output group j of a type-i row when every
// bit of b equals i's or j's; transposed, dX[I_i, g_k] sums over the output
// groups agreeing with k wherever k differs from i, and dW[g_b, g_j] over the
// rows of the types agreeing with b wherever b differs from j.
// Section 5.3: separate gradient kernels with one owner per output element,
// so every dW / dX element is written once and the result does not depend on
// scheduling.
//
// Output tiles are GEMM tiles of BM x BN:
//   dX  tile (256 rows of type i, BN columns of input group k), both operands
//       contraction-contiguous (dY rows; W rows, the transposed weight block
//       read in place).  Contraction: complete law, k == i: all N columns (a
//       "long" tile); k != i: group k's r columns.  Recursive law: the
//       2^(L - |i ^ k|) output groups above, r columns each.
//   dW  tile (BM = 256 or 192 features of group b, BN columns of output group
//       j), both operands row-major over the contraction (token rows of X and
//       dY, read into LDS as is, turned into MFMA fragments by the transposing
//       LDS read).  Contraction: complete law, b == j: every typed row
//       ("long"); b != j: the rows of type b.  Recursive law: the rows of the
//       2^(L - |b ^ j|) types above (all typed rows when b == j).
// Rows of a type: for a cyclic schedule (detected by the index) the
// progression (i - o) mod q + m q in closed form; otherwise the index's row
// list.  dX tiles gather their rows (clamped into the type's rows; extra rows
// are not stored).  dW contractions walk their types' rows 32 per k-step: each
// wave looks up the rows its copies carry (8 with 4 waves, 4 with 8) as
// scalars and copies through a buffer resource, so that the rows past a
// type's last one read as zeros.
//
// Pipeline: one workgroup per CU, operands copied global -> LDS directly; dX
// in two 64-deep stages (contraction-major rows are whole 128-byte lines; the
// publishing barrier after the third of four MFMA quarter steps), dW in four
// 32-deep stages (copies three k-steps ahead; the barrier mid-step); MFMAs
// interleaved one by one with fragment reads (in the order the MFMAs use them)
// and copies, v_mfma_f32_32x32x16_bf16 on wave tiles of BM/2 x BN/2 (4 waves;
// dX with 256-column tiles: 8 waves of BM/2 x BN/4, two per SIMD, 1.4 %
// faster), one RNE rounding, output restaged through LDS into whole pieces.
//
// Work balance.  Tiles fall in classes by contraction length: long and short
// (complete law), or d = |i ^ k| (dX) and d = |b ^ j| (dW) under the
// recursive law, 2^(L - d) segments each.  A dW tile's contraction runs over
// many rows, and there are few dW tiles: each class's tiles are cut into
// `np` pieces of nearly equal k-steps, each writing an fp32 partial tile that
// a reduction sums in piece order and rounds once (bitwise reproducible).  The
// units (tiles or pieces) of each XCD are a contiguous share of every class.
// Complete law: its workgroups are dealt the long units round robin, then the
// workgroups that got one long unit fewer take up to t_long / t_short short
// units each before the rest are dealt round robin.  Recursive law: the
// concatenation of the classes, longest first, round robin.
#include <initializer_list>
#include <type_traits>

#include "qalg.h"
#include "qalg_device.h"
#include "qalg_internal.h"

namespace qalg {

namespace {

using namespace dev;

// Pipeline depth per operation: dX reads both operands contraction-major, so
// 64-deep k-steps make every row copy a whole 128-byte line (two stages);
// dW reads token rows that are whole lines already, and keeps 32-deep
// k-steps in four stages (copies three k-steps ahead), measured faster there.
constexpr int kBKDx = 64, kBKDw = 32;
constexpr int kMaxClasses = 8;  // recursive law: d = 0 .. L, L <= 6

template <int BM_, int BN_, bool A_KM_, bool B_KM_, int BK_, int STAGES_, int NW_ = 4>
struct GradCfg {
  static constexpr int NW = NW_;  // waves: 4 (2 x 2 wave tiles) or 8 (2 x 4)
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  static constexpr int BK = BK_;          // contraction per k-step
  static constexpr int STAGES = STAGES_;  // LDS stages
  static constexpr int Q = BK / 16;       // MFMA quarter steps per k-step
  static_assert((BK == 64 && STAGES == 2) || (BK == 32 && STAGES == 4), "pipeline shapes");
  static constexpr int BM = BM_, BN = BN_, WGM = 2, WGN = NW / 2;
  static constexpr bool A_KM = A_KM_, B_KM = B_KM_;  // contraction-major (else row-major over it)
  static constexpr int THREADS = 64 * NW;
  static constexpr int WTM = BM / WGM, WTN = BN / WGN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0 && FM >= 1 && FN >= 1, "wave tile");
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  static constexpr int KROWB = BK * 2;                    // contraction-major layout: bytes per tile row
  static constexpr int KPC = BK / 8;                      // its 16-byte pieces per row
  static constexpr int A_ROWB = BM * 2, B_ROWB = BN * 2;  // row-major layout: bytes per contraction row
  static constexpr int A_NCH = BM / 8, B_NCH = BN / 8;    // 16-byte pieces per such row
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0, "whole 1 KB copies per wave");
  static constexpr int A_DMA = A_BYTES / (1024 * NW), B_DMA = B_BYTES / (1024 * NW);
  static constexpr int DMA = A_DMA + B_DMA;
  static_assert(STAGES * DMA < 64, "vmcnt range");
  // row-major operands: wave w's copies carry contraction rows RPW w .. RPW w + RPW - 1
  static constexpr int RPW = BK / NW;
  static_assert(A_KM || A_DMA * 64 == RPW * A_NCH, "RPW contraction rows per wave (A)");
  static_assert(B_KM || B_DMA * 64 == RPW * B_NCH, "RPW contraction rows per wave (B)");
  // epilogue: each wave restages 32 rows x WTN columns of bf16 at a time in
  // its own share of a buffer behind the stages
  static constexpr int E_PITCH = WTN * 2;          // bytes per restaged row
  static constexpr int E_NP = WTN / 8;             // 16-byte pieces per row
  static constexpr int E_BYTES = 32 * E_PITCH;
  static constexpr int E_MASK = E_NP == 12 ? 3 : E_NP - 1;  // piece swizzle: p ^ (row & E_MASK)
  static_assert(E_NP % 2 == 0 && (E_NP == 12 || (E_NP & E_MASK) == 0), "epilogue buffer");
  static constexpr int E_OFF = STAGES * STAGE;
  static constexpr int LDS_BYTES = E_OFF + NW * E_BYTES;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// piece swizzle of a contraction-major tile with rows of BK contraction values
template <int BK>
__device__ __forceinline__ int swz_km(int row) { return BK == 64 ? swz_x128(row) : swz_x(row); }

// Row id of the copy slot's contraction row, picked per lane from the R
// wave-uniform ids of the wave's rows: copy u of a row-major operand with NCH
// pieces per row carries rows (64 u + lane) / NCH of the wave's R.
template <int NCH, int R>
__device__ __forceinline__ int pick_row(const int (&o)[R], int u, int lane) {
  const int lo = (64 * u) / NCH, hi = (64 * u + 63) / NCH;
  int v = o[0];
#pragma unroll
  for (int e = 1; e < R; ++e)
    if (e == lo) v = o[e];
#pragma unroll
  for (int e = 1; e < R; ++e)
    if (e > lo && e <= hi) v = lane >= e * NCH - 64 * u ? o[e] : v;
  return v;
}

// offset that fails the buffer range check (resources never exceed 2 GiB)
constexpr uint32_t kNoRow = 0x80000000u;

struct GradArgs {
  const char* A;   // dX: dY;  dW: X
  const char* B;   // dX: W;   dW: dY
  char* C;         // dX: dX;  dW: dW
  const int32_t* ws;
  int64_t off_offsets, off_tiles, off_rows;
  int q, M, K, N, s, r;
  int L;           // recursive law Q_2^(x)L; 0: the complete law
  int cpg;         // dX: column tiles per input group (s / BN); dW: per output group (r / BN)
  int rpb;         // dW: feature tiles per input group (s / BM)
  int np[kMaxClasses];  // dW: pieces per tile of each class (1: not split)
  int t_unit[2];   // dW, complete law: k-steps per unit of a short / long tile
  float* part;     // dW: fp32 partial tiles [piece][K][N] of split tiles
  int64_t part_stride;  // floats per piece (K * N)
  uint32_t a_bytes, b_bytes;  // dW: bytes of X and dY (buffer ranges)
  const uint64_t* adj;  // graph law Q_G: per-type out-edge masks (bit j of type i: edge (i, j)); else null
  // unequal group widths (eq 18), complete law: widths = 1; first K column of
  // input group g, first N column of output group g; first tile along K of
  // input group g (dX: BN-column tiles, n_ct of them in all; dW: BM-row
  // tiles); dW: first BN-column tile along N of output group g, and the first
  // diagonal / off-diagonal tile of group g in the two classes' orders
  int widths, n_ct;
  int gk[kMaxWidthGroups + 1], gn[kMaxWidthGroups + 1], tk[kMaxWidthGroups + 1];
  int tn[kMaxWidthGroups + 1], dpre[kMaxWidthGroups + 1], opre[kMaxWidthGroups + 1];
};

// One unit of work: an output tile, or a piece of a split dW tile.
struct GTile {
  int cls;         // class (complete law: 1 long, 0 short; recursive law: d)
  int type;        // dX: row type
  int out_row0;    // dX: rank of the first row within its type;  dW: first feature
  int first;       // dX: slot of the first row in the index's row list
  int m_cnt;       // dX: valid output rows
  int n0;          // first output column
  int nk;          // k-steps of this unit
  int c0;          // dW: first k-step of this piece within its tile's contraction
  int piece;       // dW: piece of a split tile (fp32 partial output); -1 otherwise
  int seg_from, seg_mask;  // segments: the n-th is law_member(seg_from, seg_mask, n, L)
  int nseg;        // dX: 0 for one contiguous range from col0; dW: segments (0: all typed rows)
  int col0;        // dX: first contraction column of a contiguous range
  uint64_t gmask;  // graph law: the segments' groups (dX) or row types (dW) as a bit set
};

// The u-th unit of a workgroup (slot g of the G on XCD xcd of nx), in closed
// form from a few per-workgroup constants, so that a cursor carries nothing
// but u through the pipeline and a lookup costs a handful of scalar ops.
// Complete law: each XCD takes a contiguous share of the long and of the
// short units; its workgroups take the longs round robin; those left one long
// unit short then take up to t_long / t_short short units each, and the rest
// of the shorts are dealt round robin (k-steps per workgroup end within one
// unit of each other).  cls 1: long, 0: short.
struct Deal2 {
  int lx0, c0, sx0, sx1, g, G, light, lg, G_light, E, base;
  __device__ void init(int n_long, int n_short, int t_long, int t_short, int xcd, int nx, int g_, int G_) {
    g = g_;
    G = G_;
    lx0 = uni(int(int64_t(n_long) * xcd / nx));
    const int lx1 = uni(int(int64_t(n_long) * (xcd + 1) / nx));
    sx0 = uni(int(int64_t(n_short) * xcd / nx));
    sx1 = uni(int(int64_t(n_short) * (xcd + 1) / nx));
    const int nl = lx1 - lx0, ns = sx1 - sx0;
    c0 = uni(g < nl ? (nl - g + G - 1) / G : 0);  // longs of this workgroup
    const int rem = nl % G;
    G_light = rem != 0 ? G - rem : 0;
    const int e = t_short > 0 ? t_long / t_short : 0;
    E = uni(rem != 0 ? min(e, ns / G_light) : 0);
    base = uni(G_light * E);
    light = rem != 0 && g >= rem;
    lg = g - rem;
  }
  template <class A>
  __device__ bool at(const A&, int u, int* cls, int* idx) const {
    if (u < c0) {
      *cls = 1;
      *idx = lx0 + g + u * G;
      return true;
    }
    u -= c0;
    *cls = 0;
    if (light) {
      if (u < E) {
        *idx = sx0 + lg + u * G_light;
        return true;
      }
      u -= E;
    }
    *idx = sx0 + base + g + u * G;
    return *idx < sx1;
  }
};

// Recursive law: each XCD takes a contiguous share of every class; its
// workgroups take the concatenation, class 0 (the longest) first, round robin.
// Class c holds mul * C(L, c) tiles (times np[c] pieces each for dW).
struct DealC {
  int L, mul, xcd, sh, g, G;
  bool pieces;
  template <class A>
  __device__ void init(const A& a, int mul_, bool pieces_, int xcd_, int nx, int g_, int G_) {
    L = a.L;
    mul = mul_;
    pieces = pieces_;
    xcd = xcd_;
    sh = nx == 8 ? 3 : 0;  // shares of 1/nx: nx is 8 or 1
    g = g_;
    G = G_;
  }
  template <class A>
  __device__ bool at(const A& a, int u, int* cls, int* idx) const {
    int p = g + u * G;
    int bn = 1;  // C(L, c)
    for (int c = 0; c <= L; ++c) {
      if (c > 0) bn = bn * (L - c + 1) / c;
      const int T = mul * bn * (pieces ? a.np[c] : 1);
      const int x0 = (T * xcd) >> sh, x1 = (T * (xcd + 1)) >> sh;
      if (p < x1 - x0) {
        *cls = c;
        *idx = x0 + p;
        return true;
      }
      p -= x1 - x0;
    }
    return false;
  }
};

// GRAPH: the graph law Q_G (section 3.1, eq 9-12) with the complete law's
// tiles: a type-i row's dx_i sums over the output groups j of {i} and i's
// out-neighbours (segments of the long tile), its dx_k (k != i) exists only
// for an edge (i, k); dW_jj sums over the rows of j and of j's in-neighbours
// (segments of the diagonal tile), dW_bj (b != j) exists only for an edge
// (b, j).  Tiles of absent edges have no k-steps: the compute cursor writes
// their zeros.
template <class C, Op OP, bool LISTED, bool TENSOR, bool GRAPH>
__device__ __forceinline__ void grad_body(const GradArgs& a, char* smem) {
  const int32_t* ws = a.ws;
  const int32_t* rows = ws + a.off_rows;
  const cint_ptr s_off = to_const(ws + a.off_offsets);
  const cint_ptr s_rows = to_const(rows);
  const int q = a.q;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);

  // the type index: closed form for a cyclic schedule, the tables otherwise
  // (row tiles of 256 rows; dW decodes no row tiles)
  using IX = std::conditional_t<LISTED, MemIndex, CycIndex>;
  IX ix;
  const int cyc = LISTED ? -1 : uni(ws[4]);
  if constexpr (LISTED)
    ix = MemIndex{s_off, to_const(ws + a.off_tiles + tile_height_slot(256) * (q + 1)), q};
  else
    ix = CycIndex::make(q, cyc, a.M, 256);
  // first row of type i in a cyclic schedule
  auto type_start = [&](int i) { return i >= cyc ? i - cyc : i - cyc + q; };
  const int typed = LISTED ? uni(s_off[q]) : a.M;  // rows with a type in range

  // graph law: out-edge mask of type t (two scalar loads)
  auto adj_of = [&](int t) -> uint64_t {
    const cint_ptr e = to_const(reinterpret_cast<const int32_t*>(a.adj));
    return uint64_t(uint32_t(uni(e[2 * t]))) | (uint64_t(uint32_t(uni(e[2 * t + 1]))) << 32);
  };
  // the n-th segment's group (dX) or row type (dW) of unit t
  auto member = [&](const GTile& t, int n) -> int {
    if constexpr (GRAPH) {
      uint64_t m = t.gmask;
      for (int k = 0; k < n; ++k) m &= m - 1;
      return uni(int(__builtin_ctzll(m)));
    } else if constexpr (TENSOR) {
      return law_member(t.seg_from, t.seg_mask, n, a.L);
    } else {
      return t.seg_from;
    }
  };
  // rows of dW segment n of unit t: count, start (cyclic) or list slot, and
  // how rows are found (0: rows 0.. in order; 1: start + m q; 2: row list)
  auto seg_rows = [&](const GTile& t, int n, int& cnt, int& base, int& mode) {
    if (t.nseg == 0) {
      cnt = typed;
      base = 0;
      mode = typed == a.M ? 0 : 2;
      return;
    }
    const int ty = member(t, n);
    cnt = ix.count(ty);
    base = LISTED ? ix.offset(ty) : type_start(ty);
    mode = LISTED ? 2 : 1;
  };

  const int n_rt = OP == Op::Dx ? ix.tiles_before(q) : 0;
  const int tpb = a.rpb * a.cpg;
  auto decode = [&](int cls, int idx) -> GTile {
    GTile t;
    t.cls = cls;
    t.c0 = 0;
    t.piece = -1;
    if constexpr (OP == Op::Dx && !TENSOR && !GRAPH) {
      if (a.widths) {
        // unequal widths: one class, groups of 4 row tiles x all dX column
        // tiles (row tile fastest); column tile c2 lies in input group k; the
        // contraction runs over all N output columns when k is the row type
        // (eq 31-32's long sum), else over output group k alone
        constexpr int G = 4;
        const int span = G * a.n_ct;
        const int grp = idx / span, w = idx - grp * span;
        const int first_rt = grp * G;
        const int gm = min(n_rt - first_rt, G);
        const int rt = first_rt + w % gm, c2 = w / gm;
        const int i = ix.group_of_tile(rt);
        int k = 0;
        while (k + 1 < q && c2 >= a.tk[k + 1]) k = uni(k + 1);
        t.type = i;
        t.out_row0 = (rt - ix.tiles_before(i)) * C::BM;
        t.m_cnt = min(C::BM, ix.count(i) - t.out_row0);
        t.first = ix.offset(i) + t.out_row0;
        t.seg_from = t.seg_mask = 0;
        t.gmask = 0;
        t.nseg = 0;
        t.col0 = k == i ? 0 : a.gn[k];
        t.nk = uni(k == i ? a.N / C::BK : (a.gn[k + 1] - a.gn[k]) / C::BK);
        t.n0 = a.gk[k] + (c2 - a.tk[k]) * C::BN;
        return t;
      }
    }
    if constexpr (OP == Op::Dx) {
      constexpr int G = 4;
      const int ngrp = TENSOR ? binom_small(a.L, cls) : (cls ? 1 : q - 1);
      const int span = G * ngrp * a.cpg;
      const int grp = idx / span, w = idx - grp * span;
      const int first_rt = grp * G;
      const int gm = min(n_rt - first_rt, G);
      const int rt = first_rt + w % gm, c2 = w / gm;
      const int jj = c2 / a.cpg, cc = c2 - jj * a.cpg;
      const int i = ix.group_of_tile(rt);
      t.type = i;
      t.out_row0 = (rt - ix.tiles_before(i)) * C::BM;
      t.m_cnt = min(C::BM, ix.count(i) - t.out_row0);
      t.first = ix.offset(i) + t.out_row0;
      int k;
      const int kts = a.r / C::BK;
      if constexpr (TENSOR) {
        const int m = unrank_mask(jj, cls, a.L);
        k = i ^ m;
        // output groups agreeing with k where k differs from i (all when k == i)
        t.seg_from = k;
        t.seg_mask = m;
        t.nseg = cls > 0 ? 1 << (a.L - cls) : 0;
        t.col0 = 0;
        t.nk = (1 << (a.L - cls)) * kts;
      } else if constexpr (GRAPH) {
        // bits at or past q are not types (ignored, as the forward ignores them)
        const uint64_t valid = q >= 64 ? ~uint64_t(0) : (uint64_t(1) << q) - 1;
        const uint64_t out = adj_of(i) & valid & ~(uint64_t(1) << i);
        k = cls ? i : (jj < i ? jj : jj + 1);
        t.seg_from = i;
        t.seg_mask = 0;
        if (cls) {
          // dx_i: output groups i and the out-neighbours of i
          t.gmask = out | (uint64_t(1) << i);
          t.nseg = uni(__builtin_popcountll(t.gmask));
          t.col0 = 0;
          t.nk = t.nseg * kts;
        } else {
          // dx_k = dy_k W_kk^T only for an edge (i, k)
          t.gmask = 0;
          t.nseg = 0;
          t.col0 = k * a.r;
          t.nk = ((out >> k) & 1) ? kts : 0;
        }
      } else {
        k = cls ? i : (jj < i ? jj : jj + 1);
        t.seg_from = t.seg_mask = 0;
        t.nseg = 0;
        t.col0 = cls ? 0 : k * a.r;
        t.nk = cls ? a.N / C::BK : kts;
      }
      t.n0 = k * a.s + cc * C::BN;
    } else {
      const int npc = a.np[cls];
      const int tix = idx / npc;
      const int piece = idx - tix * npc;
      const int blk = tix / tpb, w = tix - blk * tpb;
      int b, j;
      if constexpr (TENSOR) {
        const int nb = binom_small(a.L, cls);
        b = blk / nb;
        const int m = unrank_mask(blk - b * nb, cls, a.L);
        j = b ^ m;
        // rows of the types agreeing with b where b differs from j
        t.seg_from = b;
        t.seg_mask = m;
        t.nseg = cls > 0 ? 1 << (a.L - cls) : 0;
      } else if (cls) {
        b = j = blk;
        t.seg_from = b;
        t.seg_mask = 0;
        t.nseg = 0;
        if constexpr (GRAPH) {
          // dW_jj: the rows of j and of every type with an edge into j
          uint64_t m = uint64_t(1) << j;
          for (int ty = 0; ty < q; ++ty)
            if ((adj_of(ty) >> j) & 1) m |= uint64_t(1) << ty;
          t.gmask = m;
          t.nseg = uni(__builtin_popcountll(m));
        }
      } else {
        b = blk / (q - 1);
        const int jj = blk - b * (q - 1);
        j = jj < b ? jj : jj + 1;
        t.seg_from = b;
        t.seg_mask = 0;
        t.nseg = 1;
        if constexpr (GRAPH) t.gmask = uint64_t(1) << b;
      }
      if (a.widths) {
        // unequal widths (no split pieces): diagonal tiles of group j in
        // order, feature tile fastest; off-diagonal tiles by input group b,
        // over every column tile outside b's own output group
        int r, c;
        if (cls) {
          int g = 0;
          while (g + 1 < q && idx >= a.dpre[g + 1]) g = uni(g + 1);
          const int local = idx - a.dpre[g];
          const int rpb = a.tk[g + 1] - a.tk[g];
          r = local % rpb;
          c = a.tn[g] + local / rpb;
          b = j = g;
        } else {
          int g = 0;
          while (g + 1 < q && idx >= a.opre[g + 1]) g = uni(g + 1);
          const int local = idx - a.opre[g];
          const int rpb = a.tk[g + 1] - a.tk[g];
          r = local % rpb;
          const int cp = local / rpb;
          c = cp < a.tn[g] ? cp : cp + (a.tn[g + 1] - a.tn[g]);
          int jj = 0;
          while (jj + 1 < q && c >= a.tn[jj + 1]) jj = uni(jj + 1);
          b = g;
          j = jj;
          t.seg_from = b;
        }
        t.out_row0 = a.gk[b] + r * C::BM;
        t.n0 = a.gn[j] + (c - a.tn[j]) * C::BN;
      } else {
        const int rt = w % a.rpb, ct = w / a.rpb;
        t.out_row0 = b * a.s + rt * C::BM;
        t.n0 = j * a.r + ct * C::BN;
      }
      t.type = -1;
      t.first = 0;
      t.m_cnt = C::BM;
      t.col0 = 0;
      // k-steps of the whole contraction: each segment rounded up to whole k-steps
      int nk_all = 0;
      const int ns = t.nseg == 0 ? 1 : t.nseg;
      for (int n = 0; n < ns; ++n) {
        int cnt, base, mode;
        seg_rows(t, n, cnt, base, mode);
        nk_all += (cnt + C::BK - 1) / C::BK;
      }
      if constexpr (GRAPH) {
        // dW_bj (b != j) only for an edge (b, j)
        if (b != j && !((adj_of(b) >> j) & 1)) nk_all = 0;
      }
      const int per = (nk_all + npc - 1) / npc;
      t.c0 = uni(piece * per);
      t.nk = uni(max(0, min(per, nk_all - t.c0)));
      t.piece = npc > 1 ? piece : -1;
    }
    return t;
  };

  // this XCD's units
  const int nx = gridDim.x >= 8 ? 8 : 1;
  const int per_x = gridDim.x / nx;
  const int xcd = blockIdx.x % nx, slot = blockIdx.x / nx;
  // dX rows of an out-of-range type (listed after the typed rows by the
  // index; a cyclic schedule has none) are zero: written here, by every
  // workgroup in turn, instead of by a launch of their own
  if constexpr (OP == Op::Dx && LISTED) {
    const int nbad = a.M - typed;
    const int row_u4 = a.K / 8;  // 16-byte pieces per dX row
    for (int b = blockIdx.x; b < nbad; b += gridDim.x) {
      u32x4* xr = reinterpret_cast<u32x4*>(a.C + int64_t(rows[typed + b]) * a.K * 2);
      for (int x = tid; x < row_u4; x += C::THREADS) xr[x] = (u32x4){0u, 0u, 0u, 0u};
    }
  }
  if (slot >= per_x) return;
  std::conditional_t<TENSOR, DealC, Deal2> deal;
  if constexpr (TENSOR)
    deal.init(a, OP == Op::Dx ? n_rt * a.cpg : q * tpb, OP == Op::Dw, xcd, nx, slot, per_x);
  else if constexpr (OP == Op::Dx) {
    if (a.widths)
      deal.init(n_rt * a.n_ct, 0, a.N / C::BK, 1, xcd, nx, slot, per_x);  // one class, all tiles
    else
      deal.init(n_rt * a.cpg, n_rt * (q - 1) * a.cpg, a.N / C::BK, a.r / C::BK, xcd, nx, slot, per_x);
  }
  else if (a.widths)
    deal.init(a.dpre[q], a.opre[q], a.t_unit[1], a.t_unit[0], xcd, nx, slot, per_x);
  else
    deal.init(q * tpb * a.np[1], q * (q - 1) * tpb * a.np[0], a.t_unit[1], a.t_unit[0], xcd, nx, slot, per_x);
  auto unit_at = [&](int u, int* cls, int* idx) -> bool {
    const bool ok = deal.at(a, u, cls, idx);
    *cls = uni(*cls);
    *idx = uni(*idx);
    return ok;
  };
  // cursors over the units: the copy cursor's next unit, the compute cursor's
  int u_copy = 0, u_comp = 0;
  // the next unit with k-steps (dW pieces and tiles of types without rows
  // can have none: the compute cursor writes their zeros, the copy cursor
  // skips them)
  auto next_work = [&](GTile* t) -> bool {
    for (;;) {
      int cls, idx;
      if (!unit_at(u_copy, &cls, &idx)) return false;
      u_copy = uni(u_copy + 1);
      *t = decode(cls, idx);
      if (t->nk > 0) return true;
    }
  };

  const uint32_t a_ld = uint32_t(OP == Op::Dx ? a.N : a.K) * 2u;   // bytes per row of A
  const uint32_t b_ld = uint32_t(a.N) * 2u;                         // bytes per row of B (W or dY)
  const uint32_t c_ld = uint32_t(OP == Op::Dx ? a.K : a.N) * 2u;    // bytes per row of C

  // per-lane copy slots: KM operand -> (tile row, swizzled piece); RM operand -> (contraction row, piece)
  int a_r[C::A_DMA], a_c[C::A_DMA], b_r[C::B_DMA], b_c[C::B_DMA];
#pragma unroll
  for (int u = 0; u < C::A_DMA; ++u) {
    const int sl = (wid * C::A_DMA + u) * 64 + lane;
    if constexpr (C::A_KM) {
      a_r[u] = sl / C::KPC;
      a_c[u] = (sl % C::KPC) ^ swz_km<C::BK>(sl / C::KPC);
    } else {
      a_r[u] = sl / C::A_NCH;
      a_c[u] = (sl - (sl / C::A_NCH) * C::A_NCH) ^ swz_rm<C::A_ROWB>(sl / C::A_NCH);
    }
  }
#pragma unroll
  for (int u = 0; u < C::B_DMA; ++u) {
    const int sl = (wid * C::B_DMA + u) * 64 + lane;
    if constexpr (C::B_KM) {
      b_r[u] = sl / C::KPC;
      b_c[u] = (sl % C::KPC) ^ swz_km<C::BK>(sl / C::KPC);
    } else {
      b_r[u] = sl / C::B_NCH;
      b_c[u] = (sl - (sl / C::B_NCH) * C::B_NCH) ^ swz_rm<C::B_ROWB>(sl / C::B_NCH);
    }
  }
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>(smem)));
  const u32x4 rs_a = buffer_rsrc(a.A, a.a_bytes), rs_b = buffer_rsrc(a.B, a.b_bytes);

  // ---------------- copy cursor ----------------
  GTile lt;
  bool more = next_work(&lt);  // the copy cursor has not passed the last k-step
  int lk = 0;

  // dX: byte offsets of the lane's A rows (dY rows of the tile's type), and,
  // for a listed schedule, the row ids of the next tile, loaded a tile ahead
  // and taken after the wait that closes a k-step's copies (the wait for them
  // then costs nothing)
  uint32_t a_roff[OP == Op::Dx ? C::A_DMA : 1];
  int pre_row[(OP == Op::Dx && LISTED) ? C::A_DMA : 1];
  bool rows_pending = false;
  GTile nt = lt;   // dX, listed: the unit after lt (its rows prefetched)
  bool have_nt = false;
  auto prefetch_rows = [&](const GTile& t) {
    if constexpr (OP == Op::Dx && LISTED) {
#pragma unroll
      for (int u = 0; u < C::A_DMA; ++u) pre_row[u] = rows[t.first + min(a_r[u], t.m_cnt - 1)];
    }
  };
  auto set_rows = [&](const GTile& t) {
    if constexpr (OP == Op::Dx) {
#pragma unroll
      for (int u = 0; u < C::A_DMA; ++u) {
        int row;
        if constexpr (LISTED)
          row = pre_row[u];
        else
          row = type_start(t.type) + (t.out_row0 + min(a_r[u], t.m_cnt - 1)) * q;
        a_roff[u] = uint32_t(row) * a_ld;
      }
    }
  };
  // dX contraction cursor: column of the current k-step (segment walk for the recursive law)
  int cx_n = 0, cx_kk = 0, cx_col = 0;
  // dW contraction cursor: segment w_n of the unit's contraction covers
  // k-steps [w_k0, w_k0 + w_kn) with w_cnt rows from w_base (mode as seg_rows)
  int w_n = 0, w_k0 = 0, w_kn = 0, w_cnt = 0, w_base = 0, w_mode = 0;
  // dW, cyclic schedule: rows in closed form, row r0 + e st for the wave's
  // row e, with stride st = 1 (all rows in order) or q (the rows of one type);
  // each copy's offset is a per-lane part at that stride (p1, pq, fixed for the
  // kernel) plus a wave-uniform part per k-step
  constexpr bool CYC_DW = OP == Op::Dw && !LISTED;
  // the complete law on a cyclic schedule: one segment per unit, no walk
  constexpr bool SIMPLE = CYC_DW && !TENSOR && !GRAPH;
  uint32_t p1[CYC_DW ? C::DMA : 1], pq[CYC_DW ? C::DMA : 1];
  if constexpr (CYC_DW) {
#pragma unroll
    for (int u = 0; u < C::A_DMA; ++u) {
      const int e = a_r[u] - C::RPW * wid;
      p1[u] = uint32_t(e) * a_ld + uint32_t(a_c[u]) * 16u;
      pq[u] = uint32_t(e * q) * a_ld + uint32_t(a_c[u]) * 16u;
    }
#pragma unroll
    for (int v = 0; v < C::B_DMA; ++v) {
      const int e = b_r[v] - C::RPW * wid;
      p1[C::A_DMA + v] = uint32_t(e) * b_ld + uint32_t(b_c[v]) * 16u;
      pq[C::A_DMA + v] = uint32_t(e * q) * b_ld + uint32_t(b_c[v]) * 16u;
    }
  }
  int w_rbase = 0, w_rstep = 1;  // cyclic: row of the segment's rank j is w_rbase + j w_rstep
  auto seg_enter = [&](int n) {
    w_n = n;
    seg_rows(lt, n, w_cnt, w_base, w_mode);
    w_kn = (w_cnt + C::BK - 1) / C::BK;
    if constexpr (!LISTED) {
      w_rstep = uni(w_mode == 0 ? 1 : q);
      w_rbase = uni(w_mode == 0 ? 0 : w_base);
    }
  };
  auto seg_walk = [&](int kabs) {
    if constexpr (!SIMPLE) {
      const int ns = lt.nseg == 0 ? 1 : lt.nseg;
      while (kabs >= w_k0 + w_kn && w_n + 1 < ns) {
        w_k0 += w_kn;
        seg_enter(w_n + 1);
      }
    }
  };
  // start of a unit: contraction cursors at its first k-step
  auto unit_start = [&]() {
    if constexpr (OP == Op::Dx) {
      cx_n = 0;
      cx_kk = 0;
      cx_col = lt.nseg ? member(lt, 0) * a.r : lt.col0;
    } else if constexpr (!SIMPLE) {
      w_k0 = 0;
      seg_enter(0);
      seg_walk(lt.c0);
    }
  };
  // dW: ids of the RPW rows this wave copies at the cursor's k-step, and how
  // many of them lie inside the segment (w_rem; the others read as zeros)
  int w_id[C::RPW];
  int w_rem = 0;
  uint32_t w_ua = 0, w_ub = 0;  // cyclic: wave-uniform offset parts of the A and B copies
  auto prep_rows = [&]() {
    if constexpr (CYC_DW) {
      // rows past a type's last one (or past M) lie past the end of X and dY:
      // the buffer range check reads them as zeros, no test needed
      int r0;
      if constexpr (SIMPLE) {
        // long units: every row in order; short ones: the rows of type seg_from
        const int j0 = uni((lt.c0 + lk) * C::BK + C::RPW * wid);
        w_rstep = lt.nseg == 0 ? 1 : q;
        r0 = lt.nseg == 0 ? j0 : type_start(lt.seg_from) + j0 * q;
      } else {
        const int j0 = uni((lt.c0 + lk - w_k0) * C::BK + C::RPW * wid);
        r0 = w_rbase + j0 * w_rstep;
      }
      w_ua = uint32_t(uni(int(uint32_t(r0) * a_ld + uint32_t(lt.out_row0) * 2u)));
      w_ub = uint32_t(uni(int(uint32_t(r0) * b_ld + uint32_t(lt.n0) * 2u)));
    } else if constexpr (OP == Op::Dw) {
      const int j0 = (lt.c0 + lk - w_k0) * C::BK + C::RPW * wid;  // segment rank of the wave's first row
      w_rem = uni(w_cnt - j0);
      if (w_mode == 2) {
#pragma unroll
        for (int e = 0; e < C::RPW; ++e) w_id[e] = uni(s_rows[w_base + j0 + e]);  // may read the spare tail
      } else {
        const int r0 = w_mode == 0 ? j0 : w_base + j0 * q, st = w_mode == 0 ? 1 : q;
#pragma unroll
        for (int e = 0; e < C::RPW; ++e) w_id[e] = uni(r0 + e * st);
      }
    }
  };
  // dW: byte offset of a copy's row (local row e of the wave's RPW), or one that
  // fails the range check past the segment's rows
  auto row_off = [&](int id, int e, uint32_t ld, uint32_t col_bytes) -> uint32_t {
    const uint32_t ro = __umul24(uint32_t(id), ld);
    return (e < w_rem ? ro : kNoRow) + col_bytes;
  };
  // dW: source offsets of the wave's copies for the cursor's k-step, worked
  // out in the first quarter step (rows after its first MFMA, offsets in the
  // MFMA slots that carry no fragment read), off the slots that issue the copies
  uint32_t c_off[OP == Op::Dw ? C::DMA : 1];
  auto off_u = [&](int u) {
    if constexpr (CYC_DW) {
      c_off[u] = (w_rstep == 1 ? p1[u] : pq[u]) + (u < C::A_DMA ? w_ua : w_ub);
    } else if constexpr (OP == Op::Dw) {
      if (u < C::A_DMA) {
        c_off[u] = row_off(pick_row<C::A_NCH, C::RPW>(w_id, u, lane), a_r[u] - C::RPW * wid, a_ld,
                           uint32_t(lt.out_row0 + a_c[u] * 8) * 2u);
      } else {
        const int v = u - C::A_DMA;
        c_off[u] = row_off(pick_row<C::B_NCH, C::RPW>(w_id, v, lane), b_r[v] - C::RPW * wid, b_ld,
                           uint32_t(lt.n0 + b_c[v] * 8) * 2u);
      }
    }
  };
  auto copy_u = [&](int stage, int u) {
    const uint32_t S = lds0 + uint32_t(stage * C::STAGE);
    if constexpr (OP == Op::Dx) {
      // A = dY rows of type lt.type (tile rows), B = W rows n0.. (tile rows);
      // contraction columns cx_col..
      if (u < C::A_DMA) {
        copy16_to_lds(a.A, a_roff[u] + uint32_t(cx_col + a_c[u] * 8) * 2u,
                      S + uint32_t((wid * C::A_DMA + u) * 1024));
      } else {
        const int v = u - C::A_DMA;
        copy16_to_lds(a.B, uint32_t(lt.n0 + b_r[v]) * b_ld + uint32_t(cx_col + b_c[v] * 8) * 2u,
                      S + uint32_t(C::A_BYTES + (wid * C::B_DMA + v) * 1024));
      }
    } else {
      // contraction rows of the k-step; output features / columns along the rows
      if (u < C::A_DMA)
        copy16_to_lds_buf(rs_a, c_off[u], S + uint32_t((wid * C::A_DMA + u) * 1024));
      else
        copy16_to_lds_buf(rs_b, c_off[u], S + uint32_t(C::A_BYTES + (wid * C::B_DMA + (u - C::A_DMA)) * 1024));
    }
  };
  // called after the wait that ends a k-step's outstanding copies (and in the
  // prologue): a new dX tile's rows are taken here
  auto prep_copies = [&]() {
    if constexpr (OP == Op::Dx) {
      if (rows_pending) {
        rows_pending = false;
        set_rows(lt);
        if constexpr (LISTED) {
          have_nt = next_work(&nt);
          if (have_nt) prefetch_rows(nt);
        }
      }
    }
  };
  // next k-step of the copy cursor.  After the last k-step the cursor stays
  // on it: the copies issued for the k-steps past the end repeat it into
  // stages that are never read (drained before exit), so that the pipeline
  // needs no conditions.
  auto advance_copies = [&]() {
    if (!more) return;
    lk = uni(lk + 1);
    if (lk < lt.nk) {
      if constexpr (OP == Op::Dx) {
        if (lt.nseg) {
          cx_kk = uni(cx_kk + 1);
          if (cx_kk == a.r / C::BK) {
            cx_kk = 0;
            cx_n = uni(cx_n + 1);
            cx_col = member(lt, cx_n) * a.r;
          } else {
            cx_col = uni(cx_col + C::BK);
          }
        } else {
          cx_col = uni(cx_col + C::BK);
        }
      } else {
        seg_walk(lt.c0 + lk);
      }
    } else {
      bool got;
      GTile t2;
      if constexpr (OP == Op::Dx && LISTED) {
        got = have_nt;
        t2 = nt;
      } else {
        got = next_work(&t2);
      }
      if (got) {
        lt = t2;
        lk = 0;
        unit_start();
        rows_pending = true;
      } else {
        more = false;
        lk = uni(lt.nk - 1);
      }
    }
  };
  auto issue_copies = [&](int stage) {
    prep_copies();
    prep_rows();
#pragma unroll
    for (int u = 0; u < C::DMA; ++u) {
      off_u(u);
      copy_u(stage, u);
    }
    advance_copies();
  };

  // ---------------- fragment reads ----------------
  const int wm = wid / C::WGN, wn = wid % C::WGN;
  const int l32 = lane & 31, lhi = lane >> 5;
  // contraction-major operand: 128-bit read of row l32, piece 2*ks + lhi
  auto km_rd = [&](int w0, int ks) { return (w0 + l32) * C::KROWB + (((2 * ks + lhi) ^ swz_km<C::BK>(l32)) << 4); };
  // contraction-major operands: one offset per quarter step
  int a_rd[C::Q], b_rd[C::Q];
#pragma unroll
  for (int x = 0; x < C::Q; ++x) {
    a_rd[x] = C::A_KM ? km_rd(wm * C::WTM, x) : 0;
    b_rd[x] = C::A_BYTES + (C::B_KM ? km_rd(wn * C::WTN, x) : 0);
  }
  const int am0 = wm * (C::WTM / 32), bm0 = wn * (C::WTN / 32);
  // row-major operands, read with the transposing LDS read: in a 16-lane group
  // (gq = lane / 16, t = lane % 16) lane t reads row 8*(gq/2) + t/4 (+4),
  // columns 16*(gq%2) + 4*(t%4) of the 32-column block; the lane's offset for
  // each of the wave's fragments (block am0 + fm or bm0 + fn, stored as group
  // block ^ s(row); rows 4 and 16 further have the same s)
  int a_rm[C::A_KM ? 1 : C::FM], b_rm[C::B_KM ? 1 : C::FN];
  {
    const int gq = lane >> 4, t = lane & 15;
    const int k_l = 8 * (gq >> 1) + (t >> 2);
    const int r2 = 2 * (gq & 1) + ((t & 3) >> 1);
    if constexpr (!C::A_KM) {
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm)
        a_rm[fm] = k_l * C::A_ROWB + ((((am0 + fm) * 4) ^ swz_rm<C::A_ROWB>(k_l)) + r2) * 16 + 8 * (t & 1);
    }
    if constexpr (!C::B_KM) {
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
        b_rm[fn] = C::A_BYTES + k_l * C::B_ROWB + ((((bm0 + fn) * 4) ^ swz_rm<C::B_ROWB>(k_l)) + r2) * 16 +
                   8 * (t & 1);
    }
  }

  f32x16 acc[C::FM][C::FN];
  bf16x8 fa0[C::FM], fb0[C::FN], fa1[C::FM], fb1[C::FN];
  auto read_a = [&](int stage, int ks, int fm) -> bf16x8 {
    const char* S = smem + stage * C::STAGE;
    if constexpr (C::A_KM) {
      return *reinterpret_cast<const bf16x8*>(S + a_rd[ks] + fm * 32 * C::KROWB);
    } else {
      const char* p = S + a_rm[fm] + 16 * ks * C::A_ROWB;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(p));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(p + 4 * C::A_ROWB));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  auto read_b = [&](int stage, int ks, int fn) -> bf16x8 {
    const char* S = smem + stage * C::STAGE;
    if constexpr (C::B_KM) {
      return *reinterpret_cast<const bf16x8*>(S + b_rd[ks] + fn * 32 * C::KROWB);
    } else {
      const char* p = S + b_rm[fn] + 16 * ks * C::B_ROWB;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(p));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(p + 4 * C::B_ROWB));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  auto load_frags = [&](int stage, int ks, bf16x8 (&fa)[C::FM], bf16x8 (&fb)[C::FN]) {
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) fa[fm] = read_a(stage, ks, fm);
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) fb[fn] = read_b(stage, ks, fn);
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

  // ---------------- pipeline (as in the forward) ----------------
  static_assert(C::FM + C::FN <= C::FM * C::FN, "fragment reads fit a quarter step");
  constexpr int S = C::STAGES;
  if (more) {
    unit_start();
    if constexpr (OP == Op::Dx) {
      // the first unit's rows are taken by the first prep_copies (which also
      // finds the unit after it and prefetches its rows)
      prefetch_rows(lt);
      rows_pending = true;
    }
#pragma unroll
    for (int st = 0; st < S - 1 + (S == 2 ? 1 : 0); ++st) issue_copies(st);
    // two stages: step 1 may be in flight; four: steps 1 and 2
    wait_vmcnt<(S == 2 ? 1 : 2) * C::DMA>();
    lds_barrier();
    load_frags(0, 0, fa0, fb0);
  }

  int stage = 0;  // LDS stage of the current k-step
  // one quarter step: MFMAs on fragments (fa, fb) of quarter ks, each followed
  // by one read of quarter ks + 1's fragments into (ga, gb)
  auto quarter = [&](int ks, const bf16x8 (&fa)[C::FM], const bf16x8 (&fb)[C::FN], bf16x8 (&ga)[C::FM],
                     bf16x8 (&gb)[C::FN]) {
    // dW, first quarter: the slots past the reads work out the copy offsets
    constexpr int R = C::FM + C::FN, F = C::FM * C::FN - R;
    static_assert(OP != Op::Dw || F >= 1, "a free slot for the copy offsets");
#pragma unroll
    for (int x = 0; x < C::FM * C::FN; ++x) {
      const int fm = x / C::FN, fn = x % C::FN;
      acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[fn], fa[fm], acc[fm][fn], 0, 0, 0);
      if (x < R) read_slot(x, stage, ks + 1, ga, gb);
      if (OP == Op::Dw && ks == 0 && x == 0) prep_rows();
      if (OP == Op::Dw && ks == 0 && x >= R) {
        const int f = x - R;
#pragma unroll
        for (int u = f * C::DMA / (F > 0 ? F : 1); u < (f + 1) * C::DMA / (F > 0 ? F : 1); ++u) off_u(u);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // last quarter: MFMAs on fragments 1 interleaved with the reads of the next
  // k-step's first fragments from stage nstage (stale past the last k-step,
  // never used) and the copies into stage cstage.  With two stages the copies
  // start with the reads (one of each per MFMA); with four they follow the
  // reads.  Narrow tiles have fewer MFMAs than reads and copies, the slots
  // past the last MFMA carry the rest.
  auto last_quarter = [&](int nstage, int cstage) {
    constexpr int R = C::FM + C::FN;
    constexpr int C0 = S == 2 ? 0 : R;  // slot of the first copy
    constexpr int kSlots = C::FM * C::FN > C0 + C::DMA ? C::FM * C::FN : C0 + C::DMA;
#pragma unroll
    for (int x = 0; x < kSlots; ++x) {
      if (x < C::FM * C::FN) {
        const int fm = x / C::FN, fn = x % C::FN;
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb1[fn], fa1[fm], acc[fm][fn], 0, 0, 0);
      }
      if (x < R) read_slot(x, nstage, 0, fa0, fb0);
      if (x >= C0 && x - C0 < C::DMA) copy_u(cstage, x - C0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (;;) {
    int c_cls, c_idx;
    if (!unit_at(u_comp, &c_cls, &c_idx)) break;
    u_comp = uni(u_comp + 1);
    const GTile ct = decode(c_cls, c_idx);
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) acc[fm][fn] = (f32x16){};

    for (int ck = 0; ck < ct.nk; ++ck) {
      if constexpr (S == 2) {
        // 64-deep k-step: the barrier after the third quarter publishes the
        // next stage (the only copies in flight) and frees this one, which the
        // last quarter refills with the k-step after next
        quarter(0, fa0, fb0, fa1, fb1);
        quarter(1, fa1, fb1, fa0, fb0);
        quarter(2, fa0, fb0, fa1, fb1);
        wait_vmcnt<0>();
        lds_barrier();
        prep_copies();
        last_quarter(stage ^ 1, stage);
        stage = uni(stage ^ 1);
      } else {
        // 32-deep k-step: the barrier in the middle publishes the next stage
        // (at most the copies of the k-step after it still in flight); the
        // second half refills the stage consumed by the previous k-step
        quarter(0, fa0, fb0, fa1, fb1);
        wait_vmcnt<C::DMA>();
        lds_barrier();
        prep_copies();
        const int nstage = (stage + 1) & 3;
        last_quarter(nstage, (stage + 3) & 3);
        stage = uni(nstage);
      }
      advance_copies();
    }

    bool partial = false;
    if constexpr (OP == Op::Dw) partial = ct.piece >= 0;
    if (partial) {
      // a piece of a split tile: its fp32 sums go to the piece's partial tile
      // (lane (l32, lhi) holds 4 consecutive columns of one row per group gg,
      // i.e. one 16-byte piece); the reduction rounds them
      float* P = a.part + size_t(ct.piece) * size_t(a.part_stride);
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm) {
        const size_t row = size_t(ct.out_row0 + wm * C::WTM + fm * 32 + l32);
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) {
#pragma unroll
          for (int gg = 0; gg < 4; ++gg) {
            const f32x16& v = acc[fm][fn];
            const int col = ct.n0 + wn * C::WTN + fn * 32 + gg * 8 + lhi * 4;
            const u32x4 val = {__float_as_uint(v[4 * gg]), __float_as_uint(v[4 * gg + 1]),
                               __float_as_uint(v[4 * gg + 2]), __float_as_uint(v[4 * gg + 3])};
            *reinterpret_cast<u32x4*>(P + row * size_t(a.N) + size_t(col)) = val;
          }
        }
      }
    } else {
      // epilogue: one rounding of each fp32 sum, restaged through the wave's
      // share of the LDS behind the stages so that each store instruction
      // writes whole 16-byte pieces of a few rows
      char* ebuf = smem + C::E_OFF + wid * C::E_BYTES;
      const uint32_t col0 = uint32_t(ct.n0 + wn * C::WTN) * 2u;
      const int ostart = (OP == Op::Dx && !LISTED) ? type_start(ct.type) : 0;
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm) {
        // lane (l32, lhi) holds row l32, columns fn*32 + g*8 + lhi*4 .. +3
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) {
#pragma unroll
          for (int gg = 0; gg < 4; ++gg) {
            const f32x16& v = acc[fm][fn];
            const int pc = (fn * 4 + gg) ^ (l32 & C::E_MASK);
            *reinterpret_cast<u32x2*>(ebuf + l32 * C::E_PITCH + pc * 16 + lhi * 8) =
                pack4_bf16(v[4 * gg], v[4 * gg + 1], v[4 * gg + 2], v[4 * gg + 3]);
          }
        }
        // read back: 64 lanes take 64 consecutive (row, piece) slots per instruction
#pragma unroll
        for (int it = 0; it < C::E_NP / 2; ++it) {
          const int sl = it * 64 + lane;
          const int row = sl / C::E_NP, pc = sl - row * C::E_NP;
          const u32x4 val = *reinterpret_cast<const u32x4*>(ebuf + row * C::E_PITCH + ((pc ^ (row & C::E_MASK)) << 4));
          const int ml = wm * C::WTM + fm * 32 + row;
          // non-temporal whole-line stores keep the output out of L2 (as in the forward)
          if (ml < ct.m_cnt) {
            int orow;
            if constexpr (OP == Op::Dx)
              orow = LISTED ? rows[ct.first + ml] : ostart + (ct.out_row0 + ml) * q;
            else
              orow = ct.out_row0 + ml;
            __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(a.C + (uint32_t(orow) * c_ld + col0 + uint32_t(pc) * 16u)));
          }
        }
      }
    }
  }
  // the repeated copies past the last k-step land in LDS: drain them before
  // the workgroup's LDS can be handed to another workgroup
  wait_vmcnt<0>();
}

template <class C, Op OP, bool TENSOR, bool GRAPH>
__global__ __launch_bounds__(C::THREADS, 1) void grad_persistent_kernel(GradArgs a) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int32_t* ws = a.ws;
  if (ws[1] != kIndexMagic || ws[2] != a.q || ws[3] != a.M) return;
  // two bodies: the cyclic one never reads the row list
  if (ws[4] >= 0)
    grad_body<C, OP, false, TENSOR, GRAPH>(a, smem);
  else
    grad_body<C, OP, true, TENSOR, GRAPH>(a, smem);
}

// dW of split tiles: dW = bf16(sum over pieces of the fp32 partial tiles),
// pieces in order, one rounding.  Workgroups cover the blocks (b, j) of the
// split classes in class order, wpb workgroups of 1024 elements per block.
struct ReduceArgs {
  const int32_t* ws;
  int q, M, L;
  const float* part;
  int64_t stride;  // floats per piece
  int N, s, r, wpb;
  int np[kMaxClasses];
  int first[kMaxClasses + 1];  // first workgroup of each class (classes not split have none)
  uint16_t* dW;
};

__global__ __launch_bounds__(256) void dw_piece_reduce_kernel(ReduceArgs a) {
  const int32_t* ws = a.ws;
  if (ws[1] != kIndexMagic || ws[2] != a.q || ws[3] != a.M) return;
  const int bid = blockIdx.x;
  int c = 0;
  while (c + 1 < kMaxClasses && bid >= a.first[c + 1]) ++c;
  const int local = bid - a.first[c];
  const int blk = local / a.wpb, w = local - blk * a.wpb;
  int b, j;
  if (a.L > 0) {
    const int nb = binom_small(a.L, c);
    b = blk / nb;
    j = b ^ unrank_mask(blk - b * nb, c, a.L);
  } else if (c == 1) {
    b = j = blk;
  } else {
    b = blk / (a.q - 1);
    const int jj = blk - b * (a.q - 1);
    j = jj < b ? jj : jj + 1;
  }
  const int64_t e = (int64_t(w) * 256 + threadIdx.x) * 4;
  if (e >= int64_t(a.s) * a.r) return;
  const int64_t f = e / a.r, cc = e - f * a.r;
  const int64_t off = (int64_t(b) * a.s + f) * a.N + int64_t(j) * a.r + cc;
  u32x4 x = *reinterpret_cast<const u32x4*>(a.part + off);
  float v0 = __uint_as_float(x[0]), v1 = __uint_as_float(x[1]), v2 = __uint_as_float(x[2]), v3 = __uint_as_float(x[3]);
  for (int p = 1; p < a.np[c]; ++p) {
    x = *reinterpret_cast<const u32x4*>(a.part + p * a.stride + off);
    v0 += __uint_as_float(x[0]);
    v1 += __uint_as_float(x[1]);
    v2 += __uint_as_float(x[2]);
    v3 += __uint_as_float(x[3]);
  }
  *reinterpret_cast<u32x2*>(a.dW + off) = pack4_bf16(v0, v1, v2, v3);
}

template <int BN>
using DxCfg = GradCfg<256, BN, true, true, kBKDx, 2, BN == 256 ? 8 : 4>;
template <int BM, int BN>
using DwCfg = GradCfg<BM, BN, false, false, kBKDw, 4, BM == 256 && BN == 256 ? 8 : 4>;

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

int binom_host(int L, int d) {
  int c = 1;
  for (int k = 0; k < d; ++k) c = c * (L - k) / (k + 1);
  return c;
}

int tensor_levels_of(int q) {
  int L = 0;
  while ((1 << L) < q) ++L;
  return L;
}

template <class C, Op OP, bool TENSOR, bool GRAPH>
hipError_t launch_grad(const ProblemDesc& p, hipStream_t s) {
  static bool attr_set = false;
  const int lds = C::LDS_BYTES;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&grad_persistent_kernel<C, OP, TENSOR, GRAPH>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  GradArgs a{};
  a.A = static_cast<const char*>(p.A);
  a.B = static_cast<const char*>(p.B);
  a.C = static_cast<char*>(p.C);
  a.ws = p.ws;
  const WsLayout Lw = ws_layout(p.q, p.M);
  a.off_offsets = Lw.offsets;
  a.off_tiles = Lw.tile_off;
  a.off_rows = Lw.rows;
  a.q = p.q;
  a.M = int(p.M);
  a.K = int(p.K);
  a.N = int(p.N);
  a.s = int(p.K / p.q);
  a.r = int(p.N / p.q);
  a.L = TENSOR ? tensor_levels_of(p.q) : 0;
  a.adj = GRAPH ? p.graph_adj : nullptr;
  a.a_bytes = uint32_t(p.M * p.K * 2);
  a.b_bytes = uint32_t(p.M * p.N * 2);
  if (OP == Op::Dx) {
    a.cpg = a.s / C::BN;
    a.rpb = 0;
    if (p.in_widths != nullptr) {
      a.widths = 1;
      a.gk[0] = a.gn[0] = a.tk[0] = 0;
      for (int g = 0; g < p.q; ++g) {
        a.gk[g + 1] = a.gk[g] + int(p.in_widths[g]);
        a.gn[g + 1] = a.gn[g] + int(p.out_widths[g]);
        a.tk[g + 1] = a.tk[g] + int(p.in_widths[g] / C::BN);
      }
      a.n_ct = a.tk[p.q];
      a.cpg = 0;
    }
  } else {
    a.cpg = a.r / C::BN;
    a.rpb = a.s / C::BM;
    if (p.in_widths != nullptr) {
      a.widths = 1;
      a.gk[0] = a.gn[0] = a.tk[0] = a.tn[0] = 0;
      for (int g = 0; g < p.q; ++g) {
        a.gk[g + 1] = a.gk[g] + int(p.in_widths[g]);
        a.gn[g + 1] = a.gn[g] + int(p.out_widths[g]);
        a.tk[g + 1] = a.tk[g] + int(p.in_widths[g] / C::BM);
        a.tn[g + 1] = a.tn[g] + int(p.out_widths[g] / C::BN);
      }
      a.dpre[0] = a.opre[0] = 0;
      for (int g = 0; g < p.q; ++g) {
        const int rpb = a.tk[g + 1] - a.tk[g], cpg = a.tn[g + 1] - a.tn[g];
        a.dpre[g + 1] = a.dpre[g] + rpb * cpg;
        a.opre[g + 1] = a.opre[g] + rpb * (a.tn[p.q] - cpg);
      }
      a.cpg = a.rpb = 1;  // unused by the widths decode; keeps its divisions defined
    }
  }
  int grid = cu_count();
  grid = grid >= 8 ? grid / 8 * 8 : grid;
  for (int c = 0; c < kMaxClasses; ++c) a.np[c] = 1;
  a.t_unit[0] = a.t_unit[1] = 1;
  a.part = nullptr;
  a.part_stride = 0;
  int ncls = 0;
  int64_t nblk[kMaxClasses] = {};  // dW blocks of each class
  if (OP == Op::Dw) {
    // contraction k-steps of each class's tiles, from M / q rows per type
    const int64_t kd = C::BK;
    const int64_t per_type = (p.M + p.q - 1) / p.q;
    int64_t nk[kMaxClasses] = {};
    if (TENSOR) {
      ncls = a.L + 1;
      for (int d = 0; d <= a.L; ++d) {
        nblk[d] = int64_t(p.q) * binom_host(a.L, d);
        nk[d] = d == 0 ? (p.M + kd - 1) / kd : (int64_t(1) << (a.L - d)) * ((per_type + kd - 1) / kd);
      }
    } else {
      ncls = 2;
      nblk[1] = p.q;
      nblk[0] = int64_t(p.q) * (p.q - 1);
      nk[1] = (p.M + kd - 1) / kd;
      nk[0] = (per_type + kd - 1) / kd;
    }
    const int64_t tpb = int64_t(a.rpb) * a.cpg;
    int64_t total = 0;
    for (int c = 0; c < ncls; ++c) total += nblk[c] * tpb * nk[c];
    const int64_t avg = (total + grid - 1) / grid;
    if (p.dw_part != nullptr && p.in_widths == nullptr) {
      // cut a class's tiles until a piece is no longer than the average
      // k-steps per workgroup (powers of two, at most kDwMaxSplits pieces)
      for (int c = 0; c < ncls; ++c) {
        int sp = 1;
        while (sp * 2 <= kDwMaxSplits && (nk[c] + sp - 1) / sp > avg && nk[c] / (sp * 2) >= 1) sp *= 2;
        a.np[c] = sp;
      }
      a.part = static_cast<float*>(p.dw_part);
      a.part_stride = p.K * p.N;
    }
    if (!TENSOR) {
      a.t_unit[0] = int((nk[0] + a.np[0] - 1) / a.np[0]);
      a.t_unit[1] = int((nk[1] + a.np[1] - 1) / a.np[1]);
    }
  }
  const size_t shm = C::LDS_BYTES;
  hipLaunchKernelGGL((grad_persistent_kernel<C, OP, TENSOR, GRAPH>), dim3(grid), dim3(C::THREADS), shm, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || OP != Op::Dw) return e;
  // reduce the split classes
  ReduceArgs ra{};
  ra.ws = p.ws;
  ra.q = a.q;
  ra.M = a.M;
  ra.L = a.L;
  ra.part = a.part;
  ra.stride = a.part_stride;
  ra.N = a.N;
  ra.s = a.s;
  ra.r = a.r;
  ra.wpb = int((int64_t(a.s) * a.r / 4 + 255) / 256);
  ra.dW = static_cast<uint16_t*>(p.C);
  int64_t wgs = 0;
  for (int c = 0; c < kMaxClasses; ++c) {
    ra.np[c] = a.np[c];
    ra.first[c] = int(wgs);
    if (c < ncls && a.np[c] > 1) wgs += nblk[c] * ra.wpb;
  }
  ra.first[kMaxClasses] = int(wgs);
  if (wgs == 0) return hipSuccess;
  hipLaunchKernelGGL(dw_piece_reduce_kernel, dim3(unsigned(wgs)), dim3(256), 0, s, ra);
  return hipGetLastError();
}

int pick_bn(int64_t w) { return w % 256 == 0 ? 256 : w % 192 == 0 ? 192 : w % 128 == 0 ? 128 : 0; }
int pick_bm_dw(int64_t w) { return w % 256 == 0 ? 256 : w % 192 == 0 ? 192 : 0; }
// the widest tile extent (of those offered) that divides every group width
int pick_widths(const int64_t* w, int q, std::initializer_list<int> sizes) {
  for (const int t : sizes) {
    bool ok = true;
    for (int g = 0; g < q; ++g) ok = ok && w[g] % t == 0;
    if (ok) return t;
  }
  return 0;
}
int pick_bn_widths(const ProblemDesc& p) { return pick_widths(p.in_widths, p.q, {256, 192, 128}); }

template <Op OP, bool TENSOR, bool GRAPH>
hipError_t launch_op(const ProblemDesc& p, hipStream_t s) {
  if (OP == Op::Dx) {
    const int bn = p.in_widths != nullptr ? pick_bn_widths(p) : pick_bn(p.K / p.q);
    if (bn == 256) return launch_grad<DxCfg<256>, Op::Dx, TENSOR, GRAPH>(p, s);
    if (bn == 192) return launch_grad<DxCfg<192>, Op::Dx, TENSOR, GRAPH>(p, s);
    return launch_grad<DxCfg<128>, Op::Dx, TENSOR, GRAPH>(p, s);
  }
  const int bm = p.in_widths != nullptr ? pick_widths(p.in_widths, p.q, {256, 192}) : pick_bm_dw(p.K / p.q);
  const int bn = p.in_widths != nullptr ? pick_widths(p.out_widths, p.q, {256, 192, 128}) : pick_bn(p.N / p.q);
  if (bm == 256) {
    if (bn == 256) return launch_grad<DwCfg<256, 256>, Op::Dw, TENSOR, GRAPH>(p, s);
    if (bn == 192) return launch_grad<DwCfg<256, 192>, Op::Dw, TENSOR, GRAPH>(p, s);
    return launch_grad<DwCfg<256, 128>, Op::Dw, TENSOR, GRAPH>(p, s);
  }
  if (bn == 256) return launch_grad<DwCfg<192, 256>, Op::Dw, TENSOR, GRAPH>(p, s);
  if (bn == 192) return launch_grad<DwCfg<192, 192>, Op::Dw, TENSOR, GRAPH>(p, s);
  return launch_grad<DwCfg<192, 128>, Op::Dw, TENSOR, GRAPH>(p, s);
}

}  // namespace

bool grad_persistent_supported(const ProblemDesc& p) {
  if (p.E != 1 || (p.op != Op::Dx && p.op != Op::Dw)) return false;
  if (p.in_widths != nullptr) {
    // unequal widths (complete law).  dX: input groups in whole column tiles,
    // output groups in whole 64-deep k-steps, 256-row tiles; dW: input groups
    // in whole 256- or 192-row tiles, output groups in whole column tiles
    if (p.law_L != 0 || p.graph_adj != nullptr || p.q > kMaxWidthGroups) return false;
    const int64_t lim = int64_t(1) << 30;
    if (p.M * p.K >= lim || p.K * p.N >= lim || p.M * p.N >= lim) return false;
    if (p.op == Op::Dw)
      return pick_widths(p.in_widths, p.q, {256, 192}) != 0 && pick_widths(p.out_widths, p.q, {256, 192, 128}) != 0 &&
             p.M >= int64_t(kBKDw) * p.q;
    for (int g = 0; g < p.q; ++g)
      if (p.out_widths[g] % kBKDx != 0) return false;
    return (p.M + p.q - 1) / p.q >= 128 && pick_bn_widths(p) != 0;
  }
  if (p.law_L > 6) return false;
  if (p.graph_adj != nullptr && (p.law_L > 0 || p.q > 64)) return false;  // one 64-bit mask per type
  const int64_t s = p.K / p.q, r = p.N / p.q;
  // 32-bit offsets; dW's buffer ranges stay below 2 GiB
  const int64_t lim = int64_t(1) << 30;
  if (p.M * p.K >= lim || p.K * p.N >= lim || p.M * p.N >= lim) return false;
  if (p.op == Op::Dx) {
    // rows of a type in 256-row tiles; columns of an input group in BN tiles;
    // contraction lengths N and r in whole k-steps
    return (p.M + p.q - 1) / p.q >= 128 && pick_bn(s) != 0 && r % kBKDx == 0;
  }
  // features of a group in 256- or 192-row tiles, output group columns in BN
  // tiles; rows in 32-row k-steps (a type's last k-step reads zeros past its rows)
  return pick_bm_dw(s) != 0 && pick_bn(r) != 0 && p.M >= int64_t(kBKDw) * p.q;
}

hipError_t launch_grad_persistent_bf16(const ProblemDesc& p, hipStream_t s) {
  if (p.graph_adj != nullptr)
    return p.op == Op::Dx ? launch_op<Op::Dx, false, true>(p, s) : launch_op<Op::Dw, false, true>(p, s);
  if (p.op == Op::Dx) return p.law_L > 0 ? launch_op<Op::Dx, true, false>(p, s) : launch_op<Op::Dx, false, false>(p, s);
  return p.law_L > 0 ? launch_op<Op::Dw, true, false>(p, s) : launch_op<Op::Dw, false, false>(p, s);
}

}  // namespace qalg
