// Persistent matrix-core gradients of the row-typed Q_q projection (bf16 in,
// fp32 accumulate, bf16 out) for gfx950, cyclic schedules.
//
// Paper: arXiv 2609.32814, appendix B (eq 31-35).  For a row of type i:
//   dx_i = sum_j dy_j W_ij^T,   dx_k = dy_k W_kk^T (k != i)             (eq 31-32)
//   dW_jj += x_j^T dy_j (every row),  dW_ij += x_i^T dy_j (rows of type i)  (eq 33-35)
// Section 5.3: separate gradient kernels with one owner per output element,
// so every dW / dX element is written once and the result does not depend on
// scheduling.
//
// Output tiles are GEMM tiles of 256 x BN (BN = 256, 192 or 128):
//   dX  tile (256 rows of type i, BN columns of input group k):
//         k == i: dY[rows, :] W[cols, :]^T     (contraction N: a "long" tile)
//         k != i: dY[rows, g_k] W[cols, g_k]^T (contraction r)
//   dW  tile (256 features of group b, BN columns of output group j):
//         b == j: X[:, f]^T dY[:, cols] over all M rows   ("long")
//         b != j: the same over the rows of type b         (M / q rows)
// The dX operands are both contraction-contiguous (dY rows; W rows, i.e. the
// transpose of the weight block is read in place); the dW operands are both
// row-major over the contraction (token rows of X and dY), read into LDS as is
// and turned into MFMA fragments with the transposing LDS read.
//
// Pipeline (as in the forward): one workgroup per CU, operands copied
// global -> LDS directly (global_load_lds_dwordx4); dX in two 64-deep stages
// (contraction-major rows are whole 128-byte lines; the publishing barrier
// after the third of four MFMA quarter steps), dW in four 32-deep stages
// (copies three k-steps ahead; the barrier mid-step); MFMAs interleaved one by one with fragment reads (in the
// order the MFMAs use them) and copies, v_mfma_f32_32x32x16_bf16 on 128x128
// wave tiles, one RNE rounding, output restaged through LDS into whole pieces.
//
// Work balance.  Long tiles carry q times the contraction of short ones.  The
// tiles of each XCD (a contiguous share of the long and of the short tiles)
// are dealt to its workgroups round robin, longs first; workgroups that got
// one long tile fewer then take up to q short tiles each before the remaining
// short tiles are dealt round robin, so every workgroup ends with nearly the
// same number of k-steps.  A dW long tile (a diagonal block, contracted over
// all M rows) can still exceed the average load of a workgroup by far (at
// q = 8: 512 k-steps against an average of 360); given fp32 scratch, its
// contraction is cut into `splits` equal pieces dealt as separate long tiles,
// each writing an fp32 partial tile, and a reduction sums the pieces in order
// and rounds once (bitwise reproducible).
//
// Rows of type i are the arithmetic progression (i - o) mod q + k q of a
// cyclic schedule (detected by the index); a launch on any other schedule
// returns at once and the register-staged gradient kernels run instead.
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

template <int BM_, int BN_, bool A_KM_, bool B_KM_, int BK_, int STAGES_>
struct GradCfg {
  static constexpr int BK = BK_;          // contraction per k-step
  static constexpr int STAGES = STAGES_;  // LDS stages
  static constexpr int Q = BK / 16;       // MFMA quarter steps per k-step
  static_assert((BK == 64 && STAGES == 2) || (BK == 32 && STAGES == 4), "pipeline shapes");
  static constexpr int BM = BM_, BN = BN_, WGM = 2, WGN = 2;
  static constexpr bool A_KM = A_KM_, B_KM = B_KM_;  // contraction-major (else row-major over it)
  static constexpr int THREADS = 256;
  static constexpr int WTM = BM / WGM, WTN = BN / WGN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0 && FM >= 1 && FN >= 1, "wave tile");
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  static constexpr int KROWB = BK * 2;                    // contraction-major layout: bytes per tile row
  static constexpr int KPC = BK / 8;                      // its 16-byte pieces per row
  static constexpr int A_ROWB = BM * 2, B_ROWB = BN * 2;  // row-major layout: bytes per contraction row
  static constexpr int A_NCH = BM / 8, B_NCH = BN / 8;    // 16-byte pieces per such row
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static_assert(A_BYTES % 4096 == 0 && B_BYTES % 4096 == 0, "whole 1 KB copies per wave");
  static constexpr int A_DMA = A_BYTES / 4096, B_DMA = B_BYTES / 4096;
  static constexpr int DMA = A_DMA + B_DMA;
  static_assert(STAGES * DMA < 64, "vmcnt range");
  // epilogue: each wave restages 32 rows x WTN columns of bf16 at a time in
  // its own share of a buffer behind the stages
  static constexpr int E_PITCH = WTN * 2;          // bytes per restaged row
  static constexpr int E_NP = WTN / 8;             // 16-byte pieces per row
  static constexpr int E_BYTES = 32 * E_PITCH;
  static constexpr int E_MASK = E_NP == 12 ? 3 : E_NP - 1;  // piece swizzle: p ^ (row & E_MASK)
  static_assert(E_NP % 2 == 0 && (E_NP == 12 || (E_NP & E_MASK) == 0), "epilogue buffer");
  static constexpr int E_OFF = STAGES * STAGE;
  static constexpr int LDS_BYTES = E_OFF + 4 * E_BYTES;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// piece swizzle of a contraction-major tile with rows of BK contraction values
template <int BK>
__device__ __forceinline__ int swz_km(int row) { return BK == 64 ? swz_x128(row) : swz_x(row); }

struct GradArgs {
  const char* A;   // dX: dY;  dW: X
  const char* B;   // dX: W;   dW: dY
  char* C;         // dX: dX;  dW: dW
  const int32_t* ws;
  int64_t off_offsets, off_tiles;
  int q, M, K, N, s, r;
  int n_rt;        // dX: row tiles over all types (from the index; read on device)
  int cpg;         // dX: column tiles per input group (s / BN); dW: per output group (r / BN)
  int rpb;         // dW: row tiles per feature group (s / BM)
  int splits;      // dW: pieces of each long tile's contraction (1: none)
  float* part;     // dW, splits > 1: fp32 partial tiles [splits][K][N] (diagonal blocks only)
  int64_t part_stride;  // floats per piece (K * N)
};

// One output tile.
struct GTile {
  int out_row0;    // dX: rank of the first row within its type;  dW: first feature
  int type;        // dX: row type;  dW: type whose rows are contracted (-1: all rows)
  int m_cnt;       // valid output rows (dX ragged row tiles)
  int n0;          // first output column
  int c0;          // dX: first contraction column (in N);  dW: first k-step of a split piece
  int nk;          // k-steps
  int piece;       // dW: piece of a split long tile (fp32 partial output); -1 otherwise
};


// Tile decode.  dX long tiles: (row tile, column tile of the row's own group);
// short: (row tile, other group, column tile); both in groups of 4 row tiles
// by all columns, row tile fastest.  dW long tiles: (block b == j, row tile,
// column tile); short: (b, j != b, row tile, column tile), b slowest.
template <class C, Op OP>
__device__ __forceinline__ GTile decode(const GradArgs& a, const CycIndex& ix, bool is_long, int idx) {
  GTile t;
  if constexpr (OP == Op::Dx) {
    constexpr int G = 4;
    const int ncol = is_long ? a.cpg : (a.q - 1) * a.cpg;
    const int span = G * ncol;
    const int grp = idx / span, w = idx - grp * span;
    const int first_rt = grp * G;
    const int gm = min(a.n_rt - first_rt, G);
    const int rt = first_rt + w % gm, ct = w / gm;
    const int i = ix.group_of_tile(rt);
    t.type = i;
    t.out_row0 = (rt - ix.tiles_before(i)) * C::BM;
    t.m_cnt = min(C::BM, ix.count(i) - t.out_row0);
    int k, cc;
    if (is_long) {
      k = i;
      cc = ct;
    } else {
      const int kk = ct / a.cpg;
      cc = ct - kk * a.cpg;
      k = kk < i ? kk : kk + 1;
    }
    t.n0 = k * a.s + cc * C::BN;
    t.c0 = is_long ? 0 : k * a.r;
    t.piece = -1;
    t.nk = uni((is_long ? a.N : a.r) / C::BK);
  } else {
    const int tpb = a.rpb * a.cpg;
    // split long tiles: consecutive indices are the pieces of one tile
    int piece = -1;
    if (is_long && a.splits > 1) {
      const int tix = idx / a.splits;
      piece = idx - tix * a.splits;
      idx = tix;
    }
    const int blk = idx / tpb, w = idx - blk * tpb;
    int b, j;
    if (is_long) {
      b = j = blk;
    } else {
      b = blk / (a.q - 1);
      const int jj = blk - b * (a.q - 1);
      j = jj < b ? jj : jj + 1;
    }
    const int rt = w % a.rpb, ct = w / a.rpb;
    t.out_row0 = b * a.s + rt * C::BM;
    t.m_cnt = C::BM;
    t.n0 = j * a.r + ct * C::BN;
    t.type = is_long ? -1 : b;
    t.nk = uni((is_long ? a.M / a.splits : a.M / a.q) / C::BK);
    t.c0 = piece > 0 ? piece * t.nk : 0;
    t.piece = piece;
  }
  return t;
}

template <class C, Op OP>
__global__ __launch_bounds__(C::THREADS, 1) void grad_persistent_kernel(GradArgs a) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int32_t* ws = a.ws;
  if (ws[1] != kIndexMagic || ws[2] != a.q || ws[3] != a.M) return;
  const int cyc = ws[4];
  if (cyc < 0) return;  // listed schedule: the register-staged kernel handles it
  const int q = a.q;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);

  // the type index of the cyclic schedule, in closed form
  const CycIndex ix = CycIndex::make(q, uni(cyc), a.M, C::BM);
  // first row of each type in the cyclic schedule
  auto type_start = [&](int i) { return i >= cyc ? i - cyc : i - cyc + q; };

  GradArgs g = a;
  int n_long, n_short, t_long, t_short;
  if constexpr (OP == Op::Dx) {
    g.n_rt = ix.tiles_before(q);
    n_long = g.n_rt * g.cpg;
    n_short = g.n_rt * (q - 1) * g.cpg;
    t_long = g.N / C::BK;
    t_short = g.r / C::BK;
  } else {
    const int tpb = g.rpb * g.cpg;
    n_long = q * tpb * g.splits;  // pieces of the split long tiles
    n_short = q * (q - 1) * tpb;
    t_long = g.M / g.splits / C::BK;
    t_short = g.M / q / C::BK;
  }

  const int nx = gridDim.x >= 8 ? 8 : 1;
  const int per_x = gridDim.x / nx;
  const int xcd = blockIdx.x % nx, slot = blockIdx.x / nx;
  if (slot >= per_x) return;

  const uint32_t a_ld = uint32_t(OP == Op::Dx ? g.N : g.K) * 2u;   // bytes per row of A
  const uint32_t b_ld = uint32_t(g.N) * 2u;                         // bytes per row of B (W or dY)
  const uint32_t c_ld = uint32_t(OP == Op::Dx ? g.K : g.N) * 2u;    // bytes per row of C

  // ---------------- copy cursor ----------------
  TileDeal dcopy;
  dcopy.init(n_long, n_short, t_long, t_short, xcd, nx, slot, per_x);
  bool l_long;
  int l_idx;
  if (!dcopy.next(&l_long, &l_idx)) return;
  GTile lt = decode<C, OP>(g, ix, l_long, l_idx);
  int lk = 0;
  bool more = true;  // the copy cursor has not passed the last k-step

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
      a_c[u] = (sl - (sl / C::A_NCH) * C::A_NCH) ^ swz_w(sl / C::A_NCH);
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
      b_c[u] = (sl - (sl / C::B_NCH) * C::B_NCH) ^ swz_w(sl / C::B_NCH);
    }
  }
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>(smem)));

  // copy cursor in three parts (per-step offsets, one copy, advance) so that
  // the copies can be interleaved with MFMAs
  int cp_kc = 0, cp_start = 0, cp_rbase = 0, cp_rstep = 1;
  auto prep_copies = [&]() {
    if constexpr (OP == Op::Dx) {
      cp_kc = lt.c0 + lk * C::BK;
      cp_start = type_start(lt.type);
    } else {
      const int k0 = (lt.c0 + lk) * C::BK;  // c0: a split piece's first k-step
      cp_rbase = lt.type < 0 ? k0 : type_start(lt.type) + k0 * q;
      cp_rstep = lt.type < 0 ? 1 : q;
    }
  };
  auto copy_u = [&](int stage, int u) {
    const uint32_t S = lds0 + uint32_t(stage * C::STAGE);
    if constexpr (OP == Op::Dx) {
      // A = dY rows of type lt.type (tile rows), B = W rows n0.. (tile rows);
      // contraction columns cp_kc..
      if (u < C::A_DMA) {
        const int row = cp_start + (lt.out_row0 + min(a_r[u], lt.m_cnt - 1)) * q;
        copy16_to_lds(g.A, uint32_t(row) * a_ld + uint32_t(cp_kc + a_c[u] * 8) * 2u,
                      S + uint32_t((wid * C::A_DMA + u) * 1024));
      } else {
        const int v = u - C::A_DMA;
        copy16_to_lds(g.B, uint32_t(lt.n0 + b_r[v]) * b_ld + uint32_t(cp_kc + b_c[v] * 8) * 2u,
                      S + uint32_t(C::A_BYTES + (wid * C::B_DMA + v) * 1024));
      }
    } else {
      // contraction rows: all rows (long tiles) or the rows of type lt.type
      if (u < C::A_DMA) {
        const int row = cp_rbase + a_r[u] * cp_rstep;
        copy16_to_lds(g.A, uint32_t(row) * a_ld + uint32_t(lt.out_row0 + a_c[u] * 8) * 2u,
                      S + uint32_t((wid * C::A_DMA + u) * 1024));
      } else {
        const int v = u - C::A_DMA;
        const int row = cp_rbase + b_r[v] * cp_rstep;
        copy16_to_lds(g.B, uint32_t(row) * b_ld + uint32_t(lt.n0 + b_c[v] * 8) * 2u,
                      S + uint32_t(C::A_BYTES + (wid * C::B_DMA + v) * 1024));
      }
    }
  };
  // After the last k-step the cursor stays on it: the copies issued for the
  // k-steps past the end repeat it into stages that are never read (drained
  // before exit), so that the pipeline needs no conditions.
  auto advance_copies = [&]() {
    if (more && (lk = uni(lk + 1)) >= lt.nk) {
      if (dcopy.next(&l_long, &l_idx)) {
        lt = decode<C, OP>(g, ix, l_long, uni(l_idx));
        lk = 0;
      } else {
        more = false;
        lk = uni(lt.nk - 1);
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
  // contraction-major operand: 128-bit read of row l32, piece 2*ks + lhi
  auto km_rd = [&](int w0, int ks) { return (w0 + l32) * C::KROWB + (((2 * ks + lhi) ^ swz_km<C::BK>(l32)) << 4); };
  // row-major operand with rows of rowb bytes: per-lane offsets of the two
  // transposing reads, by parity of the fragment's 32-column block index
  auto rm_rd = [&](int rowb, int par) {
    const int gq = lane >> 4, t = lane & 15;
    const int k_l = 8 * (gq >> 1) + (t >> 2);
    const int f = swz_w(k_l);
    const int r2 = 2 * (gq & 1) + ((t & 3) >> 1);
    const int lo = ((r2 ^ (f & 2)) << 4) + 8 * (t & 1) + k_l * rowb;
    const int dm = (f >> 2) ? 64 : 0;
    return par == 0 ? lo + dm : lo - dm;
  };
  // contraction-major: one offset per quarter step; row-major: one per
  // parity of the 32-column block index (entries 2, 3 unused)
  int a_rd[C::Q], b_rd[C::Q];
#pragma unroll
  for (int x = 0; x < C::Q; ++x) {
    a_rd[x] = C::A_KM ? km_rd(wm * C::WTM, x) : rm_rd(C::A_ROWB, x & 1);
    b_rd[x] = C::A_BYTES + (C::B_KM ? km_rd(wn * C::WTN, x) : rm_rd(C::B_ROWB, x & 1));
  }
  const int am0 = wm * (C::WTM / 32), bm0 = wn * (C::WTN / 32);

  f32x16 acc[C::FM][C::FN];
  bf16x8 fa0[C::FM], fb0[C::FN], fa1[C::FM], fb1[C::FN];
  auto read_a = [&](int stage, int ks, int fm) -> bf16x8 {
    const char* S = smem + stage * C::STAGE;
    if constexpr (C::A_KM) {
      return *reinterpret_cast<const bf16x8*>(S + a_rd[ks] + fm * 32 * C::KROWB);
    } else {
      const int m = am0 + fm;
      const char* p = S + a_rd[m & 1] + 64 * m + 16 * ks * C::A_ROWB;
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
      const int m = bm0 + fn;
      const char* p = S + b_rd[m & 1] + 64 * m + 16 * ks * C::B_ROWB;
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
#pragma unroll
  for (int st = 0; st < S - 1 + (S == 2 ? 1 : 0); ++st) issue_copies(st);
  // two stages: step 1 may be in flight; four: steps 1 and 2
  wait_vmcnt<(S == 2 ? 1 : 2) * C::DMA>();
  lds_barrier();
  load_frags(0, 0, fa0, fb0);

  TileDeal dcomp;
  dcomp.init(n_long, n_short, t_long, t_short, xcd, nx, slot, per_x);
  bool c_long;
  int c_idx;
  dcomp.next(&c_long, &c_idx);
  GTile ct = decode<C, OP>(g, ix, c_long, uni(c_idx));
  int stage = 0;  // LDS stage of the current k-step
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
      // a piece of a split long tile: its fp32 sums go to the piece's partial
      // tile (lane (l32, lhi) holds 4 consecutive columns of one row per
      // group gg, i.e. one 16-byte piece); the reduction rounds them
      float* P = g.part + size_t(ct.piece) * size_t(g.part_stride);
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
            *reinterpret_cast<u32x4*>(P + row * size_t(g.N) + size_t(col)) = val;
          }
        }
      }
    } else {
      // epilogue: one rounding of each fp32 sum, restaged through the wave's
      // share of the LDS behind the stages so that each store instruction
      // writes whole 16-byte pieces of a few rows
      char* ebuf = smem + C::E_OFF + wid * C::E_BYTES;
      const uint32_t col0 = uint32_t(ct.n0 + wn * C::WTN) * 2u;
      const int ostart = OP == Op::Dx ? type_start(ct.type) : 0;
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
          const int orow = OP == Op::Dx ? ostart + (ct.out_row0 + ml) * q : ct.out_row0 + ml;
          // non-temporal whole-line stores keep the output out of L2 (as in the forward)
          if (ml < ct.m_cnt)
            __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(g.C + (uint32_t(orow) * c_ld + col0 + uint32_t(pc) * 16u)));
        }
      }
    }
    if (!dcomp.next(&c_long, &c_idx)) break;
    ct = decode<C, OP>(g, ix, c_long, uni(c_idx));
  }
  // the repeated copies past the last k-step land in LDS: drain them before
  // the workgroup's LDS can be handed to another workgroup
  wait_vmcnt<0>();
}

// dW of a split launch: dW[diagonal block] = bf16(sum over pieces of the fp32
// partial tiles), pieces in order, one rounding.  One thread per 4 consecutive
// elements of the q diagonal blocks (s x r each).  Like the persistent kernel
// it does nothing unless the index holds a cyclic schedule of this problem
// (on other schedules the register-staged kernel writes all of dW).
__global__ __launch_bounds__(256) void dw_diag_reduce_kernel(const int32_t* __restrict__ ws, int q, int M,
                                                             const float* __restrict__ part, int splits,
                                                             int64_t stride, int N, int s, int r,
                                                             uint16_t* __restrict__ dW) {
  if (ws[1] != kIndexMagic || ws[2] != q || ws[3] != M || ws[4] < 0) return;
  const int64_t r4 = r / 4;
  const int64_t per_blk = int64_t(s) * r4;
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= q * per_blk) return;
  const int b = int(i / per_blk);
  const int64_t w = i - b * per_blk;
  const int64_t f = w / r4, c4 = w - f * r4;
  const int64_t off = (int64_t(b) * s + f) * N + int64_t(b) * r + c4 * 4;
  u32x4 x = *reinterpret_cast<const u32x4*>(part + off);
  float v0 = __uint_as_float(x[0]), v1 = __uint_as_float(x[1]), v2 = __uint_as_float(x[2]), v3 = __uint_as_float(x[3]);
  for (int p = 1; p < splits; ++p) {
    x = *reinterpret_cast<const u32x4*>(part + p * stride + off);
    v0 += __uint_as_float(x[0]);
    v1 += __uint_as_float(x[1]);
    v2 += __uint_as_float(x[2]);
    v3 += __uint_as_float(x[3]);
  }
  *reinterpret_cast<u32x2*>(dW + off) = pack4_bf16(v0, v1, v2, v3);
}

template <int BN>
using DxCfg = GradCfg<256, BN, true, true, kBKDx, 2>;
template <int BN>
using DwCfg = GradCfg<256, BN, false, false, kBKDw, 4>;

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

template <class C, Op OP>
hipError_t launch_grad(const ProblemDesc& p, hipStream_t s) {
  static bool attr_set = false;
  const int lds = C::LDS_BYTES;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&grad_persistent_kernel<C, OP>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  GradArgs a{};
  a.A = static_cast<const char*>(p.A);
  a.B = static_cast<const char*>(p.B);
  a.C = static_cast<char*>(p.C);
  a.ws = p.ws;
  const WsLayout L = ws_layout(p.q, p.M);
  a.off_offsets = L.offsets;
  a.off_tiles = L.tile_off;
  a.q = p.q;
  a.M = int(p.M);
  a.K = int(p.K);
  a.N = int(p.N);
  a.s = int(p.K / p.q);
  a.r = int(p.N / p.q);
  if (OP == Op::Dx) {
    a.cpg = a.s / C::BN;
    a.rpb = 0;
  } else {
    a.cpg = a.r / C::BN;
    a.rpb = a.s / C::BM;
  }
  int grid = cu_count();
  grid = grid >= 8 ? grid / 8 * 8 : grid;
  a.splits = 1;
  a.part = nullptr;
  a.part_stride = 0;
  if (OP == Op::Dw && p.dw_part != nullptr) {
    // split the long (diagonal) tiles until a piece is no longer than the
    // average k-steps per workgroup
    const int64_t tpb = int64_t(a.rpb) * a.cpg;
    const int64_t t_long = p.M / C::BK, t_short = p.M / p.q / C::BK;
    const int64_t total = p.q * tpb * t_long + p.q * (p.q - 1) * tpb * t_short;
    const int64_t avg = (total + grid - 1) / grid;
    int sp = 1;
    while (sp * 2 <= kDwMaxSplits && t_long % (sp * 2) == 0 && t_long / sp > avg) sp *= 2;
    a.splits = sp;
    a.part = static_cast<float*>(p.dw_part);
    a.part_stride = p.K * p.N;
  }
  const size_t shm = C::LDS_BYTES;
  hipLaunchKernelGGL((grad_persistent_kernel<C, OP>), dim3(grid), dim3(C::THREADS), shm, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  const int64_t threads = p.q * int64_t(a.s) * (a.r / 4);
  hipLaunchKernelGGL(dw_diag_reduce_kernel, dim3(unsigned((threads + 255) / 256)), dim3(256), 0, s, p.ws, a.q, a.M,
                     a.part, a.splits, a.part_stride, a.N, a.s, a.r, static_cast<uint16_t*>(p.C));
  return hipGetLastError();
}

int pick_bn(int64_t w) { return w % 256 == 0 ? 256 : w % 192 == 0 ? 192 : w % 128 == 0 ? 128 : 0; }

}  // namespace

bool grad_persistent_supported(const ProblemDesc& p) {
  if (p.E != 1 || (p.op != Op::Dx && p.op != Op::Dw)) return false;
  const int64_t s = p.K / p.q, r = p.N / p.q;
  const int64_t lim = int64_t(1) << 31;
  if (p.M * p.K >= lim || p.K * p.N >= lim || p.M * p.N >= lim) return false;
  if (p.op == Op::Dx) {
    // rows of a type in 256-row tiles; columns of an input group in BN tiles;
    // contraction lengths N and r in whole k-steps
    return (p.M + p.q - 1) / p.q >= 128 && pick_bn(s) != 0 && r % kBKDx == 0;
  }
  // features of a group in 256-row tiles, output group columns in BN tiles,
  // every type's rows (M / q of a cyclic schedule) in whole k-steps
  return s % 256 == 0 && pick_bn(r) != 0 && p.M % (int64_t(kBKDw) * p.q) == 0 && p.M >= int64_t(kBKDw) * p.q;
}

hipError_t launch_grad_persistent_bf16(const ProblemDesc& p, hipStream_t s) {
  const int bn = pick_bn(p.op == Op::Dx ? p.K / p.q : p.N / p.q);
  if (p.op == Op::Dx) {
    if (bn == 256) return launch_grad<DxCfg<256>, Op::Dx>(p, s);
    if (bn == 192) return launch_grad<DxCfg<192>, Op::Dx>(p, s);
    return launch_grad<DxCfg<128>, Op::Dx>(p, s);
  }
  if (bn == 256) return launch_grad<DwCfg<256>, Op::Dw>(p, s);
  if (bn == 192) return launch_grad<DwCfg<192>, Op::Dw>(p, s);
  return launch_grad<DwCfg<128>, Op::Dw>(p, s);
}

}  // namespace qalg
