// Causal attention with the algebraic score (arXiv 2609.32814, appendix G),
// forward, bf16 in and out, fp32 softmax statistics and accumulation.
//
// A query at position p (type i = p mod q; rows s of a chunk whose first row
// sits at absolute position p0 have p = p0 + s) and a key at u (type j) compare only
// the feature groups F(i, j) of the head: {i} if i == j, else {i, j} (eq 38;
// eq 42 for the recursive law Q_2^(x)L: every group whose bits each come from i
// or j).  The score r_pu (eq 39) is scaled by 1/sqrt(|F| m), m = d / q (eq 41),
// masked to u <= p (eq 43), softmaxed, and the values are aggregated densely
// (eq 44).  Algorithm 2, steps 3-7, for one sequence per head.
//
// Work.  A workgroup owns 128 queries of one type i of one head (rows
// s_i + q t for 128 consecutive t, s_i = (i - p0) mod q), 32 per wave, and walks
// the keys type by type: keys of type j are the rows s_j + q t', so a block of 64 of them shares
// one support F(i, j), i.e. one contraction of |F| m features instead of d.
// Per key block: S = Q K^T over the support's groups (MFMA 32x32x16, K read
// row-major from LDS), the causal mask on the actual positions, an online
// softmax (running row max and sum, flash-attention style), then O += P V
// over all d features (MFMA with V read transposed from LDS).  K and V blocks
// travel global -> LDS by direct copies into two stages, the next block's
// while the current one is computed (one barrier per block); a block that
// lies wholly before the wave's earliest query skips the mask.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "qalg_internal.h"
#include "qalg_device.h"

namespace qalg {
namespace {

using dev::bf16x8;
using dev::bf16x2;
using dev::f32x16;
using dev::s16x4;
using dev::u32x2;
using dev::u32x4;
using dev::pack4_bf16;
using dev::uni;
using dev::copy16_to_lds;
using dev::lds_barrier;
using dev::wait_vmcnt;

constexpr int kAttnQ = 128;   // queries per workgroup (32 per wave)
constexpr int kAttnK = 64;    // keys per block
constexpr int kAttnThreads = 256;

struct AttnArgs {
  const char* Q;
  const char* K;
  const char* V;
  char* O;
  int Hq, Hkv, S, q, L;
  int m;          // features per group (d / q)
  int n_qblk;     // query blocks per (head, type)
  int o;          // type of row 0: rows s have positions p0 + s and types (o + s) mod q, o = p0 mod q
  float* lse;     // Hq x S natural-log sums of exp(score) per query (for the backward), or null
};

// groups compared by types (i, j): count, and the b-th one
__device__ __forceinline__ int support_count(int i, int j, int L) {
  if (L == 0) return i == j ? 1 : 2;
  return 1 << __builtin_popcount(i ^ j);
}
__device__ __forceinline__ int support_group(int i, int j, int L, int b) {
  if (L == 0) return b == 0 ? i : j;
  const int f = i ^ j;
  int g = i & ~f;
  for (int k = 0, n = b; k < L; ++k)
    if ((f >> k) & 1) {
      if (n & 1) g |= 1 << k;
      n >>= 1;
    }
  return g;
}

// LDS swizzles for rows of D features.  The 64 banks cover 256 bytes: a row of
// 128 features is one bank window, a row of 64 half of one.
// K (read 16 bytes per lane, 16 rows at a time): row r keeps piece c at c ^ swk(r).
template <int D>
__device__ __forceinline__ int swk(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
// V (read transposed: 4 rows x four 16-byte pieces of one 64-byte column block
// per 16 lanes): row r keeps column block b at b ^ swv(r), so that the 4 rows
// land in 4 different blocks of the bank window.
template <int D>
__device__ __forceinline__ int swv(int r) { return D == 128 ? (r & 3) : ((r >> 1) & 1); }

template <int D>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_fwd_kernel(AttnArgs a) {
  constexpr int ROWB = D * 2;          // bytes per K / V row
  constexpr int NP = D / 8;            // 16-byte pieces per row
  constexpr int KS = D / 16;           // 16-feature MFMA steps over a row (2 pieces each)
  constexpr int DB = D / 32;           // 32-feature output blocks
  constexpr int BLK = kAttnK * ROWB;   // bytes of a K (or V) block
  constexpr int LOADS = BLK / (4 * 1024);  // 1 KB direct-to-LDS copies per wave per block (K and V each)
  static_assert(BLK % 4096 == 0, "whole 1 KB copies per wave");
  // two stages of [K block | V block]
  __shared__ __attribute__((aligned(1024))) char smem[2 * 2 * BLK];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, lhi = lane >> 5;
  // block -> (head, query type, query block); heavy (late) query blocks first
  int bid = blockIdx.x;
  const int qb = a.n_qblk - 1 - bid % a.n_qblk;
  bid /= a.n_qblk;
  const int i = bid % a.q;
  const int h = bid / a.q;
  const int kvh = h / (a.Hq / a.Hkv);
  const int q = a.q, S = a.S;
  // rows of type t are first_row(t) + q k (the type offset o shifts them)
  auto first_row = [&](int t) -> int { return t >= a.o ? t - a.o : t - a.o + q; };
  const int si = first_row(i);
  const int n_i = S > si ? (S - si + q - 1) / q : 0;  // queries of type i
  const int t0 = qb * kAttnQ;
  if (t0 >= n_i) return;
  const int t_last = min(t0 + kAttnQ, n_i) - 1;
  const int p_last = si + q * t_last;                // latest query row in the block
  const int p_wave0 = si + q * min(t0 + 32 * wid, n_i - 1);  // earliest query row of the wave
  const int p_wave1 = si + q * min(t0 + 32 * wid + 31, n_i - 1);  // latest query row of the wave

  const char* Qh = a.Q + int64_t(h) * S * ROWB;
  const char* Kh = a.K + int64_t(kvh) * S * ROWB;
  const char* Vh = a.V + int64_t(kvh) * S * ROWB;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>(smem)));

  // this lane's query row (row l32 of the wave's 32); the fragments of the
  // support's groups are loaded from it whenever the key type changes
  const int tq = t0 + wid * 32 + l32;
  const bool q_ok = tq < n_i;
  const int tqc = min(tq, n_i - 1);
  const int pq = si + q * tqc;
  const char* q_row = Qh + int64_t(pq) * ROWB + 16 * lhi;

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = (f32x16){};
  float m_run = -INFINITY, l_run = 0.f;

  // LDS layouts above; the direct-to-LDS copies land lane-linear, so each
  // lane fetches the global piece that belongs at its slot.  Transposed V
  // reads: in a 16-lane group (g = lane / 16, t = lane % 16) lane t reads 8
  // bytes of row 8 (g / 2) + t / 4 (and the row 4 below), piece 2 (g % 2) +
  // (t % 4) / 2 of the column block, half t % 2; the transpose hands lane t
  // column t of the block with 4 consecutive rows from each read.
  int v_rd[DB];
  {
    const int g = lane >> 4, t = lane & 15;
    const int k_l = 8 * (g >> 1) + (t >> 2);
    const int r2 = 2 * (g & 1) + ((t & 3) >> 1);
    const int lo = k_l * ROWB + (r2 << 4) + 8 * (t & 1);
#pragma unroll
    for (int db = 0; db < DB; ++db) v_rd[db] = lo + ((db ^ swv<D>(k_l)) << 6);
  }
  int k_row[LOADS];
  uint32_t k_pc[LOADS], v_pc[LOADS];
#pragma unroll
  for (int x = 0; x < LOADS; ++x) {
    const int sl = (wid * LOADS + x) * 64 + lane;
    k_row[x] = sl / NP;
    const int c = sl % NP;
    k_pc[x] = uint32_t(c ^ swk<D>(k_row[x])) * 16u;
    v_pc[x] = uint32_t(c ^ (swv<D>(k_row[x]) << 2)) * 16u;
  }

  // key blocks, type by type; the cursor (cj, ct) names the next block to copy
  int cj = 0, ct = 0;
  auto keys_of = [&](int j) -> int {
    // keys of type j that some query of the block may see: u = first_row(j) + q t' <= p_last < S
    const int sj = first_row(j);
    return p_last >= sj ? (p_last - sj) / q + 1 : 0;
  };
  auto skip_empty = [&]() {
    while (cj < q && ct >= keys_of(cj)) {
      cj = uni(cj + 1);
      ct = 0;
    }
  };
  auto issue = [&](int stage) {
    const int nk = keys_of(cj);
    const uint32_t base = lds0 + uint32_t(stage * 2 * BLK) + uint32_t(wid * LOADS * 1024);
#pragma unroll
    for (int x = 0; x < LOADS; ++x) {
      const uint32_t u = uint32_t(first_row(cj) + q * min(ct + k_row[x], nk - 1));
      copy16_to_lds(Kh, u * ROWB + k_pc[x], base + uint32_t(x * 1024));
      copy16_to_lds(Vh, u * ROWB + v_pc[x], base + uint32_t(BLK + x * 1024));
    }
  };

  const float log2e = 1.4426950408889634f;
  // the current key type's support as MFMA slots (see below)
  int cur_j = -1, tot = 0;
  int kp[KS];
  bf16x8 qsl[KS];
  skip_empty();
  int stage = 0;
  int bj = cj, btb = ct;  // the block in flight
  issue(0);
  ct = uni(ct + kAttnK);
  skip_empty();
  for (;;) {
    // this block's copies have landed; every wave is done with the other stage
    wait_vmcnt<0>();
    lds_barrier();
    const int j = bj, tb = btb;
    const bool more = cj < q;
    // scores of the wave's 32 queries against the 64 keys over the support's
    // groups only.  When the key type changes, the support's k-steps are laid
    // out as slots: slot x holds the query fragment and the K piece of the
    // x-th 16-feature step of F(i, j); the block then runs exactly `tot`
    // MFMA steps per 32-key tile, through a switch on tot, so that no MFMA is
    // conditional inside straight-line code.  The slot loads are waited for
    // here, before the next block's copies are issued: the copies then never
    // sit behind a wait for them.
    if (j != cur_j) {
      cur_j = j;
      const int ms = a.m / 16;
      tot = uni(support_count(i, j, a.L) * ms);
#pragma unroll
      for (int x = 0; x < KS; ++x) {
        const int step = x < tot ? support_group(i, j, a.L, x / ms) * ms + x % ms : 0;
        kp[x] = uni(2 * step);
        qsl[x] = *reinterpret_cast<const bf16x8*>(q_row + 32 * step);
      }
      wait_vmcnt<0>();
    }
    if (more) {
      bj = cj;
      btb = ct;
      issue(stage ^ 1);
      ct = uni(ct + kAttnK);
      skip_empty();
    }
    const char* sK = smem + stage * 2 * BLK;
    const char* sV = sK + BLK;

    // a block whose first key lies past the wave's latest query adds nothing
    // to its rows: the wave only takes part in the copies and barriers
    if (first_row(j) + q * tb <= p_wave1) {
      f32x16 sc[2];
      auto scores = [&](auto tot_c) {
        constexpr int T = decltype(tot_c)::value;
        sc[0] = (f32x16){};
        sc[1] = (f32x16){};
        // the block's K fragment reads are written ahead of its MFMAs, which
        // leaves the scheduler free to issue them as early as registers allow
        bf16x8 kf[T][2];
#pragma unroll
        for (int x = 0; x < T; ++x) {
          const int pc = kp[x] + lhi;
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            const int row = nb * 32 + l32;
            kf[x][nb] = *reinterpret_cast<const bf16x8*>(sK + row * ROWB + ((pc ^ swk<D>(row)) << 4));
          }
        }
#pragma unroll
        for (int x = 0; x < T; ++x)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            sc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[x][nb], qsl[x], sc[nb], 0, 0, 0);
      };
      switch (tot) {
        case 1: scores(std::integral_constant<int, 1>{}); break;
        case 2: scores(std::integral_constant<int, 2>{}); break;
        case 3: scores(std::integral_constant<int, 3>{}); break;
        case 4: scores(std::integral_constant<int, 4>{}); break;
        case 5: scores(std::integral_constant<int, 5>{}); break;
        case 6: scores(std::integral_constant<int, 6>{}); break;
        case 7: scores(std::integral_constant<int, 7>{}); break;
        default: scores(std::integral_constant<int, KS>{}); break;
      }
      const int nf = tot / (a.m / 16);
      // causal mask (only blocks that reach past the wave's earliest query, or past the type's keys)
      const int nk_j = keys_of(j);
      const int sj = first_row(j);
      const bool full = tb + kAttnK <= nk_j && sj + q * (tb + kAttnK - 1) <= p_wave0;
      if (!full) {
        // key u = sj + q tk is allowed iff u <= pq = si + q tqc, i.e. (both first
        // rows in [0, q)) iff tk <= tqc - [si < sj]; keys past the type's last
        // allowed one fail it too (pq <= p_last).  One compare per score against
        // the lane's limit, offset to the element's constant key index.
        const int lim = tqc - (si < sj ? 1 : 0) - tb - 4 * lhi;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (nb * 32 + 8 * (e >> 2) + (e & 3) > lim) sc[nb][e] = -INFINITY;
      }
      // online softmax in the log2 domain: scale folded into the exponent
      const float scl = log2e * __builtin_amdgcn_rsqf(float(nf * a.m));
      float mx = -INFINITY;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[nb][e]);
      mx = fmaxf(mx, __shfl_xor(mx, 32)) * scl;
      // the running max moves only when some row's block max passes it by more
      // than 8 (factors of 2): probabilities then stay below 2^8, and most blocks
      // skip rescaling the output accumulators
      if (__any(mx > m_run + 8.0f)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[db][e] *= alpha;
        m_run = m_new;
      }
      const float base = m_run == -INFINITY ? 0.f : m_run;
      float rs = 0.f;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[nb][e], scl, -base));
          sc[nb][e] = pv;
          rs += pv;
        }
      rs += __shfl_xor(rs, 32);
      l_run += rs;

      // O += P V: 16 keys per step; the lane pair (l32, 0/1) exchanges half its
      // probabilities so that each lane holds 8 consecutive keys of its row
#pragma unroll
      for (int ks = 0; ks < kAttnK / 16; ++ks) {
        const int nb = ks >> 1;
        // keys 16 ks .. +15 are groups ga = 2 (ks & 1) and ga + 1 of the score
        // tile: lane half 0 keeps group ga and sends ga + 1, half 1 the reverse
        // (register indices stay compile-time; only the choice is per lane)
        const int ga = 2 * (ks & 1);
        const u32x2 pa = pack4_bf16(sc[nb][4 * ga], sc[nb][4 * ga + 1], sc[nb][4 * ga + 2], sc[nb][4 * ga + 3]);
        const u32x2 pb = pack4_bf16(sc[nb][4 * ga + 4], sc[nb][4 * ga + 5], sc[nb][4 * ga + 6], sc[nb][4 * ga + 7]);
        // v_permlane32_swap exchanges lanes 32-63 of its first operand with
        // lanes 0-31 of its second: on (pa, pb) half 0 ends with its own
        // group-ga piece and the partner's, half 1 with the partner's group-ga+1
        // piece and its own, in key order in both, with no per-lane selects
        const auto s0 = __builtin_amdgcn_permlane32_swap(pa[0], pb[0], false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(pa[1], pb[1], false, false);
        const u32x4 pw = {s0[0], s1[0], s0[1], s1[1]};
        const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const char* pp = sV + v_rd[db] + 16 * ks * ROWB;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(pp));
          const s16x4 hi =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(pp + 4 * ROWB));
          const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, acc[db], 0, 0, 0);
        }
      }
    }
    if (!more) break;
    stage ^= 1;
  }

  // O = acc / l, one rounding; lane holds row l32, features 32 db + 8 g + 4 lhi + 0..3
  if (q_ok) {
    const float inv = 1.0f / l_run;
    char* orow = a.O + (int64_t(h) * S + pq) * ROWB;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2 v = pack4_bf16(acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv, acc[db][4 * g + 2] * inv,
                                   acc[db][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + (32 * db + 8 * g + 4 * lhi) * 2) = v;
      }
    // log of the softmax denominator in the scores' own units: the running
    // max and sum live in the log2 domain of the scaled scores
    if (a.lse != nullptr && lhi == 0) a.lse[int64_t(h) * S + pq] = (m_run + __log2f(l_run)) * 0.6931471805599453f;
  }
}

// ---------------------------------------------------------------------------
// Cached decoding (appendix G, Algorithm 3; G.2): one new query row per
// sequence against that sequence's full-key cache.
//
// The cache is HBM-bound work: every allowed slot's value row is read once,
// and of its key row only the feature groups F(i, j) that the query's type i
// and the key's type j compare (m or 2m of the d features for Q_q), so the key
// bytes shrink with the score arithmetic (eq 57).  A key's type comes from its
// absolute position (G.2), through the same schedule as the projections.
//
// Split over the cache: a workgroup takes a chunk of kDecCh slots of one
// (sequence, key/value head) and serves all G = Hq / Hkv query heads that read
// that head (GQA), so each slot is read once for all of them.  It writes, per
// query head, the chunk's max score, the sum of exp(score - max) and the
// unnormalised value sum in fp32; a second kernel combines the chunks in a
// fixed order (the result does not depend on scheduling).
//
// Lanes map to features: in a group of D / 8 lanes (16 for d = 128) lane p
// owns the 16-byte piece p (features 8p .. 8p + 7) of a row, and holds the G
// query heads' values of those features in registers.  A wave covers 64 / (D / 8)
// slots at a time.  Scores: each lane loads its key piece only when the piece's
// group is in F(i, j) (so only the compared groups are read), multiplies it
// with its query features (v_dot2_f32_bf16), and the group's lanes sum the G
// partial dot products with DPP row shifts (and a permlane exchange across
// rows for 32-lane groups); all key pieces of the chunk are in flight before
// the first is used.  Then one wave per query head takes the chunk max and the
// exponentials.  Values: the same lane/piece map over the value rows of the
// allowed slots, fp32 sums per head, reduced across the lane groups of a wave
// and then across waves in a fixed order.
// ---------------------------------------------------------------------------

constexpr int kDecCh = 128;       // cache slots per workgroup
constexpr int kDecThreads = 256;
constexpr int kDecMaxG = 8;       // query heads per key/value head
constexpr int kDecMaxChunks = 2048;  // chunks the combination takes (N <= kDecCh * kDecMaxChunks)

struct DecArgs {
  const char* Q;       // B x Hq x d
  const char* K;       // B x Hkv x N x d
  const char* V;
  const int64_t* q_pos;    // B
  const int64_t* key_pos;  // B x N
  float* part;         // B x Hq x chunks x (d + 4)
  char* O;             // B x Hq x d
  int B, Hq, Hkv, G, q, L, m, kind, chunks;
  int64_t N, period;
};

static_assert(kDecCh <= kDecThreads, "one slot per thread at most");

// the position schedule (section 4; appendix D.5): -1 for a negative position
__device__ __forceinline__ int dec_type(int64_t pos, int q, int kind, int64_t period) {
  if (pos < 0) return -1;
  if (kind == 0) return int(pos % q);
  return int((pos % period) / (period / q));
}

// is group a one of F(i, j)?  Q_q: a = i or a = j (eq 38); the recursive law:
// each bit of a equals i's or j's (eq 42)
__device__ __forceinline__ bool in_support(int a, int i, int j, int L) {
  if (L == 0) return a == i || a == j;
  return ((a ^ i) & (a ^ j)) == 0;
}

// Cross-lane sums on the VALU (no LDS traffic).  row_tail_sum: the lane at
// position n - 1 of each group of n consecutive lanes (n = 8 or 16, groups
// inside a 16-lane row) receives the group's sum, through DPP row shifts that
// read 0 past the row start (bound_ctrl).
template <int k>
__device__ __forceinline__ float add_row_shr(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + k, 0xf, 0xf, true));
}
template <int n>
__device__ __forceinline__ float row_tail_sum(float x) {
  static_assert(n == 8 || n == 16, "groups of 8 or 16 lanes");
  x = add_row_shr<1>(x);
  x = add_row_shr<2>(x);
  x = add_row_shr<4>(x);
  if constexpr (n == 16) x = add_row_shr<8>(x);
  return x;
}
// every lane receives the sum over the lanes with its position in the 16-lane
// row (the four rows), by v_permlane16_swap then v_permlane32_swap
__device__ __forceinline__ float rows_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// the sum of lane l and lane l ^ 8 (the two halves of a 16-lane row), by a row rotation
__device__ __forceinline__ float half_rows_sum(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));
}

__device__ __forceinline__ void unpack8(const u32x4 v, float (&f)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = __uint_as_float(v[e] << 16);
    f[2 * e + 1] = __uint_as_float(v[e] & 0xffff0000u);
  }
}

// GM: the query heads per key/value head rounded up to a power of two (register arrays)
template <int D, int GM>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(3))) void attn_decode_kernel(DecArgs a) {
  constexpr int NP = D / 8;                    // lanes (16-byte pieces) per row
  constexpr int SPW = 64 / NP;                 // slots per wave step
  constexpr int SPB = kDecThreads / NP;        // slots per workgroup step
  constexpr int STEPS = kDecCh / SPB;          // steps over the chunk
  __shared__ float ssc[kDecCh][GM];      // scores, then exp(score - max)
  __shared__ int styp[kDecThreads];            // key type of each slot, -1: not allowed (slots past the chunk: -1)
  __shared__ float smax[GM], ssum[GM];
  __shared__ float sred[4][GM][D];       // per-wave value sums

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int c = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int G = a.G, q = a.q, m = a.m;
  const int64_t p = a.q_pos[b];
  const int i = dec_type(p, q, a.kind, a.period);
  const int64_t slot0 = int64_t(c) * kDecCh;
  const int nslot = int(min<int64_t>(kDecCh, a.N - slot0));
  const int pc = lane % NP;                    // this lane's piece of a row
  const int sub = tid / NP;                    // slot of this lane within a step
  const int grp = (pc * 8) / m;                // the feature group of the piece

  // allowed slots and their key types
  {
    int t = -1;
    if (tid < nslot && tid < kDecCh && i >= 0) {
      const int64_t u = a.key_pos[int64_t(b) * a.N + slot0 + tid];
      if (u >= 0 && u <= p) t = dec_type(u, q, a.kind, a.period);
    }
    styp[tid] = t;
  }
  // the G query heads' features of this lane's piece, as bf16 pairs
  u32x4 qv[GM];
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    qv[g] = (u32x4){0u, 0u, 0u, 0u};
    if (g < G) qv[g] = *reinterpret_cast<const u32x4*>(a.Q + ((int64_t(b) * a.Hq + kvh * G + g) * D + pc * 8) * 2);
  }
  __syncthreads();

  const int64_t row0 = (int64_t(b) * a.Hkv + kvh) * a.N + slot0;  // first slot's row in K / V
  // every needed key piece and every allowed value piece of the chunk is
  // requested before the first is used: one memory round trip per workgroup
  u32x4 kreg[STEPS], vreg[STEPS];
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    const int sl = st * SPB + sub;
    const int j = styp[sl];
    kreg[st] = (u32x4){0u, 0u, 0u, 0u};
    if (j >= 0 && in_support(grp, i, j, a.L))
      kreg[st] = *reinterpret_cast<const u32x4*>(a.K + ((row0 + sl) * D + pc * 8) * 2);
  }
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    const int sl = st * SPB + sub;
    vreg[st] = (u32x4){0u, 0u, 0u, 0u};
    if (styp[sl] >= 0) vreg[st] = *reinterpret_cast<const u32x4*>(a.V + ((row0 + sl) * D + pc * 8) * 2);
  }
  // scores
  {
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const int sl = st * SPB + sub;
      const int j = styp[sl];
      float r[GM];
      // (plain arrays: a bit cast of a vector-type element subscript loses the subscript in this compiler)
      const unsigned kw[4] = {kreg[st].x, kreg[st].y, kreg[st].z, kreg[st].w};
#pragma unroll
      for (int g = 0; g < GM; ++g) {
        const unsigned qw[4] = {qv[g].x, qv[g].y, qv[g].z, qv[g].w};
        r[g] = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          r[g] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kw[e]), __builtin_bit_cast(bf16x2, qw[e]),
                                                 r[g], false);
        // the row's pieces sit in NP consecutive lanes: their sum lands in the last one
        r[g] = row_tail_sum<NP>(r[g]);
      }
      if (pc == NP - 1) {
        const float scl = j >= 0 ? __builtin_amdgcn_rsqf(float(support_count(i, j, a.L) * m)) : 0.f;
#pragma unroll
        for (int g = 0; g < GM; ++g) ssc[sl][g] = g >= G ? 0.f : (j >= 0 ? r[g] * scl : -INFINITY);
      }
    }
  }
  __syncthreads();

  // per query head: chunk max, exponentials, their sum (one wave per head)
  for (int g = wid; g < G; g += 4) {
    float mx = -INFINITY;
    for (int sl = lane; sl < kDecCh; sl += 64) mx = fmaxf(mx, ssc[sl][g]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    float sum = 0.f;
    for (int sl = lane; sl < kDecCh; sl += 64) {
      const float e = mx == -INFINITY ? 0.f : __expf(ssc[sl][g] - mx);
      ssc[sl][g] = e;
      sum += e;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
    if (lane == 0) {
      smax[g] = mx;
      ssum[g] = sum;
    }
  }
  __syncthreads();

  // value sums over the allowed slots: this lane's 8 features, per head
  float acc[GM][8];
#pragma unroll
  for (int g = 0; g < GM; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
  {
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const int sl = st * SPB + sub;
      float vf[8];
      unpack8(vreg[st], vf);
      float w[GM];
#pragma unroll
      for (int g = 0; g < GM; ++g) w[g] = ssc[sl][g];
#pragma unroll
      for (int g = 0; g < GM; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = __builtin_fmaf(w[g], vf[e], acc[g][e]);
    }
  }
  // lane groups of a wave (same piece) in a fixed tree, then the waves in order
#pragma unroll
  for (int g = 0; g < GM; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (NP == 8) acc[g][e] = half_rows_sum(acc[g][e]);
      acc[g][e] = rows_sum(acc[g][e]);
    }
  if (lane < NP) {
#pragma unroll
    for (int g = 0; g < GM; ++g)
      if (g < G)
#pragma unroll
        for (int e = 0; e < 8; ++e) sred[wid][g][pc * 8 + e] = acc[g][e];
  }
  __syncthreads();
  float* part = a.part + ((int64_t(b) * a.Hq + kvh * G) * a.chunks + c) * (D + 4);
  for (int x = tid; x < G * D; x += kDecThreads) {
    const int g = x / D, f = x - g * D;
    const float v = ((sred[0][g][f] + sred[1][g][f]) + sred[2][g][f]) + sred[3][g][f];
    part[int64_t(g) * a.chunks * (D + 4) + f] = v;
  }
  if (tid < G) {
    float* pg = part + int64_t(tid) * a.chunks * (D + 4);
    pg[D] = smax[tid];
    pg[D + 1] = ssum[tid];
  }
}

// O = sum_c e^(M_c - M) O_c / sum_c e^(M_c - M) L_c over the chunks c with
// L_c > 0; one workgroup of D threads per (sequence, query head).  The chunk
// weights are formed once (thread t takes chunks t, t + D, ...; block max and
// sum in a fixed tree), then thread f sums its feature over the chunks in
// order.  Rows with no allowed slot (every L_c = 0) are written as zeros.
template <int D>
__global__ __launch_bounds__(D) void attn_decode_combine_kernel(const float* __restrict__ part, int chunks,
                                                                char* __restrict__ O) {
  constexpr int W = D / 64;
  __shared__ float sw[kDecMaxChunks];  // chunk weights
  __shared__ float sr[W];
  const int64_t row = blockIdx.x;
  const int f = threadIdx.x, lane = f & 63, wv = f >> 6;
  const float* pr = part + row * chunks * (D + 4);
  auto block_reduce = [&](float x, bool is_max) -> float {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float y = __shfl_xor(x, o);
      x = is_max ? fmaxf(x, y) : x + y;
    }
    __syncthreads();
    if (lane == 0) sr[wv] = x;
    __syncthreads();
    float t = sr[0];
    for (int w = 1; w < W; ++w) t = is_max ? fmaxf(t, sr[w]) : t + sr[w];
    return t;
  };
  float mloc = -INFINITY;
  for (int cc = f; cc < chunks; cc += D) {
    const float* pc = pr + int64_t(cc) * (D + 4);
    if (pc[D + 1] > 0.f) mloc = fmaxf(mloc, pc[D]);
  }
  const float M = block_reduce(mloc, true);
  float lloc = 0.f;
  for (int cc = f; cc < chunks; cc += D) {
    const float* pc = pr + int64_t(cc) * (D + 4);
    const float w = (M != -INFINITY && pc[D + 1] > 0.f) ? __expf(pc[D] - M) : 0.f;
    sw[cc] = w;
    lloc = __builtin_fmaf(w, pc[D + 1], lloc);
  }
  const float Lsum = block_reduce(lloc, false);  // its barriers also publish sw
  float acc = 0.f;
  for (int cc = 0; cc < chunks; ++cc) acc = __builtin_fmaf(sw[cc], pr[int64_t(cc) * (D + 4) + f], acc);
  const float v = Lsum > 0.f ? acc / Lsum : 0.f;
  const bf16x2 h = __builtin_convertvector((dev::f32x2){v, 0.f}, bf16x2);
  reinterpret_cast<uint16_t*>(O)[row * D + f] = uint16_t(__builtin_bit_cast(uint32_t, h) & 0xffffu);
}


// ---------------------------------------------------------------------------
// Backward (Algorithm 2, step 9): gradients of the algebraic-score attention.
// With P the softmax rows (recomputed from the scores and the forward's
// log-sum-exp), dP_pu = <dO_p, V_u> and D_p = <dO_p, O_p> (= sum_u P_pu dP_pu):
//   dS_pu = P_pu (dP_pu - D_p) / sqrt(|F(i, j)| m)      (softmax, then eq 41's scale)
//   dQ_p^(a) = sum_u dS_pu K_u^(a),  dK_u^(a) = sum_p dS_pu Q_p^(a)   (a in F(i, j) only, eq 39)
//   dV_u = sum_p P_pu dO_p
// attn_bwd_dq_kernel takes the forward's work split (128 queries of one type
// of one head) and its walk over the key blocks, type by type: scores over
// the support, P, dP = dO V^T over all d, dS, then dQ^T += K^T dS over the
// feature blocks that meet the support (K read transposed from LDS, features
// outside F(i, j) zeroed in the fragment).  It also stores each query's
// (log2-domain log-sum-exp, D) pair, grouped by type, for the second kernel.
// attn_bwd_dkdv_kernel owns 128 keys of one type of one key/value head (32 per
// wave, K and V rows in registers) and walks, for every query head that reads
// that head (GQA), the 64-query blocks of every type at or after its first key:
// S^T = Q K^T over the support, P^T, dP^T = dO V^T, dS^T, then dV^T += dO^T P
// and dK^T += Q^T dS (Q and dO read transposed).  Each key's dK and dV come
// from one workgroup, so no atomics and bitwise reproducible.  P and dS enter
// the MFMAs in bf16; everything else stays fp32 until the one rounding of dQ,
// dK and dV.  Rows live in LDS in the layout swb below (good for both the
// row and the transposing reads).
// ---------------------------------------------------------------------------

// LDS layout of the backward's row blocks: rows are read both as rows (16
// bytes per lane, 16 consecutive rows per pass) and transposed (8 bytes per
// lane, 4 rows x 4 pieces of one 64-byte column block per 32 lanes), so row r
// keeps its 16-byte piece c at c ^ swb(r), which is a permutation of the
// pieces over any 16 consecutive rows and sends the 4 rows of a transposed
// read to 4 different 64-byte blocks: both reads are free of bank conflicts
// (the K layout above gives the transposed read 4-way conflicts).  d = 128: a
// row fills the 64-bank window and swb swaps the two 2-bit fields of r mod 16;
// d = 64: two rows share a window (halves by r & 1), and swb takes the row
// pair index k = r / 2 to (k & 1) * 4 + (k / 2) % 4.
template <int D>
__device__ __forceinline__ int swb(int r) {
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

struct AttnBwdArgs {
  const char* Q;
  const char* K;
  const char* V;
  const char* O;
  const char* dO;
  const float* lse;   // Hq x S, natural log of each query's softmax denominator
  float* stat;        // (head, query type): n_pad pairs (log2-domain lse, D), then 64 spare pairs
  char* dQ;
  char* dK;
  char* dV;
  float* part;        // hsplit > 1: fp32 dK, dV of each head share, hsplit x 2 x Hkv x S x d
  int Hq, Hkv, S, q, L, m, o;
  int n_qblk;         // 128-query blocks per (head, type)
  int n_kblk;         // 128-key blocks per (key/value head, type)
  int n_pad;          // pairs per (head, type): ceil(S / q) rounded up to 64
  int hsplit;         // workgroups sharing a key block's query heads (1 or 2)
};

// Transposing-read offsets for a 16-row step of swb rows: lane (g = lane / 16,
// t = lane % 16) reads 8 bytes of rows k_l and k_l + 4 of the step, k_l =
// 8 (g / 2) + t / 4, logical piece 4 db + 2 (g % 2) + (t % 4) / 2, half t % 2
// (the forward's V read, with the swb swizzle, which within a step of 16 rows
// does not depend on the step).
template <int D>
__device__ __forceinline__ void tr_offsets(int lane, int (&lo)[D / 32], int (&hi)[D / 32]) {
  constexpr int ROWB = D * 2;
  const int g = lane >> 4, t = lane & 15;
  const int k_l = 8 * (g >> 1) + (t >> 2);
  const int r2 = 2 * (g & 1) + ((t & 3) >> 1);
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    lo[db] = k_l * ROWB + (((4 * db + r2) ^ swb<D>(k_l)) << 4) + 8 * (t & 1);
    hi[db] = (k_l + 4) * ROWB + (((4 * db + r2) ^ swb<D>(k_l + 4)) << 4) + 8 * (t & 1);
  }
}

// A operand (32 features x 16 rows) of feature block db, row step st, from swb rows
template <int D>
__device__ __forceinline__ bf16x8 read_tr(const char* base, int st, int lo, int hi) {
  const char* p = base + st * 16 * (D * 2);
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p + lo));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p + hi));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// A operand (32 rows x 16 features) from swb rows: row r, logical piece pc
template <int D>
__device__ __forceinline__ bf16x8 read_row(const char* base, int r, int pc) {
  return *reinterpret_cast<const bf16x8*>(base + r * (D * 2) + ((pc ^ swb<D>(r)) << 4));
}

// rows 16 ks .. 16 ks + 15 of a 64-row tile of fp32 results (two 32x32 MFMA
// outputs, rows in registers) as a bf16 B operand with those rows as the
// contraction: the forward's probability exchange (v_permlane32_swap)
template <int KS4>
__device__ __forceinline__ bf16x8 pack_rows(const f32x16 (&x)[2]) {
  constexpr int nb = KS4 >> 1, ga = 2 * (KS4 & 1);
  const u32x2 pa = pack4_bf16(x[nb][4 * ga], x[nb][4 * ga + 1], x[nb][4 * ga + 2], x[nb][4 * ga + 3]);
  const u32x2 pb = pack4_bf16(x[nb][4 * ga + 4], x[nb][4 * ga + 5], x[nb][4 * ga + 6], x[nb][4 * ga + 7]);
  const auto s0 = __builtin_amdgcn_permlane32_swap(pa[0], pb[0], false, false);
  const auto s1 = __builtin_amdgcn_permlane32_swap(pa[1], pb[1], false, false);
  const u32x4 w = {s0[0], s1[0], s0[1], s1[1]};
  return __builtin_bit_cast(bf16x8, w);
}

// the support of types (i, j) as MFMA slots: slot x is the x-th 16-feature
// step of F(i, j) (piece 2 step + lhi of a row; its B fragment is loaded again
// from the lane's own row in global memory when the pair of types changes,
// which is rarer than a register select over all d / 16 fragments is cheap);
// per 32-feature block, whether it meets F(i, j) (uniform) and whether this
// lane's feature (32 db + l32) lies in it
template <int D>
struct BwdSupport {
  int tot, nf;
  int kp[D / 16];
  bf16x8 sl[D / 16];
  bool blk[D / 32], lane_in[D / 32];
  // row: the lane's row in global memory, advanced by 16 lhi bytes
  __device__ __forceinline__ void set(int i, int j, int L, int m, int l32, const char* row) {
    constexpr int KS = D / 16;
    const int ms = m / 16;
    nf = uni(support_count(i, j, L));
    tot = uni(nf * ms);
#pragma unroll
    for (int x = 0; x < KS; ++x) {
      const int step = x < tot ? support_group(i, j, L, x / ms) * ms + x % ms : 0;
      kp[x] = uni(2 * step);
      sl[x] = *reinterpret_cast<const bf16x8*>(row + 32 * step);
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      blk[db] = in_support(32 * db / m, i, j, L) || in_support((32 * db + 31) / m, i, j, L);
      lane_in[db] = in_support((32 * db + l32) / m, i, j, L);
    }
  }
};

// sc[nb] (rows nb * 32 + 8 (e / 4) + 4 lhi + e % 4, column = lane) = rows of
// `base` times the support slots
template <int D, int T>
__device__ __forceinline__ void support_scores(f32x16 (&sc)[2], const char* base, const BwdSupport<D>& sp, int l32,
                                               int lhi) {
  sc[0] = (f32x16){};
  sc[1] = (f32x16){};
#pragma unroll
  for (int x = 0; x < T; ++x)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
      sc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_row<D>(base, nb * 32 + l32, sp.kp[x] + lhi), sp.sl[x],
                                                       sc[nb], 0, 0, 0);
}
template <int D>
__device__ __forceinline__ void support_scores_any(f32x16 (&sc)[2], const char* base, const BwdSupport<D>& sp,
                                                   int l32, int lhi) {
  switch (sp.tot) {
    case 1: support_scores<D, 1>(sc, base, sp, l32, lhi); break;
    case 2: support_scores<D, 2>(sc, base, sp, l32, lhi); break;
    case 3: support_scores<D, 3>(sc, base, sp, l32, lhi); break;
    case 4: support_scores<D, 4>(sc, base, sp, l32, lhi); break;
    case 5: support_scores<D, 5>(sc, base, sp, l32, lhi); break;
    case 6: support_scores<D, 6>(sc, base, sp, l32, lhi); break;
    case 7: support_scores<D, 7>(sc, base, sp, l32, lhi); break;
    default: support_scores<D, D / 16>(sc, base, sp, l32, lhi); break;
  }
}

// dp[nb] = rows of `base` (all d features) times the lane's fragments f
template <int D>
__device__ __forceinline__ void full_scores(f32x16 (&dp)[2], const char* base, const bf16x8 (&f)[D / 16], int l32,
                                            int lhi) {
  dp[0] = (f32x16){};
  dp[1] = (f32x16){};
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
      dp[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_row<D>(base, nb * 32 + l32, 2 * ks + lhi), f[ks], dp[nb],
                                                       0, 0, 0);
}

// acc[db] += (feature block db of the 64 swb rows at `base`, transposed) x
// (x's rows as the contraction); with MASK only the blocks and lanes of F
template <int D, bool MASK>
__device__ __forceinline__ void accumulate_tr(f32x16 (&acc)[D / 32], const char* base, const f32x16 (&x)[2],
                                              const int (&lo)[D / 32], const int (&hi)[D / 32],
                                              const BwdSupport<D>& sp) {
  auto step = [&](auto ks_c) {
    constexpr int KS4 = decltype(ks_c)::value;
    const bf16x8 b = pack_rows<KS4>(x);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      if (MASK && !sp.blk[db]) continue;
      bf16x8 a = read_tr<D>(base, KS4, lo[db], hi[db]);
      if (MASK && !sp.lane_in[db]) a = (bf16x8){};
      acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[db], 0, 0, 0);
    }
  };
  step(std::integral_constant<int, 0>{});
  step(std::integral_constant<int, 1>{});
  step(std::integral_constant<int, 2>{});
  step(std::integral_constant<int, 3>{});
}

// a lane's row of a 32-row result: features 32 db + 8 g + 4 lhi + 0..3 of row `row`
template <int D>
__device__ __forceinline__ void store_row(char* row, const f32x16 (&acc)[D / 32], int lhi) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<u32x2*>(row + (32 * db + 8 * g + 4 * lhi) * 2) =
          pack4_bf16(acc[db][4 * g], acc[db][4 * g + 1], acc[db][4 * g + 2], acc[db][4 * g + 3]);
}

template <int D>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_bwd_dq_kernel(AttnBwdArgs a) {
  constexpr int ROWB = D * 2;
  constexpr int NP = D / 8;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int BLK = kAttnK * ROWB;
  constexpr int LOADS = BLK / (4 * 1024);
  static_assert(BLK % 4096 == 0, "whole 1 KB copies per wave");
  // two stages of [K block | V block], both in the swb layout
  __shared__ __attribute__((aligned(1024))) char smem[2 * 2 * BLK];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, lhi = lane >> 5;
  int bid = blockIdx.x;
  const int qb = a.n_qblk - 1 - bid % a.n_qblk;  // late (heavy) query blocks first
  bid /= a.n_qblk;
  const int i = bid % a.q;
  const int h = bid / a.q;
  const int kvh = h / (a.Hq / a.Hkv);
  const int q = a.q, S = a.S;
  auto first_row = [&](int t) -> int { return t >= a.o ? t - a.o : t - a.o + q; };
  const int si = first_row(i);
  const int n_i = S > si ? (S - si + q - 1) / q : 0;
  const int t0 = qb * kAttnQ;
  if (t0 >= n_i) return;
  const int t_last = min(t0 + kAttnQ, n_i) - 1;
  const int p_last = si + q * t_last;
  const int p_wave0 = si + q * min(t0 + 32 * wid, n_i - 1);

  const int64_t hoff = int64_t(h) * S * ROWB;
  const char* Kh = a.K + int64_t(kvh) * S * ROWB;
  const char* Vh = a.V + int64_t(kvh) * S * ROWB;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>(smem)));

  // this lane's query row: dO fragments in registers (Q's are read per key
  // type, for the support's groups only); D = <dO, O> in fp32
  const int tq = t0 + wid * 32 + l32;
  const bool q_ok = tq < n_i;
  const int tqc = min(tq, n_i - 1);
  const int pq = si + q * tqc;
  bf16x8 df[KS];
  float dsum = 0.f;
  const char* q_row = a.Q + hoff + int64_t(pq) * ROWB + 16 * lhi;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int64_t off = hoff + int64_t(pq) * ROWB + (2 * ks + lhi) * 16;
    df[ks] = *reinterpret_cast<const bf16x8*>(a.dO + off);
    const bf16x8 of = *reinterpret_cast<const bf16x8*>(a.O + off);
#pragma unroll
    for (int e = 0; e < 8; ++e) dsum = __builtin_fmaf(float(df[ks][e]), float(of[e]), dsum);
  }
  dsum += __shfl_xor(dsum, 32);
  const float log2e = 1.4426950408889634f;
  const float lse2 = a.lse[int64_t(h) * S + pq] * log2e;
  if (q_ok && lhi == 0) {
    float* st = a.stat + 2 * (int64_t(h * q + i) * a.n_pad + tq);
    st[0] = lse2;
    st[1] = dsum;
  }

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = (f32x16){};
  int tlo[DB], thi[DB];
  tr_offsets<D>(lane, tlo, thi);
  // copy slots: slot x is row k_row0 + x (64 / NP) of the block, at byte
  // x of k_pcs (the piece's swizzled byte offset, < 256): two registers in
  // all, which keeps this kernel within two workgroups' register budget
  static_assert(LOADS <= 4 && 64 % NP == 0 && NP * 16 <= 256, "packed copy slots");
  const int k_row0 = (wid * LOADS * 64 + lane) / NP;
  uint32_t k_pcs = 0;
#pragma unroll
  for (int x = 0; x < LOADS; ++x)
    k_pcs |= uint32_t(((lane % NP) ^ swb<D>(k_row0 + x * (64 / NP))) * 16) << (8 * x);

  // key blocks, type by type (the forward's walk)
  int cj = 0, ct = 0;
  auto keys_of = [&](int j) -> int {
    const int sj = first_row(j);
    return p_last >= sj ? (p_last - sj) / q + 1 : 0;
  };
  auto skip_empty = [&]() {
    while (cj < q && ct >= keys_of(cj)) {
      cj = uni(cj + 1);
      ct = 0;
    }
  };
  auto issue = [&](int stage) {
    const int nk = keys_of(cj);
    const uint32_t base = lds0 + uint32_t(stage * 2 * BLK) + uint32_t(wid * LOADS * 1024);
    // the slots are re-derived here at each block (the empty asm hides that
    // they do not change), so the compiler cannot hoist LOADS copies of them
    // out of the loop and spill those
    int r0 = k_row0;
    uint32_t pcs = k_pcs;
    asm volatile("" : "+v"(r0), "+v"(pcs));
#pragma unroll
    for (int x = 0; x < LOADS; ++x) {
      const uint32_t u = uint32_t(first_row(cj) + q * min(ct + r0 + x * (64 / NP), nk - 1));
      const uint32_t off = u * ROWB + ((pcs >> (8 * x)) & 255u);
      copy16_to_lds(Kh, off, base + uint32_t(x * 1024));
      copy16_to_lds(Vh, off, base + uint32_t(BLK + x * 1024));
    }
  };

  BwdSupport<D> sp;
  int cur_j = -1;
  skip_empty();
  int stage = 0;
  int bj = cj, btb = ct;
  issue(0);
  ct = uni(ct + kAttnK);
  skip_empty();
  for (;;) {
    wait_vmcnt<0>();
    lds_barrier();
    const int j = bj, tb = btb;
    const bool more = cj < q;
    // a new key type's query slots are loaded and waited for before the next
    // block's copies are issued, so that no later wait stalls on the copies
    if (j != cur_j) {
      cur_j = j;
      sp.set(i, j, a.L, a.m, l32, q_row);
      wait_vmcnt<0>();
    }
    if (more) {
      bj = cj;
      btb = ct;
      issue(stage ^ 1);
      ct = uni(ct + kAttnK);
      skip_empty();
    }
    const char* sK = smem + stage * 2 * BLK;
    const char* sV = sK + BLK;
    f32x16 sc[2], dp[2];
    support_scores_any<D>(sc, sK, sp, l32, lhi);
    full_scores<D>(dp, sV, df, l32, lhi);
    const float c = __builtin_amdgcn_rsqf(float(sp.nf * a.m));
    const float scl = log2e * c;
    const int nk_j = keys_of(j);
    const int sj = first_row(j);
    const bool full = tb + kAttnK <= nk_j && sj + q * (tb + kAttnK - 1) <= p_wave0;
    // dS = P (dP - D) c; a block wholly inside every query's causal range
    // (the usual case) takes the branch without the mask
    // allowed keys: tk <= tqc - [si < sj] (the forward's causal test)
    const int lim = tqc - (si < sj ? 1 : 0) - tb - 4 * lhi;
    auto ds_pass = [&](auto full_c) {
      constexpr bool FULL = decltype(full_c)::value;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[nb][e], scl, -lse2));
          const float v = p * (dp[nb][e] - dsum) * c;
          if constexpr (FULL) {
            dp[nb][e] = v;
          } else {
            dp[nb][e] = nb * 32 + 8 * (e >> 2) + (e & 3) <= lim ? v : 0.f;
          }
        }
    };
    if (full)
      ds_pass(std::true_type{});
    else
      ds_pass(std::false_type{});
    accumulate_tr<D, true>(acc, sK, dp, tlo, thi, sp);
    if (!more) break;
    stage ^= 1;
  }
  if (q_ok) store_row<D>(a.dQ + hoff + int64_t(pq) * ROWB, acc, lhi);
}

template <int D>
__global__ __launch_bounds__(kAttnThreads, 1) void attn_bwd_dkdv_kernel(AttnBwdArgs a) {
  constexpr int ROWB = D * 2;
  constexpr int NP = D / 8;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int BLK = kAttnK * ROWB;     // 64 query rows
  constexpr int LOADS = BLK / (4 * 1024);
  constexpr int STG = 2 * BLK + 1024;    // [Q block | dO block | 64 (lse, D) pairs + pad]
  static_assert(BLK % 4096 == 0, "whole 1 KB copies per wave");
  __shared__ __attribute__((aligned(1024))) char smem[2 * STG];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, lhi = lane >> 5;
  const int q = a.q, S = a.S;
  // block -> (key block, key type, key/value head, share of the query heads),
  // early (heavy) key blocks first
  int bid = blockIdx.x;
  const int per_kb = q * a.Hkv * a.hsplit;
  const int kb = bid / per_kb;
  bid -= kb * per_kb;
  const int hp = bid % a.hsplit;
  bid /= a.hsplit;
  const int j = bid % q;
  const int hk = bid / q;
  const int Gall = a.Hq / a.Hkv;
  const int G = Gall / a.hsplit;      // query heads of this share: hk Gall + hp G + 0 .. G - 1
  auto first_row = [&](int t) -> int { return t >= a.o ? t - a.o : t - a.o + q; };
  auto n_of = [&](int t) -> int {
    const int s_ = first_row(t);
    return S > s_ ? (S - s_ + q - 1) / q : 0;
  };
  const int sj = first_row(j);
  const int n_j = n_of(j);
  const int t0 = kb * kAttnQ;
  if (t0 >= n_j) return;
  const int p_first = sj + q * t0;
  const int p_wave_last = sj + q * min(t0 + 32 * wid + 31, n_j - 1);

  // this lane's key: V fragments in registers (K's are read per query type,
  // for the support's groups only)
  const int tk = t0 + wid * 32 + l32;
  const bool k_ok = tk < n_j;
  const int tkc = min(tk, n_j - 1);
  const int pk = sj + q * tkc;
  const int64_t koff = int64_t(hk) * S * ROWB + int64_t(pk) * ROWB;
  bf16x8 vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) vf[ks] = *reinterpret_cast<const bf16x8*>(a.V + koff + (2 * ks + lhi) * 16);
  const char* k_row = a.K + koff + 16 * lhi;
  f32x16 accK[DB], accV[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    accK[db] = (f32x16){};
    accV[db] = (f32x16){};
  }
  int tlo[DB], thi[DB];
  tr_offsets<D>(lane, tlo, thi);
  int r_row[LOADS];
  uint32_t r_pc[LOADS];
#pragma unroll
  for (int x = 0; x < LOADS; ++x) {
    const int sl = (wid * LOADS + x) * 64 + lane;
    r_row[x] = sl / NP;
    r_pc[x] = uint32_t((sl % NP) ^ swb<D>(r_row[x])) * 16u;
  }
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>(smem)));

  // query blocks: for each query head of the group and each query type, the
  // queries from the first one at or after p_first (an even index, so that the
  // block's (lse, D) pairs start 16-byte aligned), 64 at a time
  auto q_first = [&](int t) -> int {
    const int s_ = first_row(t);
    return (p_first > s_ ? (p_first - s_ + q - 1) / q : 0) & ~1;
  };
  int cg = 0, ci = 0, ct = q_first(0);
  auto skip_empty = [&]() {
    while (cg < G && ct >= n_of(ci)) {
      ci = uni(ci + 1);
      if (ci == q) {
        ci = 0;
        cg = uni(cg + 1);
      }
      ct = uni(q_first(ci));
    }
  };
  auto issue = [&](int stage) {
    const int h = hk * Gall + hp * G + cg;
    const int n = n_of(ci), s_ = first_row(ci);
    const char* Qh = a.Q + int64_t(h) * S * ROWB;
    const char* dOh = a.dO + int64_t(h) * S * ROWB;
    const uint32_t base = lds0 + uint32_t(stage * STG) + uint32_t(wid * LOADS * 1024);
#pragma unroll
    for (int x = 0; x < LOADS; ++x) {
      const uint32_t u = uint32_t(s_ + q * min(ct + r_row[x], n - 1));
      copy16_to_lds(Qh, u * ROWB + r_pc[x], base + uint32_t(x * 1024));
      copy16_to_lds(dOh, u * ROWB + r_pc[x], base + uint32_t(BLK + x * 1024));
    }
    if (wid == 0) {
      // 64 pairs = 512 bytes: lanes 0-31; lanes 32-63 repeat them into the pad
      const char* st = reinterpret_cast<const char*>(a.stat + 2 * (int64_t(h * q + ci) * a.n_pad + ct));
      copy16_to_lds(st, uint32_t(lane & 31) * 16u, lds0 + uint32_t(stage * STG + 2 * BLK));
    }
  };

  const float log2e = 1.4426950408889634f;
  BwdSupport<D> sp;
  int cur_i = -1;
  skip_empty();
  int stage = 0;
  int bi = ci, btb = ct;
  issue(0);
  ct = uni(ct + kAttnK);
  skip_empty();
  for (;;) {
    wait_vmcnt<0>();
    lds_barrier();
    const int i = bi, tb = btb;
    const bool more = cg < G;
    // a new query type's key slots: loaded and waited for before the next
    // block's copies are issued (see the dQ kernel)
    if (i != cur_i) {
      cur_i = i;
      sp.set(i, j, a.L, a.m, l32, k_row);
      wait_vmcnt<0>();
    }
    if (more) {
      bi = ci;
      btb = ct;
      issue(stage ^ 1);
      ct = uni(ct + kAttnK);
      skip_empty();
    }
    const char* sQ = smem + stage * STG;
    const char* sdO = sQ + BLK;
    const char* sst = sdO + BLK;
    f32x16 sc[2], dp[2];
    support_scores_any<D>(sc, sQ, sp, l32, lhi);
    full_scores<D>(dp, sdO, vf, l32, lhi);
    const float c = __builtin_amdgcn_rsqf(float(sp.nf * a.m));
    const float scl = log2e * c;
    const int n_i = n_of(i), s_i = first_row(i);
    const bool full = tb + kAttnK <= n_i && s_i + q * tb >= p_wave_last;
    // P and dS = P (dP - D) c; masked pairs (and the rows past the type's
    // last query, whose pairs hold other data) are set to 0 by selects
    // allowed queries of the block: s_i + q tq >= pk = sj + q tkc, i.e. (both
    // first rows in [0, q)) tq >= tkc + [sj > s_i], and tq < n_i; as one
    // unsigned range test on the element's constant offset c: c - lo in [0, rg]
    int lo = tkc + (sj > s_i ? 1 : 0) - tb - 4 * lhi, rg = n_i - 1 - tb - 4 * lhi - lo;
    if (rg < 0) {
      lo = 1 << 20;
      rg = 0;
    }
    auto pds_pass = [&](auto full_c) {
      constexpr bool FULL = decltype(full_c)::value;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int r0 = nb * 32 + 8 * g4 + 4 * lhi;  // the lane's 4 consecutive queries
          const float4 w0 = *reinterpret_cast<const float4*>(sst + 8 * r0);
          const float4 w1 = *reinterpret_cast<const float4*>(sst + 8 * r0 + 16);
          const float ls[4] = {w0.x, w0.z, w1.x, w1.z};
          const float dd[4] = {w0.y, w0.w, w1.y, w1.w};
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) {
            const int e = 4 * g4 + e4;
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[nb][e], scl, -ls[e4]));
            const float v = p * (dp[nb][e] - dd[e4]) * c;
            if constexpr (FULL) {
              dp[nb][e] = v;
              sc[nb][e] = p;
            } else {
              const bool ok = uint32_t(nb * 32 + 8 * g4 + e4 - lo) <= uint32_t(rg);
              dp[nb][e] = ok ? v : 0.f;
              sc[nb][e] = ok ? p : 0.f;
            }
          }
        }
    };
    if (full)
      pds_pass(std::true_type{});
    else
      pds_pass(std::false_type{});
    accumulate_tr<D, false>(accV, sdO, sc, tlo, thi, sp);
    accumulate_tr<D, true>(accK, sQ, dp, tlo, thi, sp);
    if (!more) break;
    stage ^= 1;
  }
  if (!k_ok) return;
  if (a.hsplit == 1) {
    store_row<D>(a.dK + koff, accK, lhi);
    store_row<D>(a.dV + koff, accV, lhi);
    return;
  }
  // this share's sums in fp32; attn_bwd_reduce_kernel adds the shares in order
  const int64_t rows = int64_t(a.Hkv) * S;
  float* pk_row = a.part + ((int64_t(hp) * 2) * rows + int64_t(hk) * S + pk) * D;
  float* pv_row = pk_row + rows * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int f = 32 * db + 8 * g + 4 * lhi;
      *reinterpret_cast<float4*>(pk_row + f) =
          make_float4(accK[db][4 * g], accK[db][4 * g + 1], accK[db][4 * g + 2], accK[db][4 * g + 3]);
      *reinterpret_cast<float4*>(pv_row + f) =
          make_float4(accV[db][4 * g], accV[db][4 * g + 1], accV[db][4 * g + 2], accV[db][4 * g + 3]);
    }
}

// dK and dV from the head shares' fp32 sums, added in share order (one
// rounding; the result does not depend on scheduling): 8 features per thread
__global__ __launch_bounds__(256) void attn_bwd_reduce_kernel(const float* __restrict__ part, int hsplit,
                                                              int64_t n, char* __restrict__ dK,
                                                              char* __restrict__ dV) {
  const int64_t x = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 8;
  if (x >= 2 * n) return;
  const bool is_v = x >= n;
  const int64_t e = is_v ? x - n : x;
  float v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = 0.f;
  for (int p = 0; p < hsplit; ++p) {
    const float* src = part + int64_t(p) * 2 * n + x;
    const float4 lo = *reinterpret_cast<const float4*>(src);
    const float4 hi = *reinterpret_cast<const float4*>(src + 4);
    v[0] += lo.x;
    v[1] += lo.y;
    v[2] += lo.z;
    v[3] += lo.w;
    v[4] += hi.x;
    v[5] += hi.y;
    v[6] += hi.z;
    v[7] += hi.w;
  }
  const u32x2 a0 = pack4_bf16(v[0], v[1], v[2], v[3]);
  const u32x2 a1 = pack4_bf16(v[4], v[5], v[6], v[7]);
  *reinterpret_cast<u32x4*>((is_v ? dV : dK) + e * 2) = (u32x4){a0[0], a0[1], a1[0], a1[1]};
}

}  // namespace

bool attn_supported(int d, int q) { return (d == 64 || d == 128) && q >= 1 && d % q == 0 && (d / q) % 16 == 0; }

hipError_t launch_attn_fwd_lse_bf16(const void* Q, const void* K, const void* V, void* O, float* lse, int Hq,
                                    int Hkv, int64_t S, int d, int q, int L, int64_t first_pos, hipStream_t s) {
  AttnArgs a;
  a.Q = static_cast<const char*>(Q);
  a.K = static_cast<const char*>(K);
  a.V = static_cast<const char*>(V);
  a.O = static_cast<char*>(O);
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.S = int(S);
  a.q = q;
  a.L = L;
  a.m = d / q;
  a.o = int(first_pos % q);
  a.lse = lse;
  const int64_t n0 = (S + q - 1) / q;  // queries of the most frequent type
  a.n_qblk = int((n0 + kAttnQ - 1) / kAttnQ);
  const int64_t blocks = int64_t(Hq) * q * a.n_qblk;
  if (blocks == 0) return hipSuccess;
  if (d == 128)
    hipLaunchKernelGGL(attn_fwd_kernel<128>, dim3(unsigned(blocks)), dim3(kAttnThreads), 0, s, a);
  else
    hipLaunchKernelGGL(attn_fwd_kernel<64>, dim3(unsigned(blocks)), dim3(kAttnThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attn_fwd_bf16(const void* Q, const void* K, const void* V, void* O, int Hq, int Hkv, int64_t S,
                                int d, int q, int L, int64_t first_pos, hipStream_t s) {
  return launch_attn_fwd_lse_bf16(Q, K, V, O, nullptr, Hq, Hkv, S, d, q, L, first_pos, s);
}

size_t attn_bwd_stat_bytes(int64_t Hq, int64_t S, int q) {
  const int64_t n0 = (S + q - 1) / q;
  const int64_t n_pad = (n0 + 63) / 64 * 64;
  return size_t((Hq * q * n_pad + 64) * 2) * sizeof(float);
}

// Query heads per key/value head split over two workgroups when there are an
// even number of them: the earliest keys of a causal sequence see every query
// and the latest few, so with one workgroup per key block the first blocks
// would set the kernel's length; two shares of the heads halve the longest
// workgroups and give the scheduler twice the blocks to balance.
int attn_bwd_hsplit(int Hq, int Hkv) { return (Hq / Hkv) % 2 == 0 ? 2 : 1; }

size_t attn_bwd_ws_bytes(int64_t Hq, int64_t Hkv, int64_t S, int d, int q) {
  const size_t stat = (attn_bwd_stat_bytes(Hq, S, q) + 255) / 256 * 256;
  const int hs = attn_bwd_hsplit(int(Hq), int(Hkv));
  const size_t part = hs > 1 ? size_t(hs) * 2 * size_t(Hkv) * size_t(S) * size_t(d) * sizeof(float) : 0;
  return stat + part;
}

hipError_t launch_attn_bwd_bf16(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                                const float* lse, void* dQ, void* dK, void* dV, void* stat, int Hq, int Hkv,
                                int64_t S, int d, int q, int L, int64_t first_pos, hipStream_t s) {
  AttnBwdArgs a;
  a.Q = static_cast<const char*>(Q);
  a.K = static_cast<const char*>(K);
  a.V = static_cast<const char*>(V);
  a.O = static_cast<const char*>(O);
  a.dO = static_cast<const char*>(dO);
  a.lse = lse;
  a.stat = static_cast<float*>(stat);
  a.hsplit = attn_bwd_hsplit(Hq, Hkv);
  a.part = a.hsplit > 1 ? reinterpret_cast<float*>(static_cast<char*>(stat) +
                                                   (attn_bwd_stat_bytes(Hq, S, q) + 255) / 256 * 256)
                        : nullptr;
  a.dQ = static_cast<char*>(dQ);
  a.dK = static_cast<char*>(dK);
  a.dV = static_cast<char*>(dV);
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.S = int(S);
  a.q = q;
  a.L = L;
  a.m = d / q;
  a.o = int(first_pos % q);
  const int64_t n0 = (S + q - 1) / q;
  a.n_qblk = int((n0 + kAttnQ - 1) / kAttnQ);
  a.n_kblk = a.n_qblk;
  a.n_pad = int((n0 + 63) / 64 * 64);
  const int64_t qblocks = int64_t(Hq) * q * a.n_qblk;
  const int64_t kblocks = int64_t(Hkv) * q * a.n_kblk * a.hsplit;
  if (qblocks == 0) return hipSuccess;
  // dQ first: it also writes the (lse, D) pairs the dK / dV kernel reads
  if (d == 128) {
    hipLaunchKernelGGL(attn_bwd_dq_kernel<128>, dim3(unsigned(qblocks)), dim3(kAttnThreads), 0, s, a);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<128>, dim3(unsigned(kblocks)), dim3(kAttnThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL(attn_bwd_dq_kernel<64>, dim3(unsigned(qblocks)), dim3(kAttnThreads), 0, s, a);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<64>, dim3(unsigned(kblocks)), dim3(kAttnThreads), 0, s, a);
  }
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  if (a.hsplit > 1) {
    const int64_t n = int64_t(Hkv) * S * d;  // elements of dK (and of dV)
    const int64_t threads = 2 * n / 8;
    hipLaunchKernelGGL(attn_bwd_reduce_kernel, dim3(unsigned((threads + 255) / 256)), dim3(256), 0, s, a.part,
                       a.hsplit, n, a.dK, a.dV);
  }
  return hipGetLastError();
}

bool attn_decode_supported(int d, int q) { return (d == 64 || d == 128) && q >= 1 && d % q == 0 && (d / q) % 8 == 0; }

int64_t attn_decode_max_slots() { return int64_t(kDecCh) * kDecMaxChunks; }

size_t attn_decode_part_bytes(int64_t B, int64_t Hq, int64_t N, int d) {
  const int64_t chunks = (N + kDecCh - 1) / kDecCh;
  return size_t(B * Hq * chunks * (d + 4)) * sizeof(float);
}

hipError_t launch_attn_decode_bf16(const void* Q, const void* K, const void* V, const int64_t* q_pos,
                                   const int64_t* key_pos, void* O, int B, int Hq, int Hkv, int64_t N, int d, int q,
                                   int L, int kind, int64_t period, void* part, hipStream_t s) {
  DecArgs a;
  a.Q = static_cast<const char*>(Q);
  a.K = static_cast<const char*>(K);
  a.V = static_cast<const char*>(V);
  a.q_pos = q_pos;
  a.key_pos = key_pos;
  a.part = static_cast<float*>(part);
  a.O = static_cast<char*>(O);
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.q = q;
  a.L = L;
  a.m = d / q;
  a.kind = kind;
  a.period = period;
  a.N = N;
  a.chunks = int((N + kDecCh - 1) / kDecCh);
  const dim3 grid(unsigned(a.chunks), unsigned(Hkv), unsigned(B));
  const int gm = a.G <= 1 ? 1 : a.G <= 2 ? 2 : a.G <= 4 ? 4 : 8;
  auto run = [&](auto d_c, auto g_c) {
    constexpr int DD = decltype(d_c)::value, GG = decltype(g_c)::value;
    hipLaunchKernelGGL((attn_decode_kernel<DD, GG>), grid, dim3(kDecThreads), 0, s, a);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    hipLaunchKernelGGL(attn_decode_combine_kernel<DD>, dim3(unsigned(B * Hq)), dim3(DD), 0, s, a.part, a.chunks, a.O);
    return hipGetLastError();
  };
  using I128 = std::integral_constant<int, 128>;
  using I64 = std::integral_constant<int, 64>;
  using G1 = std::integral_constant<int, 1>;
  using G2 = std::integral_constant<int, 2>;
  using G4 = std::integral_constant<int, 4>;
  using G8 = std::integral_constant<int, 8>;
  if (d == 128) {
    if (gm == 1) return run(I128{}, G1{});
    if (gm == 2) return run(I128{}, G2{});
    if (gm == 4) return run(I128{}, G4{});
    return run(I128{}, G8{});
  }
  if (gm == 1) return run(I64{}, G1{});
  if (gm == 2) return run(I64{}, G2{});
  if (gm == 4) return run(I64{}, G4{});
  return run(I64{}, G8{});
}

}  // namespace qalg
