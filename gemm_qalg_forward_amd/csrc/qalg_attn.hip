// Causal attention with the algebraic score (arXiv 2609.32814, appendix G),
// forward, bf16 in and out, fp32 softmax statistics and accumulation.
//
// A query at position p (type i = p mod q) and a key at u (type j) compare only
// the feature groups F(i, j) of the head: {i} if i == j, else {i, j} (eq 38;
// eq 42 for the recursive law Q_2^(x)L: every group whose bits each come from i
// or j).  The score r_pu (eq 39) is scaled by 1/sqrt(|F| m), m = d / q (eq 41),
// masked to u <= p (eq 43), softmaxed, and the values are aggregated densely
// (eq 44).  Algorithm 2, steps 3-7, for one sequence per head.
//
// Work.  A workgroup owns 128 queries of one type i of one head (positions
// i + q t for 128 consecutive t), 32 per wave, and walks the keys type by type:
// keys of type j are the positions j + q t', so a block of 64 of them shares
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
  const int n_i = S > i ? (S - i + q - 1) / q : 0;  // queries of type i
  const int t0 = qb * kAttnQ;
  if (t0 >= n_i) return;
  const int t_last = min(t0 + kAttnQ, n_i) - 1;
  const int p_last = i + q * t_last;                // latest query position in the block
  const int p_wave0 = i + q * min(t0 + 32 * wid, n_i - 1);  // earliest query position of the wave

  const char* Qh = a.Q + int64_t(h) * S * ROWB;
  const char* Kh = a.K + int64_t(kvh) * S * ROWB;
  const char* Vh = a.V + int64_t(kvh) * S * ROWB;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>(smem)));

  // this lane's query row (row l32 of the wave's 32): its fragments stay in registers
  const int tq = t0 + wid * 32 + l32;
  const bool q_ok = tq < n_i;
  const int pq = i + q * min(tq, n_i - 1);
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qf[ks] = *reinterpret_cast<const bf16x8*>(Qh + int64_t(pq) * ROWB + (2 * ks + lhi) * 16);

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
    // keys of type j that some query of the block may see: u = j + q t' <= p_last < S
    return p_last >= j ? (p_last - j) / q + 1 : 0;
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
      const uint32_t u = uint32_t(cj + q * min(ct + k_row[x], nk - 1));
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
    if (more) {
      bj = cj;
      btb = ct;
      issue(stage ^ 1);
      ct = uni(ct + kAttnK);
      skip_empty();
    }
    const char* sK = smem + stage * 2 * BLK;
    const char* sV = sK + BLK;

    // scores of the wave's 32 queries against the 64 keys over the support's
    // groups only.  When the key type changes, the support's k-steps are laid
    // out as slots: slot x holds the query fragment and the K piece of the
    // x-th 16-feature step of F(i, j); the block then runs exactly `tot`
    // MFMA steps per 32-key tile, through a switch on tot, so that no MFMA is
    // conditional inside straight-line code.
    if (j != cur_j) {
      cur_j = j;
      const int ms = a.m / 16;
      tot = uni(support_count(i, j, a.L) * ms);
#pragma unroll
      for (int x = 0; x < KS; ++x) {
        const int step = x < tot ? support_group(i, j, a.L, x / ms) * ms + x % ms : 0;
        kp[x] = uni(2 * step);
        bf16x8 v = qf[0];
#pragma unroll
        for (int z = 1; z < KS; ++z)
          if (z == step) v = qf[z];
        qsl[x] = v;
      }
    }
    f32x16 sc[2];
    auto scores = [&](auto tot_c) {
      constexpr int T = decltype(tot_c)::value;
      sc[0] = (f32x16){};
      sc[1] = (f32x16){};
#pragma unroll
      for (int x = 0; x < T; ++x) {
        const int pc = kp[x] + lhi;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int row = nb * 32 + l32;
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sK + row * ROWB + ((pc ^ swk<D>(row)) << 4));
          sc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qsl[x], sc[nb], 0, 0, 0);
        }
      }
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
    const bool full = tb + kAttnK <= nk_j && j + q * (tb + kAttnK - 1) <= p_wave0;
    if (!full) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int tk = tb + nb * 32 + 8 * (e >> 2) + 4 * lhi + (e & 3);
          if (!(tk < nk_j && j + q * tk <= pq)) sc[nb][e] = -INFINITY;
        }
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
  }
}

}  // namespace

bool attn_supported(int d, int q) { return (d == 64 || d == 128) && q >= 1 && d % q == 0 && (d / q) % 16 == 0; }

hipError_t launch_attn_fwd_bf16(const void* Q, const void* K, const void* V, void* O, int Hq, int Hkv, int64_t S,
                                int d, int q, int L, hipStream_t s) {
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
  const int64_t n0 = (S + q - 1) / q;  // queries of type 0, the most of any type
  a.n_qblk = int((n0 + kAttnQ - 1) / kAttnQ);
  const int64_t blocks = int64_t(Hq) * q * a.n_qblk;
  if (blocks == 0) return hipSuccess;
  if (d == 128)
    hipLaunchKernelGGL(attn_fwd_kernel<128>, dim3(unsigned(blocks)), dim3(kAttnThreads), 0, s, a);
  else
    hipLaunchKernelGGL(attn_fwd_kernel<64>, dim3(unsigned(blocks)), dim3(kAttnThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace qalg
