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
// over all d features (MFMA with V read transposed from LDS).  The next key
// block's K and V rows are fetched into registers while the current one is
// computed.
#include <hip/hip_runtime.h>

#include <cstdint>

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
using dev::swz_w;
using dev::uni;

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

template <int D>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_fwd_kernel(AttnArgs a) {
  constexpr int ROWB = D * 2;          // bytes per K / V row
  constexpr int NP = D / 8;            // 16-byte pieces per row
  constexpr int KS = D / 16;           // 16-feature MFMA steps over a row (2 pieces each)
  constexpr int DB = D / 32;           // 32-feature output blocks
  constexpr int LOADS = kAttnK * NP / kAttnThreads;  // 16-byte pieces per thread per block (K and V each)
  static_assert(kAttnK * NP % kAttnThreads == 0, "whole pieces per thread");
  __shared__ __attribute__((aligned(16))) char sK[kAttnK * ROWB];
  __shared__ __attribute__((aligned(16))) char sV[kAttnK * ROWB];
  __shared__ __attribute__((aligned(16))) char sQ[kAttnQ * ROWB];  // 32 rows per wave

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

  const char* Qh = a.Q + int64_t(h) * S * ROWB;
  const char* Kh = a.K + int64_t(kvh) * S * ROWB;
  const char* Vh = a.V + int64_t(kvh) * S * ROWB;

  // this lane's query row (row l32 of the wave's 32), staged in the wave's
  // share of LDS (piece c of row r at c ^ (r & 7)); a support's groups are
  // then read by feature offset
  const int tq = t0 + wid * 32 + l32;
  const bool q_ok = tq < n_i;
  const int pq = i + q * min(tq, n_i - 1);
  char* sQw = sQ + wid * 32 * ROWB;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int pc = 2 * ks + lhi;
    *reinterpret_cast<u32x4*>(sQw + l32 * ROWB + ((pc ^ (l32 & 7)) << 4)) =
        *reinterpret_cast<const u32x4*>(Qh + int64_t(pq) * ROWB + pc * 16);
  }

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = (f32x16){};
  float m_run = -INFINITY, l_run = 0.f;

  // K rows in LDS: piece c of row k at c ^ (k & 7); V rows: piece c at c ^ swz_w(k)
  // (the transposing reads below undo it)
  int v_rd[2];
  {
    const int g = lane >> 4, t = lane & 15;
    const int k_l = 8 * (g >> 1) + (t >> 2);
    const int f = swz_w(k_l);
    const int r2 = 2 * (g & 1) + ((t & 3) >> 1);
    const int lo = ((r2 ^ (f & 2)) << 4) + 8 * (t & 1) + k_l * ROWB;
    const int dm = (f >> 2) ? 64 : 0;
    v_rd[0] = lo + dm;
    v_rd[1] = lo - dm;
  }

  // key blocks, type by type: (j, first slot) in order; a cursor fetches one block ahead
  int cj = 0, ct = 0;  // cursor: key type and first slot of the next block to fetch
  auto keys_of = [&](int j) -> int {
    // keys of type j that some query of the block may see: u = j + q t' <= p_last, u < S
    return p_last >= j ? (p_last - j) / q + 1 : 0;
  };
  auto skip_empty = [&]() {
    while (cj < q && ct >= keys_of(cj)) {
      cj = uni(cj + 1);
      ct = 0;
    }
  };
  skip_empty();
  u32x4 rk[LOADS], rv[LOADS];
  int fj = 0, fct = 0;  // type and first slot of the fetched block
  auto fetch = [&]() {
    fj = cj;
    fct = ct;
    const int nk = keys_of(cj);
#pragma unroll
    for (int x = 0; x < LOADS; ++x) {
      const int sl = x * kAttnThreads + tid;
      const int row = sl / NP, c = sl - row * NP;
      const int u = cj + q * min(ct + row, nk - 1);
      rk[x] = *reinterpret_cast<const u32x4*>(Kh + int64_t(u) * ROWB + c * 16);
      rv[x] = *reinterpret_cast<const u32x4*>(Vh + int64_t(u) * ROWB + c * 16);
    }
    ct = uni(ct + kAttnK);
    skip_empty();
  };
  auto stash = [&]() {
#pragma unroll
    for (int x = 0; x < LOADS; ++x) {
      const int sl = x * kAttnThreads + tid;
      const int row = sl / NP, c = sl - row * NP;
      *reinterpret_cast<u32x4*>(sK + row * ROWB + ((c ^ (row & 7)) << 4)) = rk[x];
      *reinterpret_cast<u32x4*>(sV + row * ROWB + ((c ^ swz_w(row)) << 4)) = rv[x];
    }
  };

  const float log2e = 1.4426950408889634f;
  bool have = cj < q;
  if (have) fetch();
  while (have) {
    __syncthreads();  // the previous block's LDS reads are done
    stash();
    const int j = fj, tb = fct;
    have = cj < q;
    if (have) fetch();  // next block's rows travel while this one is computed
    __syncthreads();

    // scores of the wave's 32 queries against the 64 keys: two 32-key MFMA tiles
    f32x16 sc[2] = {(f32x16){}, (f32x16){}};
    const int nf = support_count(i, j, a.L);
    for (int b = 0; b < nf; ++b) {
      const int grp = support_group(i, j, a.L, b);
      for (int s = 0; s < a.m / 16; ++s) {
        const int ks = grp * (a.m / 16) + s;  // 16-feature step within the row
        const int pc = 2 * ks + lhi;           // this lane's piece
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int row = nb * 32 + l32;
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sK + row * ROWB + ((pc ^ (row & 7)) << 4));
          const bf16x8 qv = *reinterpret_cast<const bf16x8*>(sQw + l32 * ROWB + ((pc ^ (l32 & 7)) << 4));
          sc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qv, sc[nb], 0, 0, 0);
        }
      }
    }
    // scale (log2 domain), causal mask on positions, block row max
    const float scl = log2e * __builtin_amdgcn_rsqf(float(nf * a.m));
    const int nk_j = keys_of(j);
    float mx = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int kk = nb * 32 + 8 * (e >> 2) + 4 * lhi + (e & 3);  // key within the block
        const int tk = tb + kk;
        const int u = j + q * tk;
        const bool ok = tk < nk_j && u <= pq;
        const float v = ok ? sc[nb][e] * scl : -INFINITY;
        sc[nb][e] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float base = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - base);
    float rs = 0.f;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pv = __builtin_amdgcn_exp2f(sc[nb][e] - base);
        sc[nb][e] = pv;
        rs += pv;
      }
    rs += __shfl_xor(rs, 32);
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[db][e] *= alpha;

    // O += P V: 16 keys per step; the lane pair (l32, 0/1) exchanges half its
    // probabilities so that each lane holds 8 consecutive keys of its row
#pragma unroll
    for (int ks = 0; ks < kAttnK / 16; ++ks) {
      const int nb = ks >> 1;
      const int g_keep = 2 * (ks & 1) + lhi, g_send = 2 * (ks & 1) + (1 - lhi);
      const u32x2 own = pack4_bf16(sc[nb][4 * g_keep], sc[nb][4 * g_keep + 1], sc[nb][4 * g_keep + 2],
                                   sc[nb][4 * g_keep + 3]);
      const u32x2 snd = pack4_bf16(sc[nb][4 * g_send], sc[nb][4 * g_send + 1], sc[nb][4 * g_send + 2],
                                   sc[nb][4 * g_send + 3]);
      const unsigned r0 = __shfl_xor(snd[0], 32), r1 = __shfl_xor(snd[1], 32);
      const u32x4 pw = lhi == 0 ? (u32x4){own[0], own[1], r0, r1} : (u32x4){r0, r1, own[0], own[1]};
      const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const char* pp = sV + v_rd[db & 1] + 64 * db + 16 * ks * ROWB;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(pp));
        const s16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(pp + 4 * ROWB));
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, acc[db], 0, 0, 0);
      }
    }
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
