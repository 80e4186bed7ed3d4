// Small-M forward of the row-typed Q_q projection: a weight-streaming kernel
// for a handful of token rows per weight bank (KV-cached decode: one new row
// per sequence; tiny per-expert token counts).
//
// Paper: arXiv 2609.32814.  Section 5.2 notes that decode needs a separate
// matrix-vector implementation because the row dimension is small; section 5.3
// that the decode kernel performs vector reductions; section 6.3 and appendix G
// that single-token work is bounded by weight bandwidth.
//
// Design: weight-stationary.  A workgroup owns a chunk of 64 to 512 columns of
// one output group j of one problem.  The weight blocks that chunk needs are W_jj (every
// typed row uses it, eq 17) and W_tj for each type t != j present among the
// rows (eq 17's x_t W_tj term; W_jj alone when t == j, eq 16).  Each needed
// block is streamed from HBM exactly once, in 16-byte row pieces, and applied
// to every row that needs it; rows that do not need the block see zeros
// (staged in LDS), so the inner loop has no branches.  Blocks are visited in a
// fixed order and partial sums are reduced in a fixed tree: the result is
// bitwise reproducible.  No type index is needed: the <= 8 types are read
// directly.  The two weight rows a lane loads per step are applied together
// with bf16 dot-2 instructions on interleaved columns, against activations
// staged in LDS as the same row pairs (all needed blocks at once when they
// fit in 64 KB, else each block when the weight stream reaches it).
#include "qalg_internal.h"

namespace qalg {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kSmThreads = 256;

// wave-uniform integer quotient (both operands uniform): kept on the scalar unit
__device__ __forceinline__ int uni_div(int x, int y) {
  return __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readfirstlane(x) / __builtin_amdgcn_readfirstlane(y));
}

constexpr int kSmMaxRows = 8;
constexpr int kSmUnroll = 8;          // weight loads per thread per batch; two batches in flight
constexpr int kSmMaxXs = 16384;        // bf16 elements of one block's staged activations (32 KB)
constexpr int kSmStageAll = 32768;     // bf16 elements for staging every needed block at once (64 KB)

struct SmallArgs {
  const uint16_t* X;
  const uint16_t* W;
  const int32_t* tau;
  uint16_t* Y;
  int q, M, K, N, s, r;
  int chunks_per_group;
  int x_regions;   // staged activation regions: 1 (one block at a time) or the most blocks a chunk needs
  int xcd_order;   // 1: consecutive chunks on one XCD (column groups that are not whole cache lines)
};


// COLS output columns per workgroup: each weight row is read as COLS * 2
// contiguous bytes, 16 per lane (wider rows stream better; narrower ones give
// more workgroups)
template <int R, int COLS>
__global__ __launch_bounds__(kSmThreads) void small_m_kernel(SmallArgs a) {
  constexpr int kSmCols = COLS;
  constexpr int kSmColLanes = kSmCols / 8;             // lanes per weight row (16 bytes each)
  constexpr int kSmKLanes = kSmThreads / kSmColLanes;  // weight rows in flight per step
  static_assert(kSmColLanes <= 64 && 64 % kSmColLanes == 0, "a weight row within one wave");
  // contraction rows kk and kk + KL (KL = kSmKLanes) are the two weight rows a
  // lane applies together: the activations are staged as those pairs, u32
  // (x[kk], x[kk + KL]), and the group width is padded to whole pairs with zeros
  constexpr int KL = kSmKLanes;
  constexpr int kStep = kSmKLanes * kSmUnroll;  // weight rows of one batch (all threads)
  // the group width padded to whole batches: a batch never straddles two blocks
  const int s_pad = (a.s + kStep - 1) / kStep * kStep;
  extern __shared__ __attribute__((aligned(16))) unsigned char sm_raw[];
  uint16_t* xs16 = reinterpret_cast<uint16_t*>(sm_raw);              // [s_pad / 2][R] pairs of bf16
  const unsigned* xs2 = reinterpret_cast<const unsigned*>(sm_raw);
  const size_t x_region = size_t(s_pad) * R;  // bf16 elements of one block's staged activations
  float* red = reinterpret_cast<float*>(sm_raw + x_region * a.x_regions * 2 + 16);  // [4][R][64]
  __shared__ int s_type[R];
  __shared__ int s_blocks[R + 1];
  __shared__ int s_nblk;

  // Column groups whose rows are not whole 128-byte lines (e.g. 96 columns,
  // 192 bytes) put chunk boundaries inside cache lines.  Then workgroups are
  // renumbered so that consecutive chunks run on one XCD (workgroup w runs on
  // XCD w mod 8, w the linear id, x fastest): the chunks of a weight row meet
  // in one L2 and a line two chunks share is fetched once (2048 -> 768, q = 8,
  // one row per expert: 1.67x -> 1.17x the needed bytes, 21.9 -> 20.0 us).
  // Line-aligned groups keep the plain order, which measured 4 % faster on
  // 7168 -> 2048, q = 4.
  const int gx = gridDim.x;
  const int total = gx * gridDim.y;
  int lin = blockIdx.y * gx + blockIdx.x;
  if (a.xcd_order && (total & 7) == 0) lin = (lin & 7) * (total >> 3) + (lin >> 3);
  const int e = lin / gx;
  const int bx = lin - e * gx;
  const int j = bx / a.chunks_per_group;
  const int ch = bx - j * a.chunks_per_group;
  const int col0 = j * a.r + ch * kSmCols;
  const int ncol = min(kSmCols, a.r - ch * kSmCols);
  const int M = a.M, K = a.K, N = a.N, s = a.s, q = a.q;
  const uint16_t* X = a.X + int64_t(e) * M * K;
  const uint16_t* W = a.W + int64_t(e) * K * N;
  uint16_t* Y = a.Y + int64_t(e) * M * N;
  const int32_t* tau = a.tau + int64_t(e) * M;
  const int tid = threadIdx.x;

  if (tid < R) {
    int t = tid < M ? tau[tid] : -1;
    if (t < 0 || t >= q) t = -1;
    s_type[tid] = t;
  }
  __syncthreads();
  if (tid == 0) {
    // diagonal block first, then the source blocks of the other present types, ascending
    int n = 0;
    s_blocks[n++] = j;
    for (int m = 0; m < R; ++m) {
      const int t = s_type[m];
      if (t < 0 || t == j) continue;
      int pos = 1;
      while (pos < n && s_blocks[pos] < t) ++pos;
      if (pos < n && s_blocks[pos] == t) continue;
      for (int x = n; x > pos; --x) s_blocks[x] = s_blocks[x - 1];
      s_blocks[pos] = t;
      ++n;
    }
    s_nblk = n;
  }
  __syncthreads();

  const int l8 = tid % kSmColLanes, kr = tid / kSmColLanes;
  const bool col_on = l8 * 8 < ncol;
  float acc[R][8];
#pragma unroll
  for (int m = 0; m < R; ++m)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[m][c] = 0.f;

  const int nblk = s_nblk;
  // stage x[m, g_b] of block b into region rg as the pairs (k, k + KL) of each
  // row m, 8 contraction values (16 bytes) per load; zero for rows that do not
  // use block (b, j) and past the group width.  Value k sits in pair
  // (k / 2KL) KL + k % KL, half (k / KL) & 1.
  const int s8 = s >> 3;
  auto xs_at = [&](int k, int m) { return ((k / (2 * KL)) * KL + (k % KL)) * (R * 2) + m * 2 + ((k / KL) & 1); };
  auto stage = [&](int b, int rg) {
    uint16_t* xr16 = xs16 + rg * x_region;
    for (int x = tid; x < s8 * R; x += kSmThreads) {
      const int m = x / s8, k8 = x - m * s8;
      const int t = s_type[m];
      const bool need = t >= 0 && (b == j || t == b);
      const u32x4 v = need ? *reinterpret_cast<const u32x4*>(X + int64_t(m) * K + int64_t(b) * s + k8 * 8)
                           : (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        xr16[xs_at(k8 * 8 + 2 * d, m)] = uint16_t(v[d] & 0xffffu);
        xr16[xs_at(k8 * 8 + 2 * d + 1, m)] = uint16_t(v[d] >> 16);
      }
    }
    for (int x = tid; x < (s_pad - s) * R; x += kSmThreads) xr16[xs_at(s + x / R, x % R)] = 0;
  };
  // The weight rows of the chunk's blocks form one stream of batches: block
  // bi's rows are stream rows bi * s_pad + k, and batch n (kStep rows, 8 per
  // thread: rows n kStep + kr + u KL) lies inside block n kStep / s_pad.  The
  // two-batch pipeline therefore keeps 2 x 8 16-byte loads per thread in
  // flight across block boundaries, not only inside a block (a 256-row block
  // is a single batch).  Rows past s load nothing and meet zero activations.
  // With room for every block the chunk needs, all activations are staged up
  // front, behind the first two batches' loads.  Otherwise one region is
  // restaged at each block's first batch, between two barriers, while that
  // batch and the next are already in flight: the weight stream does not drain
  // at block boundaries.
  const int bat_per_block = s_pad / kStep;
  auto run_stream = [&](int nbat, bool restage) {
    auto load_batch = [&](int n, u32x4 (&wv)[kSmUnroll]) {
      const int bl = uni_div(n * kStep, s_pad);
      const int k0 = n * kStep - bl * s_pad + kr;
      const uint16_t* wp = n < nbat ? W + (int64_t(s_blocks[bl]) * s + k0) * N + col0 + l8 * 8 : W;
#pragma unroll
      for (int u = 0; u < kSmUnroll; ++u) {
        const int kk = k0 + u * kSmKLanes;
        wv[u] = (n < nbat && kk < s && col_on) ? *reinterpret_cast<const u32x4*>(wp + int64_t(u) * kSmKLanes * N)
                                               : (u32x4){0u, 0u, 0u, 0u};
      }
    };
    // weight rows kk (piece 2v) and kk + KL (piece 2v + 1) are applied together:
    // their columns interleaved into bf16 pairs, one v_dot2c_f32_bf16 per
    // row and column (a weight past the group width is loaded as zero, and so
    // is its activation)
    auto apply_batch = [&](int n, const u32x4 (&wv)[kSmUnroll]) {
      if (n >= nbat) return;
      const int bl = uni_div(n * kStep, s_pad);
      const int k0 = n * kStep - bl * s_pad + kr;
      if (k0 - kr >= s) return;  // a batch of padding rows only
      const unsigned* xsb = xs2 + (restage ? 0 : bl) * (x_region / 2);
#pragma unroll
      for (int v = 0; v < kSmUnroll / 2; ++v) {
        const int kk = k0 + 2 * v * KL;
        unsigned wp[8];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          wp[2 * d] = __builtin_amdgcn_perm(wv[2 * v + 1][d], wv[2 * v][d], 0x05040100u);      // column 2d
          wp[2 * d + 1] = __builtin_amdgcn_perm(wv[2 * v + 1][d], wv[2 * v][d], 0x07060302u);  // column 2d + 1
        }
        const unsigned* xr = xsb + ((kk / (2 * KL)) * KL + (kk % KL)) * R;
#pragma unroll
        for (int m = 0; m < R; ++m) {
          const bf16x2 xp = __builtin_bit_cast(bf16x2, xr[m]);
#pragma unroll
          for (int c = 0; c < 8; ++c)
            acc[m][c] = __builtin_amdgcn_fdot2_f32_bf16(xp, __builtin_bit_cast(bf16x2, wp[c]), acc[m][c], false);
        }
      }
    };
    u32x4 wa[kSmUnroll], wb[kSmUnroll];
    load_batch(0, wa);
    load_batch(1, wb);
    if (!restage) {
      for (int bi = 0; bi < nblk; ++bi) stage(s_blocks[bi], bi);
      __syncthreads();
    }
    // restage before batch n when it opens a block (n and the pacing counter
    // are uniform, so every thread meets the same barriers)
    int next_blk = 0, next_n = 0;
    auto boundary = [&](int n) {
      if (!restage || n >= nbat || n != next_n) return;
      if (n > 0) __syncthreads();  // every wave is done with the previous block
      stage(s_blocks[next_blk], 0);
      __syncthreads();
      ++next_blk;
      next_n += bat_per_block;
    };
    for (int n = 0; n < nbat; n += 2) {
      boundary(n);
      apply_batch(n, wa);
      load_batch(n + 2, wa);
      boundary(n + 1);
      apply_batch(n + 1, wb);
      load_batch(n + 3, wb);
    }
  };
  run_stream(nblk * bat_per_block, a.x_regions == 1);

  // reduce the weight-row lanes: those of a wave by a fixed shuffle tree, then
  // the 4 waves in a fixed order
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int m = 0; m < R; ++m)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float v = acc[m][c];
#pragma unroll
      for (int o = kSmColLanes; o < 64; o *= 2) v += __shfl_xor(v, o, 64);
      acc[m][c] = v;
    }
  if (lane < kSmColLanes) {
#pragma unroll
    for (int m = 0; m < R; ++m)
#pragma unroll
      for (int c = 0; c < 8; ++c) red[(wave * R + m) * kSmCols + lane * 8 + c] = acc[m][c];
  }
  __syncthreads();
  for (int x = tid; x < R * kSmCols; x += kSmThreads) {
    const int m = x / kSmCols, c = x - m * kSmCols;
    if (m >= M || c >= ncol) continue;
    const float v = ((red[(0 * R + m) * kSmCols + c] + red[(1 * R + m) * kSmCols + c]) +
                     red[(2 * R + m) * kSmCols + c]) + red[(3 * R + m) * kSmCols + c];
    const bf16x2 p = __builtin_convertvector((f32x2){v, 0.f}, bf16x2);
    Y[int64_t(m) * N + col0 + c] = uint16_t(__builtin_bit_cast(unsigned, p) & 0xffffu);
  }
}

template <int R, int COLS>
hipError_t launch_rc(SmallArgs a, int E, hipStream_t st) {
  a.chunks_per_group = (a.r + COLS - 1) / COLS;
  a.xcd_order = (2 * a.r) % 128 != 0 ? 1 : 0;
  const dim3 grid(unsigned(a.q * a.chunks_per_group), unsigned(E));
  constexpr int KL = kSmThreads / (COLS / 8);  // weight rows per step (the pair distance)
  constexpr int kStep = KL * kSmUnroll;          // weight rows per batch
  const size_t s_pad = size_t(a.s + kStep - 1) / kStep * kStep;
  // a chunk of output group j needs W_jj and W_tj for the other types among the
  // rows: at most min(q, 1 + R) blocks; stage them all when they fit kSmStageAll
  const int nb_max = a.q < 1 + R ? a.q : 1 + R;
  a.x_regions = (nb_max > 1 && s_pad * R * nb_max <= size_t(kSmStageAll)) ? nb_max : 1;
  const size_t shm = s_pad * R * 2 * a.x_regions + 16 + sizeof(float) * 4 * R * COLS;
  static bool attr_set = false;  // allow more than the default 64 KB of dynamic LDS
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&small_m_kernel<R, COLS>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             int(kSmStageAll * 2 + 16 + sizeof(float) * 4 * R * COLS));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((small_m_kernel<R, COLS>), grid, dim3(kSmThreads), shm, st, a);
  return hipGetLastError();
}

// the widest chunk that the group width fills and that still gives about two
// workgroups per CU (measured on 64 experts, 7168 -> 2048, q = 4: 64 columns
// 4.8 TB/s, 256 columns 6.0 TB/s).  A group whose rows are not whole 128-byte
// lines (e.g. 96 columns) instead runs as one chunk, the narrowest that holds
// it, when that still gives as many workgroups: no line is split between two
// chunks, and at 8 rows (3 workgroups per CU) the grid stays in one round
// (64 experts, 2048 -> 768, q = 8: one row 20.0 -> 17.2 us, eight rows
// 62.4 -> 51.5 us, flushed).
template <int R>
hipError_t launch_r(const SmallArgs& a, int E, hipStream_t st) {
  const int64_t want = 512;
  if ((2 * a.r) % 128 != 0 && a.r <= 512 && int64_t(E) * a.q >= want) {
    if (a.r <= 64) return launch_rc<R, 64>(a, E, st);
    if (a.r <= 128) return launch_rc<R, 128>(a, E, st);
    if (a.r <= 256) return launch_rc<R, 256>(a, E, st);
    return launch_rc<R, 512>(a, E, st);
  }
  auto fits = [&](int cols) { return a.r >= cols && int64_t(E) * a.q * ((a.r + cols - 1) / cols) >= want; };
  // 64-column chunks when they all fit one round of resident workgroups (8
  // rows hold 151-163 VGPRs: 3 per CU; fewer rows at most 131 of the 64-column
  // kernel's VGPRs: 4 per CU): more weight bytes in flight per CU than half as
  // many wider chunks (64 experts 2048 -> 768, q = 4, flushed: 8 rows 55.3 ->
  // 51.6 us, one row 24.6 -> 22.4 us)
  const int64_t resident = int64_t(R == 8 ? 3 : 4) * 256;
  if (int64_t(E) * a.q * ((a.r + 63) / 64) <= resident) return launch_rc<R, 64>(a, E, st);
  if (fits(512)) return launch_rc<R, 512>(a, E, st);
  if (fits(256)) return launch_rc<R, 256>(a, E, st);
  if (fits(128)) return launch_rc<R, 128>(a, E, st);
  return launch_rc<R, 64>(a, E, st);
}

}  // namespace

bool small_m_supported(const ProblemDesc& p) {
  if (p.op != Op::Fwd || p.M < 1 || p.M > kSmMaxRows) return false;
  int R = 1;
  while (R < p.M) R <<= 1;
  // the staged group width padded to whole batches (at most 256 rows: 64-column chunks)
  return ((p.K / p.q + 255) / 256 * 256) * R <= kSmMaxXs;
}

hipError_t launch_small_m_bf16(const ProblemDesc& p, hipStream_t st) {
  SmallArgs a;
  a.X = static_cast<const uint16_t*>(p.A);
  a.W = static_cast<const uint16_t*>(p.B);
  a.Y = static_cast<uint16_t*>(p.C);
  a.tau = p.tau;
  a.q = p.q;
  a.M = int(p.M);
  a.K = int(p.K);
  a.N = int(p.N);
  a.s = int(p.K / p.q);
  a.r = int(p.N / p.q);
  if (p.M <= 1) return launch_r<1>(a, p.E, st);
  if (p.M <= 2) return launch_r<2>(a, p.E, st);
  if (p.M <= 4) return launch_r<4>(a, p.E, st);
  return launch_r<8>(a, p.E, st);
}

}  // namespace qalg
