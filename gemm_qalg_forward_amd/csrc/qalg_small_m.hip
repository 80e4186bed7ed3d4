// Small-M forward of the row-typed Q_q projection: a weight-streaming kernel
// for a handful of token rows per weight bank (KV-cached decode: one new row
// per sequence; tiny per-expert token counts).
//
// Paper: arXiv 2609.32814.  Section 5.2 notes that decode needs a separate
// matrix-vector implementation because the row dimension is small; section 5.3
// that the decode kernel performs vector reductions; section 6.3 and appendix G
// that single-token work is bounded by weight bandwidth.
//
// Design: weight-stationary.  A workgroup owns a 64-column chunk of one output
// group j of one problem.  The weight blocks that chunk needs are W_jj (every
// typed row uses it, eq 17) and W_tj for each type t != j present among the
// rows (eq 17's x_t W_tj term; W_jj alone when t == j, eq 16).  Each needed
// block is streamed from HBM exactly once, in 16-byte row pieces, and applied
// to every row that needs it; rows that do not need the block see zeros
// (staged in LDS), so the inner loop has no branches.  Blocks are visited in a
// fixed order and partial sums are reduced in a fixed tree: the result is
// bitwise reproducible.  No type index is needed: the <= 8 types are read
// directly.
#include "qalg_internal.h"

namespace qalg {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kSmThreads = 256;
constexpr int kSmCols = 64;            // output columns per workgroup
constexpr int kSmKLanes = kSmThreads / (kSmCols / 8);  // 32 weight rows in flight per step
constexpr int kSmMaxRows = 8;
constexpr int kSmUnroll = 4;
constexpr int kSmMaxXs = 16384;        // bf16 elements of staged activations (32 KB)

struct SmallArgs {
  const uint16_t* X;
  const uint16_t* W;
  const int32_t* tau;
  uint16_t* Y;
  int q, M, K, N, s, r;
  int chunks_per_group;
};

__device__ __forceinline__ float lo_bf16(unsigned u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_bf16(unsigned u) { return __uint_as_float(u & 0xffff0000u); }

template <int R>
__global__ __launch_bounds__(kSmThreads) void small_m_kernel(SmallArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char sm_raw[];
  uint16_t* xs = reinterpret_cast<uint16_t*>(sm_raw);               // [s][R]
  float* red = reinterpret_cast<float*>(sm_raw + size_t(a.s) * R * 2 + 16);  // [4][R][64]
  __shared__ int s_type[R];
  __shared__ int s_blocks[R + 1];
  __shared__ int s_nblk;

  const int e = blockIdx.y;
  const int j = blockIdx.x / a.chunks_per_group;
  const int ch = blockIdx.x - j * a.chunks_per_group;
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

  const int l8 = tid & 7, kr = tid >> 3;
  const bool col_on = l8 * 8 < ncol;
  float acc[R][8];
#pragma unroll
  for (int m = 0; m < R; ++m)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[m][c] = 0.f;

  const int nblk = s_nblk;
  for (int bi = 0; bi < nblk; ++bi) {
    const int b = s_blocks[bi];
    // stage x[m, g_b] transposed (xs[k][m]); zero for rows that do not use block (b, j)
    for (int x = tid; x < s * R; x += kSmThreads) {
      const int k = x / R, m = x - (x / R) * R;
      const int t = s_type[m];
      const bool need = t >= 0 && (b == j || t == b);
      xs[x] = need ? X[int64_t(m) * K + int64_t(b) * s + k] : uint16_t(0);
    }
    __syncthreads();
    const uint16_t* wp = W + int64_t(b) * s * N + col0 + l8 * 8;
    for (int k = kr; k < s; k += kSmKLanes * kSmUnroll) {
      u32x4 wv[kSmUnroll];
#pragma unroll
      for (int u = 0; u < kSmUnroll; ++u) {
        const int kk = k + u * kSmKLanes;
        wv[u] = (kk < s && col_on) ? *reinterpret_cast<const u32x4*>(wp + int64_t(kk) * N)
                                   : (u32x4){0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < kSmUnroll; ++u) {
        const int kk = k + u * kSmKLanes;
        if (kk >= s) break;
        float w8[8];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          w8[2 * d] = lo_bf16(wv[u][d]);
          w8[2 * d + 1] = hi_bf16(wv[u][d]);
        }
        const uint16_t* xr = xs + kk * R;
#pragma unroll
        for (int m = 0; m < R; ++m) {
          const float xv = __uint_as_float(unsigned(xr[m]) << 16);
#pragma unroll
          for (int c = 0; c < 8; ++c) acc[m][c] = fmaf(xv, w8[c], acc[m][c]);
        }
      }
    }
    __syncthreads();  // xs is restaged for the next block
  }

  // reduce the 32 weight-row lanes: 8 per wave by a fixed shuffle tree, then 4 waves
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int m = 0; m < R; ++m)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float v = acc[m][c];
      v += __shfl_xor(v, 8, 64);
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      acc[m][c] = v;
    }
  if (lane < 8) {
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

template <int R>
hipError_t launch_r(const SmallArgs& a, int E, hipStream_t st) {
  const dim3 grid(unsigned(a.q * a.chunks_per_group), unsigned(E));
  const size_t shm = size_t(a.s) * R * 2 + 16 + sizeof(float) * 4 * R * kSmCols;
  hipLaunchKernelGGL((small_m_kernel<R>), grid, dim3(kSmThreads), shm, st, a);
  return hipGetLastError();
}

}  // namespace

bool small_m_supported(const ProblemDesc& p) {
  if (p.op != Op::Fwd || p.M < 1 || p.M > kSmMaxRows) return false;
  int R = 1;
  while (R < p.M) R <<= 1;
  return (p.K / p.q) * R <= kSmMaxXs;
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
  a.chunks_per_group = (a.r + kSmCols - 1) / kSmCols;
  if (p.M <= 1) return launch_r<1>(a, p.E, st);
  if (p.M <= 2) return launch_r<2>(a, p.E, st);
  if (p.M <= 4) return launch_r<4>(a, p.E, st);
  return launch_r<8>(a, p.E, st);
}

}  // namespace qalg
