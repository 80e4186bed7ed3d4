// Type schedule and type index for the row-typed Q_q projection.
//
// Paper: arXiv 2609.32814.  Section 4 gives the position-type schedule
// tau(p) (cyclic; appendix D.5 the pilot's interval form); Algorithm 1 forms
// the row sets I_i = {b : tau(p_b) = i} that every later step works on.
//
// The index is built without a sort, inside a single workgroup per problem.
// A cyclic schedule (tau[m] = (o + m) mod q, the paper's position schedule at
// any offset) is recognised by one parallel pass and its index written in
// closed form.  Any other schedule takes one counting pass and one stable
// scatter.  Each of the 16 waves owns a
// contiguous slice of the rows; within a 64-row step a wave groups its lanes
// by type with ballots (one round per distinct type present), so both passes
// cost O(M / 64 * distinct types per step) wave instructions.  The scatter
// keeps rows of a type in ascending order because slices, steps and lanes
// are visited in row order.  The type offsets and the row-tile prefix sums
// (one per tile height) are scans over q + 1 values: shuffles within one wave
// when q < 64, block-wide scans otherwise.
#include "qalg_internal.h"

namespace qalg {

namespace {

constexpr int kIdxThreads = 1024;
constexpr int kIdxWaves = kIdxThreads / 64;
constexpr int kBatch = 8;  // 64-row steps whose types are loaded together

__global__ void type_schedule_kernel(const int64_t* __restrict__ pos, int64_t M, int q, int kind,
                                     int64_t period, int32_t* __restrict__ tau) {
  const int64_t step = int64_t(gridDim.x) * blockDim.x;
  const int64_t width = kind == 1 ? period / q : 1;
  for (int64_t m = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; m < M; m += step) {
    const int64_t p = pos[m];
    int32_t t;
    if (p < 0)
      t = -1;
    else if (kind == 0)
      t = int32_t(p % q);
    else
      t = int32_t((p % period) / width);
    tau[m] = t;
  }
}

// Exclusive prefix sum over the block of a value per thread; all threads must
// call it.  `tmp` holds kIdxWaves + 1 ints of shared memory.  Returns the
// exclusive prefix; *total receives the sum.
__device__ int block_exclusive_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) tmp[w] = x;
  __syncthreads();
  if (w == 0) {
    int y = lane < kIdxWaves ? tmp[lane] : 0;
#pragma unroll
    for (int d = 1; d < kIdxWaves; d <<= 1) {
      const int z = __shfl_up(y, d, 64);
      if (lane >= d) y += z;
    }
    if (lane < kIdxWaves) tmp[lane] = y;
  }
  __syncthreads();
  const int before = w > 0 ? tmp[w - 1] : 0;
  *total = tmp[kIdxWaves - 1];
  __syncthreads();  // tmp may be reused by the next call
  return before + x - v;
}

// Inclusive prefix sum over the 64 lanes of a wave (no shared memory).
__device__ int wave_inclusive_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

// One workgroup per problem (blockIdx.x = problem).  Optional `zero_out`: the
// rows of an out-of-range type are zeroed there (row length zero_ld elements of
// zero_elem_bytes bytes), so the projection that follows need not visit them.
__global__ __launch_bounds__(kIdxThreads) void build_index_kernel(
    const int32_t* __restrict__ tau_all, int q, int M, int32_t* __restrict__ ws_all,
    int64_t ws_stride, int64_t off_counts, int64_t off_offsets, int64_t off_tiles,
    int64_t off_rows, void* zero_out, int64_t zero_ld, int zero_elem_bytes,
    int64_t zero_stride_bytes) {
  extern __shared__ int sm[];
  const int Q1 = q + 1;  // column q collects rows with an out-of-range type
  int* tab = sm;                          // [kIdxWaves][Q1]: per-wave counts, then bases
  int* tot = sm + kIdxWaves * Q1;         // [Q1]: per-type totals, then offsets
  int* tmp = tot + Q1;                    // [kIdxWaves + 1]

  const int e = blockIdx.x;
  const int32_t* tau = tau_all + int64_t(e) * M;
  int32_t* ws = ws_all + int64_t(e) * ws_stride;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  for (int x = tid; x < kIdxWaves * Q1; x += kIdxThreads) tab[x] = 0;

  const int slice = (M + kIdxWaves * 64 - 1) / (kIdxWaves * 64) * 64;
  const int r0 = min(w * slice, M), r1 = min(r0 + slice, M);
  int* my = tab + w * Q1;

  // Cyclic schedules (tau[m] = (o + m) mod q for every row, o = tau[0]) have a
  // closed-form index; checking for one is a fully parallel pass.
  __shared__ int s_cyclic;
  const int t0 = M > 0 ? tau[0] : 0;
  if (tid == 0) s_cyclic = (M > 0 && t0 >= 0 && t0 < q) ? 1 : 0;
  __syncthreads();  // also orders the zeroing of tab before pass 1
  if (s_cyclic) {
    // kBatch independent loads per thread before any comparison, so that a
    // thread waits for one memory latency per batch instead of one per row
    const int step = kIdxThreads % q;
    int want = (t0 + tid) % q;  // (t0 + m) mod q for m = tid + kIdxThreads k
    bool ok = true;
    for (int m0 = tid; m0 < M; m0 += kIdxThreads * kBatch) {
      int tv[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int m = m0 + b * kIdxThreads;
        tv[b] = m < M ? tau[m] : 0;
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int m = m0 + b * kIdxThreads;
        ok &= m >= M || tv[b] == want;
        want += step;
        if (want >= q) want -= q;
      }
    }
    if (!ok) s_cyclic = 0;
  }
  __syncthreads();
  const bool cyclic = s_cyclic != 0;

  // pass 1 (listed schedules): per-wave counts of each type in its slice.  Types
  // are loaded kBatch steps at a time so that the loads overlap.
  for (int base = r0; base < r1 && !cyclic; base += 64 * kBatch) {
    int tv[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int m = base + b * 64 + lane;
      tv[b] = (m < r1) ? tau[m] : 0;
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int m = base + b * 64 + lane;
      if (base + b * 64 >= r1) break;
      int t = -1;
      if (m < r1) {
        const int v = tv[b];
        t = (v >= 0 && v < q) ? v : q;
      }
      uint64_t left = __ballot(t >= 0);
      while (left) {
        const int leader = __builtin_ctzll(left);
        const int tl = __builtin_amdgcn_readlane(t, leader);
        const uint64_t mask = __ballot(t == tl);
        if (lane == leader) my[tl] += __popcll(mask);
        left &= ~mask;
      }
    }
  }
  if (!cyclic) __syncthreads();

  // per type: exclusive prefix over waves (in place), total per type.  With
  // q < 64 types the scans below run in one wave, and a cyclic schedule's
  // totals are formed there too.
  const bool wave_scans = Q1 <= 64;
  for (int t = tid; t < Q1 && (!cyclic || !wave_scans); t += kIdxThreads) {
    if (cyclic) {
      // rows of type t are (t - t0) mod q + k q
      const int start = (t - t0 + q) % q;
      tot[t] = (t < q && start < M) ? (M - 1 - start) / q + 1 : 0;
      continue;
    }
    int run = 0;
    for (int ww = 0; ww < kIdxWaves; ++ww) {
      const int c = tab[ww * Q1 + t];
      tab[ww * Q1 + t] = run;
      run += c;
    }
    tot[t] = run;
  }
  if (!cyclic || !wave_scans) __syncthreads();

  int32_t* counts = ws + off_counts;
  int32_t* offsets = ws + off_offsets;
  int32_t* tiles = ws + off_tiles;
  int32_t* rows = ws + off_rows;

  if (wave_scans) {
    // lane t holds type t (lane q: the out-of-range rows); the same offsets
    // and tile prefix sums as the block-wide scans below, without barriers
    if (w == 0) {
      const int t = lane;
      int cnt = 0;
      if (cyclic) {
        const int start = (t - t0 + q) % q;
        cnt = (t < q && start < M) ? (M - 1 - start) / q + 1 : 0;
      } else if (t < Q1) {
        cnt = tot[t];
      }
      const int c = t < q ? cnt : 0;
      const int inc = wave_inclusive_scan(c);
      const int valid_rows = __shfl(inc, 63, 64);
      const int nbad = __shfl(cnt, q, 64);
      if (t < q) {
        counts[t] = c;
        offsets[t] = inc - c;
      }
      if (t == 0) {
        offsets[q] = valid_rows;
        ws[0] = nbad;
      }
      if (t < Q1) tot[t] = (t < q) ? inc - c : valid_rows;
      for (int h = 0; h < kNumTileHeights; ++h) {
        const int bm = kTileHeights[h];
        const int nt = (c + bm - 1) / bm;
        const int ti = wave_inclusive_scan(nt);
        const int sum = __shfl(ti, 63, 64);
        if (t < q) tiles[h * Q1 + t] = ti - nt;
        if (t == 0) tiles[h * Q1 + q] = sum;
      }
    }
    __syncthreads();
  } else {
    // offsets over types 0..q-1; the out-of-range rows follow all valid rows
    // (q <= QALG_MAX_Q < kIdxThreads: one value per thread)
    {
      const int t = tid;
      const int cnt = (t < q) ? tot[t] : 0;
      int valid_rows;
      const int ex = block_exclusive_scan(cnt, tmp, &valid_rows);
      if (t < q) {
        counts[t] = cnt;
        offsets[t] = ex;
      }
      if (tid == 0) {
        offsets[q] = valid_rows;
        ws[0] = tot[q];  // rows with an out-of-range type
      }
      __syncthreads();
      if (t < Q1) tot[t] = (t < q) ? ex : valid_rows;  // first slot of each type
      __syncthreads();
    }

    // row-tile prefix sums for each tile height
    for (int h = 0; h < kNumTileHeights; ++h) {
      const int bm = kTileHeights[h];
      const int t = tid;
      const int c = (t < q) ? counts[t] : 0;  // same thread wrote counts[t]
      const int nt = (c + bm - 1) / bm;
      int sum;
      const int ex = block_exclusive_scan(nt, tmp, &sum);
      if (t < q) tiles[h * Q1 + t] = ex;
      if (tid == 0) tiles[h * Q1 + q] = sum;
    }
  }

  // bases: first output slot of each (wave, type); a cyclic index has no scatter
  if (!cyclic) {
    for (int x = tid; x < kIdxWaves * Q1; x += kIdxThreads) tab[x] += tot[x % Q1];
    __syncthreads();
  }

  if (cyclic) {
    // closed-form row list: slot offsets[i] + k holds (i - t0) mod q + k q
    for (int t = 0; t < q; ++t) {
      const int start = (t - t0 + q) % q;
      const int first = tot[t], cnt = tot[t + 1] - tot[t];
      for (int k = tid; k < cnt; k += kIdxThreads) rows[first + k] = start + k * q;
    }
  }

  // pass 2 (listed schedules): stable scatter of row ids
  for (int base = r0; base < r1 && !cyclic; base += 64 * kBatch) {
    int tv[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int m = base + b * 64 + lane;
      tv[b] = (m < r1) ? tau[m] : 0;
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int m = base + b * 64 + lane;
      if (base + b * 64 >= r1) break;
      int t = -1;
      if (m < r1) {
        const int v = tv[b];
        t = (v >= 0 && v < q) ? v : q;
      }
      uint64_t left = __ballot(t >= 0);
      const uint64_t below = (uint64_t(1) << lane) - 1;
      while (left) {
        const int leader = __builtin_ctzll(left);
        const int tl = __builtin_amdgcn_readlane(t, leader);
        const uint64_t mask = __ballot(t == tl);
        if (t == tl) rows[my[tl] + __popcll(mask & below)] = m;
        if (lane == leader) my[tl] += __popcll(mask);
        left &= ~mask;
      }
    }
  }

  if (tid == 0) {
    ws[2] = q;
    ws[3] = M;
    ws[4] = s_cyclic ? t0 : -1;  // cyclic schedule: rows of type i are (i - t0) mod q + k q
    ws[1] = kIndexMagic;
  }

  // zero the output rows of out-of-range types (rare; usually nothing to do)
  if (zero_out != nullptr) {
    __syncthreads();
    const int nbad = M - tot[q];  // tot[q] = first slot after the valid rows
    if (nbad > 0) {
      char* out = static_cast<char*>(zero_out) + int64_t(e) * zero_stride_bytes;
      const int64_t row_bytes = zero_ld * zero_elem_bytes;
      for (int b = 0; b < nbad; ++b) {
        const int m = rows[tot[q] + b];
        uint32_t* p = reinterpret_cast<uint32_t*>(out + int64_t(m) * row_bytes);
        for (int64_t x = tid; x < row_bytes / 4; x += kIdxThreads) p[x] = 0u;
      }
    }
  }
}

// Zero the output rows of out-of-range types listed in an existing index.
__global__ __launch_bounds__(256) void zero_bad_rows_kernel(const int32_t* __restrict__ ws_all,
                                                             int64_t ws_stride, int64_t off_offsets,
                                                             int64_t off_rows, int q, void* out_all,
                                                             int64_t row_bytes, int64_t stride_bytes,
                                                             int M) {
  const int32_t* ws = ws_all + int64_t(blockIdx.x) * ws_stride;
  if (ws[1] != kIndexMagic || ws[2] != q || ws[3] != M) return;  // not an index of this (q, M)
  const int nbad = ws[0];
  if (nbad <= 0 || nbad > M) return;
  const int first = ws[off_offsets + q];
  char* out = static_cast<char*>(out_all) + int64_t(blockIdx.x) * stride_bytes;
  for (int b = 0; b < nbad; ++b) {
    const int m = ws[off_rows + first + b];
    if (m < 0 || m >= M) continue;
    uint32_t* p = reinterpret_cast<uint32_t*>(out + int64_t(m) * row_bytes);
    for (int64_t x = threadIdx.x; x < row_bytes / 4; x += blockDim.x) p[x] = 0u;
  }
}

__global__ void fill_zero_kernel(uint32_t* p, size_t n) {
  for (size_t x = size_t(blockIdx.x) * blockDim.x + threadIdx.x; x < n; x += size_t(gridDim.x) * blockDim.x)
    p[x] = 0u;
}

}  // namespace

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, static_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

hipError_t launch_zero_bad_rows(const int32_t* ws, int q, int64_t M, int E, int64_t ws_stride_ints,
                                void* out, int64_t ld, int elem_bytes, int64_t stride_bytes,
                                hipStream_t s) {
  const WsLayout L = ws_layout(q, M);
  hipLaunchKernelGGL(zero_bad_rows_kernel, dim3(E), dim3(256), 0, s, ws, ws_stride_ints, L.offsets,
                     L.rows, q, out, ld * elem_bytes, stride_bytes, int(M));
  return hipGetLastError();
}

hipError_t launch_type_schedule(const int64_t* pos, int64_t M, int q, int kind, int64_t period,
                                int32_t* tau, hipStream_t s) {
  const int threads = 256;
  int64_t blocks = (M + threads - 1) / threads;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(type_schedule_kernel, dim3(unsigned(blocks)), dim3(threads), 0, s, pos, M, q,
                     kind, period, tau);
  return hipGetLastError();
}

hipError_t launch_build_index_zeroing(const int32_t* tau, int q, int64_t M, int E, int32_t* ws,
                                      int64_t ws_stride_ints, void* zero_out, int64_t zero_ld,
                                      int zero_elem_bytes, int64_t zero_stride_bytes,
                                      hipStream_t s) {
  const WsLayout L = ws_layout(q, M);
  const size_t shm = sizeof(int) * (size_t(kIdxWaves) * (q + 1) + (q + 1) + kIdxWaves + 1);
  hipLaunchKernelGGL(build_index_kernel, dim3(E), dim3(kIdxThreads), shm, s, tau, q, int(M), ws,
                     ws_stride_ints, L.counts, L.offsets, L.tile_off, L.rows, zero_out, zero_ld,
                     zero_elem_bytes, zero_stride_bytes);
  return hipGetLastError();
}

hipError_t launch_build_index(const int32_t* tau, int q, int64_t M, int E, int32_t* ws,
                              int64_t ws_stride_ints, hipStream_t s) {
  return launch_build_index_zeroing(tau, q, M, E, ws, ws_stride_ints, nullptr, 0, 0, 0, s);
}

}  // namespace qalg
