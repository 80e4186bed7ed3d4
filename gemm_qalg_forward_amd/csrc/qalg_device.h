// Device helpers shared by the persistent matrix-core kernels of libqalg
// (gfx950): vector types, direct-to-LDS copies with hand-tracked completion,
// an LDS-only workgroup barrier, the LDS piece swizzles and bf16 packing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qalg {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
#define LDS_AS __attribute__((address_space(3)))


// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One 16-byte piece per lane from global memory straight into LDS: lane l's
// piece lands at lds_addr + 16 l (gfx950 global_load_lds_dwordx4; lds_addr must
// be wave-uniform; M0 holds it, and one wait state must separate the M0 write
// from the load).  Written as inline assembly so that the compiler does not
// treat every later LDS read as possibly depending on the copy; completion is
// tracked by hand with wait_vmcnt before the barrier that publishes a stage.
__device__ __forceinline__ void copy16_to_lds(const char* gbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(gbase), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}

// The same copy through a buffer resource (gfx950 buffer_load_dwordx4 with
// lds): a lane whose offset lies at or past the resource's byte count reads
// nothing from memory and writes zeros into its LDS piece.  The resource is
// wave-uniform (four scalar registers, see buffer_rsrc).
__device__ __forceinline__ void copy16_to_lds_buf(u32x4 rsrc, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}

// Raw buffer resource over `bytes` bytes at base (no stride, no swizzle): the
// hardware range check returns zeros for offsets at or past `bytes`.
__device__ __forceinline__ u32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return (u32x4){uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(a)))),
                 uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(a >> 32) & 0xffffu))),
                 uint32_t(__builtin_amdgcn_readfirstlane(int(bytes))), 0x00020000u};
}

// Workgroup barrier ordering LDS only (the stage copies are waited for
// explicitly; global stores need no ordering here).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// LDS piece swizzles.  A contraction-major tile (rows of 32 contraction
// values, 64 bytes) keeps row r's 16-byte piece c at c ^ ((r >> 1) & 3), so
// that 8 consecutive lanes of the fragment reads and of the 1 KB
// direct-to-LDS copies touch distinct bank groups.
__device__ __forceinline__ int swz_x(int row) { return (row >> 1) & 3; }
// Contraction-major tile with rows of 64 contraction values (128 bytes): row
// r keeps its piece c at c ^ ((r >> 1) & 7), so that the 16 rows a
// quarter-wave reads, and the 8 rows a 1 KB copy writes, fall in distinct
// bank groups.
__device__ __forceinline__ int swz_x128(int row) { return (row >> 1) & 7; }
// Row-major tile (contraction rows of ROWB bytes, read with the transposing
// ds_read_b64_tr_b16): row k keeps its 64-byte group g (the 32 columns of one
// MFMA fragment) at g ^ s(k).  Half a wave of such a read takes 64 bytes from
// each of 4 consecutive rows, and the LDS serves 256 bytes (64 banks) per
// pass: s(k) = k & 3 when rows are a multiple of 256 bytes long, and
// (k >> 1) & 1 when they are 128 bytes past one, put the 4 groups in the 4
// distinct quarters of the bank window.  Returned as a mask on the 16-byte
// piece index.
template <int ROWB>
__device__ __forceinline__ int swz_rm(int k) {
  static_assert(ROWB % 128 == 0 && ROWB >= 256, "row-major tile rows");
  return ROWB % 256 == 0 ? 4 * (k & 3) : 4 * ((k >> 1) & 1);
}

__device__ __forceinline__ u32x2 pack4_bf16(float a, float b, float c, float d) {
  const bf16x2 lo = __builtin_convertvector((f32x2){a, b}, bf16x2);
  const bf16x2 hi = __builtin_convertvector((f32x2){c, d}, bf16x2);
  return (u32x2){__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
}

// Read-only global data addressed uniformly: loads through this pointer type
// go through the scalar data cache (s_load), which the lgkm counter tracks,
// so they never wait behind the vector-memory counter.
typedef const __attribute__((address_space(4))) int32_t* cint_ptr;
__device__ __forceinline__ cint_ptr to_const(const int32_t* p) { return (cint_ptr)(p); }

// A value the caller knows to be the same in every lane, moved to a scalar
// register so that comparisons and branches on it stay on the scalar unit.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Group g with tile_off[g] <= rt < tile_off[g + 1] (binary search over q + 1
// non-decreasing offsets; rt and the offsets are wave-uniform).
template <class P>
__device__ __forceinline__ int find_group(P tile_off, int q, int rt) {
  int lo = 0, hi = q;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (uni(tile_off[mid]) <= rt)
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

// Recursive law Q_2^(x)L (appendix C, eq 36): types and groups are L-bit
// strings.  binom_small(L, d) counts the masks with d of L bits set,
// unrank_mask(jj, d, L) is the jj-th of them in ascending order, and
// law_member(from, mask, n, L) is the L-bit string equal to `from` on the bits
// of `mask` and to the bits of n, in order, on the others (the n-th member of a
// segment list whose fixed bits are `mask`).
__device__ __forceinline__ int binom_small(int L, int d) {
  int c = 1;
  for (int k = 0; k < d; ++k) c = c * (L - k) / (k + 1);
  return c;
}
__device__ __forceinline__ int unrank_mask(int jj, int d, int L) {
  for (int m = 0; m < (1 << L); ++m)
    if (__builtin_popcount(m) == d && jj-- == 0) return m;
  return 0;
}
__device__ __forceinline__ int law_member(int fixed_from, int fixed_mask, int n, int L) {
  int g = fixed_from & fixed_mask;
  for (int k = 0; k < L; ++k)
    if (!((fixed_mask >> k) & 1)) {
      if (n & 1) g |= 1 << k;
      n >>= 1;
    }
  return g;
}

// Type index of a cyclic schedule (tau[m] = (o + m) mod q for every row m),
// in closed form: type i has M / q rows, plus one when (i - o) mod q <
// M mod q; row tiles are tile_h rows of one type.  Decoding a tile then needs
// no memory access (the workspace's tables hold the same numbers).
struct CycIndex {
  int q, o, base, rem, tile_h, per_type, uniform;
  __device__ static CycIndex make(int q, int o, int M, int tile_h) {
    CycIndex c;
    c.q = q;
    c.o = o;
    c.base = M / q;
    c.rem = M - c.base * q;
    c.tile_h = tile_h;
    // every type has the same tile count unless an extra row opens a tile
    c.uniform = c.rem == 0 || c.base % tile_h != 0;
    c.per_type = c.uniform ? (c.base + tile_h - 1) / tile_h : c.base / tile_h;
    return c;
  }
  // types j < i among the cyclic interval [o, o + rem) of types with an extra row
  __device__ int extra_before(int i) const {
    if (rem == 0) return 0;
    const int end = o + rem;
    int c = max(0, min(i, end) - o);
    if (end > q) c += min(i, end - q);
    return c;
  }
  __device__ int count(int i) const { return base + (extra_before(i + 1) - extra_before(i)); }
  __device__ int offset(int i) const { return i * base + extra_before(i); }  // first slot of type i
  __device__ int tiles_before(int i) const { return i * per_type + (uniform ? 0 : extra_before(i)); }
  __device__ int group_of_tile(int rt) const {
    if (uniform) return per_type > 0 ? min(rt / per_type, q - 1) : 0;
    int lo = 0, hi = q;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tiles_before(mid) <= rt)
        lo = mid;
      else
        hi = mid;
    }
    return lo;
  }
};

// The same queries answered from the index workspace's tables (any schedule).
struct MemIndex {
  cint_ptr offsets, tile_off;
  int q;
  __device__ int count(int i) const { return uni(offsets[i + 1]) - uni(offsets[i]); }
  __device__ int offset(int i) const { return uni(offsets[i]); }
  __device__ int tiles_before(int i) const { return uni(tile_off[i]); }
  __device__ int group_of_tile(int rt) const { return find_group(tile_off, q, rt); }
};

// Tile list of a workgroup in a persistent grid whose tiles come in two
// lengths (t_long and t_short k-steps).  Each XCD takes a contiguous share of
// the long and of the short tiles; its workgroups are dealt the longs round
// robin first; workgroups left one long tile short then take up to
// t_long / t_short short tiles each before the remaining shorts are dealt
// round robin, so that the k-steps per workgroup end within one tile of each
// other while concurrently running tiles stay neighbours in the tile order.
struct TileDeal {
  int lx0, lx1, sx0, sx1;   // this XCD's long and short tile ranges
  int g, G;                 // slot inside the XCD, workgroups per XCD
  int light, lg, G_light, E, base;
  int phase, k;
  __device__ void init(int n_long, int n_short, int t_long, int t_short, int xcd, int nx, int slot, int per_x) {
    lx0 = int(int64_t(n_long) * xcd / nx);
    lx1 = int(int64_t(n_long) * (xcd + 1) / nx);
    sx0 = int(int64_t(n_short) * xcd / nx);
    sx1 = int(int64_t(n_short) * (xcd + 1) / nx);
    g = slot;
    G = per_x;
    const int nl = lx1 - lx0, ns = sx1 - sx0;
    const int rem = nl % G;
    light = rem != 0 && g >= rem;
    G_light = rem != 0 ? G - rem : 0;
    lg = g - rem;
    const int e = t_short > 0 ? t_long / t_short : 0;
    E = (rem != 0) ? min(e, ns / G_light) : 0;
    base = G_light * E;
    phase = 0;
    k = 0;
  }
  // next tile: returns false at the end; *is_long and *idx (global class index) otherwise
  __device__ bool next(bool* is_long, int* idx) {
    if (phase == 0) {
      const int i = lx0 + g + k * G;
      if (i < lx1) {
        ++k;
        *is_long = true;
        *idx = i;
        return true;
      }
      phase = 1;
      k = 0;
    }
    if (phase == 1) {
      if (light && k < E) {
        *is_long = false;
        *idx = sx0 + lg + k * G_light;
        ++k;
        return true;
      }
      phase = 2;
      k = 0;
    }
    const int i = sx0 + base + g + k * G;
    if (i < sx1) {
      ++k;
      *is_long = false;
      *idx = i;
      return true;
    }
    return false;
  }
};

}  // namespace dev
}  // namespace qalg
