// Pointwise pieces of the gated (SwiGLU) FFN's training step on the merged
// gate/up layout.
//
// Section 4 of arXiv 2609.32814 ("Change the Product, Keep the Parameters:
// Associative Algebra Layers for Transformers"): the gate and up weights of a
// gated FFN are row-typed projections like any other, and gates and pointwise
// activations keep their usual definitions; the pilot's FFN is a bias-free
// SwiGLU (appendix D), silu(z) = z * sigmoid(z).  Section 6.2 counts the
// training step of the three projections; the activation between them is the
// extra pointwise work done here.
//
// Layout.  GU is M x 2F: the merged pre-activations, i.e. the row-typed
// product of X with the merged bank Wgu (merging permutes columns inside each
// output group, so the product with the merged bank is the merged product).
// Output group j (r = F / q columns of H) owns merged columns j*2r .. j*2r+2r-1
// in pieces of 256: piece t holds gate c0..c0+63, up c0..c0+63, gate
// c0+64..c0+127, up c0+64..c0+127 for c0 = j*r + 128 t.
//
// Work.  One thread per 8 columns of H (a 16-byte piece): the matching gate
// and up pieces are 16 contiguous bytes each, 128 bytes apart, so a wave reads
// whole 64-byte runs of both.  The kernels are bound by HBM bandwidth:
// forward 6 bytes per H element (gate, up in; H out), backward 10 (gate, up,
// dH in; dgate, dup out).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "qalg_internal.h"
#include "qalg_device.h"

namespace qalg {
namespace {

using dev::pack4_bf16;
using dev::u32x2;
using u32x4v = dev::u32x4;

constexpr int kActThreads = 256;

__device__ __forceinline__ void unpack8(const u32x4v v, float (&f)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = __uint_as_float(v[e] << 16);
    f[2 * e + 1] = __uint_as_float(v[e] & 0xffff0000u);
  }
}

__device__ __forceinline__ u32x4v pack8(const float (&f)[8]) {
  const u32x2 lo = pack4_bf16(f[0], f[1], f[2], f[3]);
  const u32x2 hi = pack4_bf16(f[4], f[5], f[6], f[7]);
  return (u32x4v){lo[0], lo[1], hi[0], hi[1]};
}

// merged column of the gate value for H column c (c a multiple of 8)
__device__ __forceinline__ int gate_col(int c, int r) {
  const int j = c / r, cc = c - j * r;
  const int t = cc >> 7, b = cc & 127;
  return j * 2 * r + t * 256 + (b >> 6) * 128 + (b & 63);
}

// sigmoid through the hardware reciprocal (about 1 ulp in fp32; every result
// is rounded to bf16 afterwards)
__device__ __forceinline__ float sigmoid(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// H = silu(G) * U.  grid.x covers the F/8 pieces of a row, grid.y strides over rows.
__global__ __launch_bounds__(kActThreads) void swiglu_fwd_kernel(const uint16_t* __restrict__ GU,
                                                                uint16_t* __restrict__ H, int64_t M, int F, int r) {
  const int pc = blockIdx.x * kActThreads + threadIdx.x;
  if (pc * 8 >= F) return;
  const int c = pc * 8;
  const int gc = gate_col(c, r);
  for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
    const uint16_t* row = GU + m * 2 * F;
    const u32x4v gv = *reinterpret_cast<const u32x4v*>(row + gc);
    const u32x4v uv = *reinterpret_cast<const u32x4v*>(row + gc + 64);
    float g[8], u[8], h[8];
    unpack8(gv, g);
    unpack8(uv, u);
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = g[e] * sigmoid(g[e]) * u[e];
    __builtin_nontemporal_store(pack8(h), reinterpret_cast<u32x4v*>(H + m * F + c));
  }
}

// dG = dH * U * silu'(G), dU = dH * silu(G), silu'(z) = s (1 + z (1 - s)), s = sigmoid(z);
// written to the merged layout of GU.
__global__ __launch_bounds__(kActThreads) void swiglu_bwd_kernel(const uint16_t* __restrict__ GU,
                                                                const uint16_t* __restrict__ dH,
                                                                uint16_t* __restrict__ dGU, int64_t M, int F, int r) {
  const int pc = blockIdx.x * kActThreads + threadIdx.x;
  if (pc * 8 >= F) return;
  const int c = pc * 8;
  const int gc = gate_col(c, r);
  for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
    const uint16_t* row = GU + m * 2 * F;
    const u32x4v gv = *reinterpret_cast<const u32x4v*>(row + gc);
    const u32x4v uv = *reinterpret_cast<const u32x4v*>(row + gc + 64);
    const u32x4v hv = *reinterpret_cast<const u32x4v*>(dH + m * F + c);
    float g[8], u[8], dh[8], dg[8], du[8];
    unpack8(gv, g);
    unpack8(uv, u);
    unpack8(hv, dh);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float s = sigmoid(g[e]);
      dg[e] = dh[e] * u[e] * (s * (1.0f + g[e] * (1.0f - s)));
      du[e] = dh[e] * (g[e] * s);
    }
    uint16_t* out = dGU + m * 2 * F;
    __builtin_nontemporal_store(pack8(dg), reinterpret_cast<u32x4v*>(out + gc));
    __builtin_nontemporal_store(pack8(du), reinterpret_cast<u32x4v*>(out + gc + 64));
  }
}

// Inverse of the merge: Wgu (K x 2F merged) -> Wg, Wu (K x F each).
__global__ __launch_bounds__(kActThreads) void split_gate_up_kernel(const uint16_t* __restrict__ Wgu,
                                                                   uint16_t* __restrict__ Wg,
                                                                   uint16_t* __restrict__ Wu, int64_t K, int F,
                                                                   int r) {
  const int pc = blockIdx.x * kActThreads + threadIdx.x;
  if (pc * 8 >= F) return;
  const int c = pc * 8;
  const int gc = gate_col(c, r);
  for (int64_t k = blockIdx.y; k < K; k += gridDim.y) {
    const uint16_t* row = Wgu + k * 2 * F;
    *reinterpret_cast<u32x4v*>(Wg + k * F + c) = *reinterpret_cast<const u32x4v*>(row + gc);
    *reinterpret_cast<u32x4v*>(Wu + k * F + c) = *reinterpret_cast<const u32x4v*>(row + gc + 64);
  }
}

// grid: x covers a row's F/8 pieces; y = rows per pass, enough workgroups to
// fill the chip several times over
dim3 act_grid(int64_t rows, int64_t F) {
  const int64_t bx = (F / 8 + kActThreads - 1) / kActThreads;
  int64_t by = (2048 + bx - 1) / bx;
  if (by > rows) by = rows;
  if (by > 65535) by = 65535;
  return dim3(unsigned(bx), unsigned(by));
}

}  // namespace

hipError_t launch_swiglu_fwd_bf16(const void* GU, void* H, int64_t M, int64_t F, int q, hipStream_t s) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_fwd_kernel, act_grid(M, F), dim3(kActThreads), 0, s, static_cast<const uint16_t*>(GU),
                     static_cast<uint16_t*>(H), M, int(F), int(F / q));
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd_bf16(const void* GU, const void* dH, void* dGU, int64_t M, int64_t F, int q,
                                  hipStream_t s) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_bwd_kernel, act_grid(M, F), dim3(kActThreads), 0, s, static_cast<const uint16_t*>(GU),
                     static_cast<const uint16_t*>(dH), static_cast<uint16_t*>(dGU), M, int(F), int(F / q));
  return hipGetLastError();
}

hipError_t launch_split_gate_up_bf16(const void* Wgu, void* Wg, void* Wu, int64_t K, int64_t F, int q,
                                     hipStream_t s) {
  hipLaunchKernelGGL(split_gate_up_kernel, act_grid(K, F), dim3(kActThreads), 0, s,
                     static_cast<const uint16_t*>(Wgu), static_cast<uint16_t*>(Wg), static_cast<uint16_t*>(Wu), K,
                     int(F), int(F / q));
  return hipGetLastError();
}

}  // namespace qalg
