// Router of the Grok-1 MoE layer on gfx950: gate GEMV, softmax over all experts, top-2.
//
// Page "Grok-1: 314B Total Parameters, 25B Active Per Token (MoE Explained)", section "Expert Routing Details":
// logits come from a Dense gate with one output per expert, the gates are the softmax of the logits (no noise
// at inference), and top_k with k = 2 returns the two largest gates with their indices.
//
// One workgroup of 4 waves per token (enough waves in flight even for a decode step of 8 tokens).  Each lane
// accumulates its strided share of the d products in fp64: a product of two bf16 (or two fp32) values is exact
// in fp64, so the only rounding is fp64 summation.  A fixed butterfly reduction inside each wave and a fixed
// order across the 4 waves make the result deterministic.  Selection uses the fp64 logits (descending, lower expert index on
// equal logits), which is the same order as the probabilities since softmax is strictly increasing.
#include "common.h"
#include "launch.h"

namespace gm {

template <bool BF16> struct Vec8;
template <> struct Vec8<true> {
  static __device__ __forceinline__ void load(const void* base, int64_t i, float v[8]) {
    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(base) + i);
#pragma unroll
    for (int j = 0; j < 4; ++j) { v[2 * j] = bf16lo(w[j]); v[2 * j + 1] = bf16hi(w[j]); }
  }
};
template <> struct Vec8<false> {
  static __device__ __forceinline__ void load(const void* base, int64_t i, float v[8]) {
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(base) + i);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(base) + i + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) { v[j] = a[j]; v[4 + j] = b[j]; }
  }
};

template <bool BF16, int EMAX>
__global__ __launch_bounds__(256) void router_topk_kernel(const void* __restrict__ x, const void* __restrict__ rw,
                                                          const float* __restrict__ bias, int T, int d, int E,
                                                          int32_t* __restrict__ idx, float* __restrict__ p) {
  // One workgroup (4 waves) per token; wave w accumulates the k in its quarter of d, lane-strided by 8.
  __shared__ double part[4][EMAX];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x;
  double acc[EMAX];
#pragma unroll
  for (int e = 0; e < EMAX; ++e) acc[e] = 0.0;
  const int64_t xrow = int64_t(t) * d;
  const int q = d >> 2;  // d is a multiple of 64, so each quarter is a multiple of 16
  const int kend = (wave + 1) * q;
  for (int k0 = wave * q + lane * 8; k0 < kend; k0 += 512) {
    float xv[8];
    Vec8<BF16>::load(x, xrow + k0, xv);
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      if (e < E) {
        float wv[8];
        Vec8<BF16>::load(rw, int64_t(e) * d + k0, wv);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[e] = __fma_rn(double(xv[i]), double(wv[i]), acc[e]);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc[e] += __shfl_xor(acc[e], off, 64);
  }
  if (lane == 0) {
#pragma unroll
    for (int e = 0; e < EMAX; ++e) part[wave][e] = acc[e];
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  double l[EMAX];
#pragma unroll
  for (int e = 0; e < EMAX; ++e)
    l[e] = (e < E) ? ((part[0][e] + part[1][e]) + (part[2][e] + part[3][e])) + (bias ? double(bias[e]) : 0.0) : 0.0;
  int e1 = 0;
#pragma unroll
  for (int e = 1; e < EMAX; ++e)
    if (e < E && l[e] > l[e1]) e1 = e;
  int e2 = -1;
  double l2 = 0.0, l1 = l[0];
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    if (e < E && e != e1 && (e2 < 0 || l[e] > l2)) { e2 = e; l2 = l[e]; }
    if (e == e1) l1 = l[e];
  }
  double s = 0.0;
#pragma unroll
  for (int e = 0; e < EMAX; ++e)
    if (e < E) s += exp(l[e] - l1);
  idx[2 * t] = e1;
  idx[2 * t + 1] = e2;
  p[2 * t] = float(1.0 / s);
  p[2 * t + 1] = float(exp(l2 - l1) / s);
}

template <bool BF16>
static hipError_t launch_router_t(const void* x, const void* rw, const float* bias, int T, int d, int E, int32_t* idx,
                                  float* p, hipStream_t s) {
  const dim3 grid(T), block(256);
  if (E <= 8) router_topk_kernel<BF16, 8><<<grid, block, 0, s>>>(x, rw, bias, T, d, E, idx, p);
  else if (E <= 16) router_topk_kernel<BF16, 16><<<grid, block, 0, s>>>(x, rw, bias, T, d, E, idx, p);
  else if (E <= 32) router_topk_kernel<BF16, 32><<<grid, block, 0, s>>>(x, rw, bias, T, d, E, idx, p);
  else router_topk_kernel<BF16, 64><<<grid, block, 0, s>>>(x, rw, bias, T, d, E, idx, p);
  return hipGetLastError();
}

hipError_t launch_router(const void* x, const void* rw, const float* bias, int T, int d, int E, bool is_bf16,
                         int32_t* idx, float* p, hipStream_t s) {
  return is_bf16 ? launch_router_t<true>(x, rw, bias, T, d, E, idx, p, s)
                 : launch_router_t<false>(x, rw, bias, T, d, E, idx, p, s);
}

}  // namespace gm
