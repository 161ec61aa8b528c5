// Router of the Grok-1 MoE layer on gfx950: gate GEMV, softmax over all experts, top-2.
//
// Page "Grok-1: 314B Total Parameters, 25B Active Per Token (MoE Explained)", section "Expert Routing Details":
// logits come from a Dense gate with one output per expert, the gates are the softmax of the logits (no noise
// at inference), and top_k with k = 2 returns the two largest gates with their indices.
//
// One workgroup of 4 waves per token, each thread striding over d in 8-element chunks.  (One thread per chunk, up to
// 1024 per workgroup, so that every load of the token is in flight at once, measured 1 us slower for routing and
// binning together at Grok-1 shape, T = 1 to 64, on MI355X.)  Each thread accumulates its products in fp64:
// a product of two bf16 (or two fp32) values is exact in fp64, so the only rounding is fp64 summation.  A fixed
// butterfly inside each wave and a fixed order across the waves make the result deterministic.  Selection runs
// on one wave with one lane per expert: the fp64 logits in descending order, the lower expert index first on
// equal logits (the same order as the probabilities, since softmax is strictly increasing), and the softmax
// denominator summed by a butterfly (every lane obtains the same sum).
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

// acc[e] += sum_i xv[i] * gate[e][k0 + i] (fp64 FMAs in ascending i) for the E experts.  The gate rows are loaded
// eight experts at a time with no branch between the loads, so that their memory latencies overlap instead of
// adding up; rows past E - 1 read row E - 1 again into partial logits that the top-2 selection never reads.
template <bool BF16, int EMAX>
__device__ __forceinline__ void gate_fma(const void* __restrict__ rw, int d, int E, int k0, const float xv[8],
                                         double acc[EMAX]) {
#pragma unroll
  for (int e0 = 0; e0 < EMAX; e0 += 8) {
    if (e0 < E) {
      float wv[8][8];
#pragma unroll
      for (int j = 0; j < 8; ++j) Vec8<BF16>::load(rw, int64_t(min(e0 + j, E - 1)) * d + k0, wv[j]);
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[e0 + j] = __fma_rn(double(xv[i]), double(wv[j][i]), acc[e0 + j]);
    }
  }
}

constexpr int kRouterWaves = 4;

// (value, index) order of the top-k: larger value first, lower index first on equal values.
__device__ __forceinline__ bool ranks_before(double a, int ia, double b, int ib) {
  return a > b || (a == b && ia < ib);
}

// The largest (value, index) pair over the wave, the same in every lane.
__device__ __forceinline__ void wave_top(double& v, int& i) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const double ov = __shfl_xor(v, off, 64);
    const int oi = __shfl_xor(i, off, 64);
    if (ranks_before(ov, oi, v, i)) { v = ov; i = oi; }
  }
}

// Selection from the per-wave partial logits part[w][e] (w < nw), called by one whole wave: lane e holds expert
// e's logit (partials summed in ascending w, then the bias), the two largest logits with the lower expert index
// first on equal logits, and their softmax probabilities over all E.  Lane 0 writes the results of token t.
template <int EMAX>
__device__ __forceinline__ void select_top2(const double (*part)[EMAX], int nw, const float* bias, int E, int t,
                                            int lane, int32_t* idx, float* p) {
  const bool valid = lane < E;
  double l = 0.0;
  if (valid) {
    l = part[0][lane];
    for (int w = 1; w < nw; ++w) l += part[w][lane];
    if (bias) l += double(bias[lane]);
  }
  double v1 = valid ? l : -__DBL_MAX__;
  int e1 = valid ? lane : 64 + lane;
  wave_top(v1, e1);
  double v2 = (valid && lane != e1) ? l : -__DBL_MAX__;
  int e2 = (valid && lane != e1) ? lane : 64 + lane;
  wave_top(v2, e2);
  double ex = valid ? exp(l - v1) : 0.0;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ex += __shfl_xor(ex, off, 64);
  if (lane == 0) {
    idx[2 * t] = e1;
    idx[2 * t + 1] = e2;
    p[2 * t] = float(1.0 / ex);
    p[2 * t + 1] = float(exp(v2 - v1) / ex);
  }
}

// Per-wave butterfly of the per-thread partial logits, then the selection by wave 0.
template <int EMAX>
__device__ __forceinline__ void reduce_select(double (&acc)[EMAX], double (*part)[EMAX], const float* bias, int E,
                                              int t, int32_t* idx, float* p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
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
  if (wave == 0) select_top2<EMAX>(part, nw, bias, E, t, lane, idx, p);
}

template <bool BF16, int EMAX>
__global__ __launch_bounds__(64 * kRouterWaves) void router_topk_kernel(const void* __restrict__ x, const void* __restrict__ rw,
                                                           const float* __restrict__ bias, int T, int d, int E,
                                                           int32_t* __restrict__ idx, float* __restrict__ p) {
  // One workgroup per token; thread i accumulates the 8-element chunks 8 i, 8 (i + blockDim), ... of d.
  __shared__ double part[kRouterWaves][EMAX];
  const int t = blockIdx.x;
  double acc[EMAX];
#pragma unroll
  for (int e = 0; e < EMAX; ++e) acc[e] = 0.0;
  const int64_t xrow = int64_t(t) * d;
  for (int k0 = 8 * threadIdx.x; k0 < d; k0 += 8 * blockDim.x) {
    float xv[8];
    Vec8<BF16>::load(x, xrow + k0, xv);
    gate_fma<BF16, EMAX>(rw, d, E, k0, xv, acc);
  }
  reduce_select<EMAX>(acc, part, bias, E, t, idx, p);
}

// float64 -> bf16 bit pattern with a single round-to-nearest-even step (bf16 keeps 8 significant bits, so 45
// of the 53 are dropped).  Finite values inside the float range.
__device__ __forceinline__ uint16_t f64_to_bf16(double v) {
  uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  u += 0xFFFFFFFFFFFull + ((u >> 45) & 1ull);  // half of 2^45, minus one, plus the kept LSB
  u &= ~((1ull << 45) - 1ull);
  const float f = static_cast<float>(__longlong_as_double(static_cast<long long>(u)));  // exact: 8 significant bits
  return static_cast<uint16_t>(__float_as_uint(f) >> 16);
}

// Router with the pre-MoE RMSNorm in front ("Grok-1-BF16", section "Architecture": four norms per layer, one
// before the MoE block): xn = x / sqrt(mean(x^2) + eps) * g in float64, stored once rounded to the activation
// type (bf16 round-to-nearest-even, or float32), and the router runs on the stored xn.  One workgroup per token:
// all 256 threads first reduce the sum of squares (fixed order), then each wave normalises its quarter of d,
// writes it, and accumulates the gate products exactly as router_topk_kernel.
template <bool BF16, int EMAX>
__global__ __launch_bounds__(256) void router_norm_kernel(const void* __restrict__ x, const void* __restrict__ g,
                                                          double eps, const void* __restrict__ rw,
                                                          const float* __restrict__ bias, int T, int d, int E,
                                                          void* __restrict__ xn, int32_t* __restrict__ idx,
                                                          float* __restrict__ p) {
  __shared__ double part[kRouterWaves][EMAX];
  __shared__ double ssq[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x;
  const int64_t xrow = int64_t(t) * d;
  double ss = 0.0;
  for (int k0 = threadIdx.x * 8; k0 < d; k0 += 2048) {
    float xv[8];
    Vec8<BF16>::load(x, xrow + k0, xv);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = __fma_rn(double(xv[i]), double(xv[i]), ss);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if (lane == 0) ssq[wave] = ss;
  __syncthreads();
  const double rms = sqrt(((ssq[0] + ssq[1]) + (ssq[2] + ssq[3])) / double(d) + eps);

  double acc[EMAX];
#pragma unroll
  for (int e = 0; e < EMAX; ++e) acc[e] = 0.0;
  const int q = d >> 2;
  const int kend = (wave + 1) * q;
  for (int k0 = wave * q + lane * 8; k0 < kend; k0 += 512) {
    float xv[8], gv[8], nv[8];
    Vec8<BF16>::load(x, xrow + k0, xv);
    Vec8<BF16>::load(g, k0, gv);
    if (BF16) {
      u32x4_t o;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = f64_to_bf16((double(xv[2 * j]) / rms) * double(gv[2 * j]));
        const uint32_t hi = f64_to_bf16((double(xv[2 * j + 1]) / rms) * double(gv[2 * j + 1]));
        o[j] = lo | (hi << 16);
        nv[2 * j] = bf16lo(o[j]);
        nv[2 * j + 1] = bf16hi(o[j]);
      }
      *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(xn) + xrow + k0) = o;
    } else {
      f32x4_t o0, o1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o0[i] = float((double(xv[i]) / rms) * double(gv[i]));
        o1[i] = float((double(xv[4 + i]) / rms) * double(gv[4 + i]));
        nv[i] = o0[i];
        nv[4 + i] = o1[i];
      }
      float* dst = static_cast<float*>(xn) + xrow + k0;
      *reinterpret_cast<f32x4_t*>(dst) = o0;
      *reinterpret_cast<f32x4_t*>(dst + 4) = o1;
    }
    gate_fma<BF16, EMAX>(rw, d, E, k0, nv, acc);
  }
  reduce_select<EMAX>(acc, part, bias, E, t, idx, p);
}

template <bool BF16>
static hipError_t launch_router_t(const void* x, const void* rw, const float* bias, int T, int d, int E, int32_t* idx,
                                  float* p, hipStream_t s) {
  const dim3 grid(T), block(64 * kRouterWaves);
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

template <bool BF16>
static hipError_t launch_router_norm_t(const void* x, const void* g, double eps, const void* rw, const float* bias,
                                       int T, int d, int E, void* xn, int32_t* idx, float* p, hipStream_t s) {
  const dim3 grid(T), block(256);
  if (E <= 8) router_norm_kernel<BF16, 8><<<grid, block, 0, s>>>(x, g, eps, rw, bias, T, d, E, xn, idx, p);
  else if (E <= 16) router_norm_kernel<BF16, 16><<<grid, block, 0, s>>>(x, g, eps, rw, bias, T, d, E, xn, idx, p);
  else if (E <= 32) router_norm_kernel<BF16, 32><<<grid, block, 0, s>>>(x, g, eps, rw, bias, T, d, E, xn, idx, p);
  else router_norm_kernel<BF16, 64><<<grid, block, 0, s>>>(x, g, eps, rw, bias, T, d, E, xn, idx, p);
  return hipGetLastError();
}

hipError_t launch_router_norm(const void* x, const void* g, double eps, const void* rw, const float* bias, int T,
                              int d, int E, bool is_bf16, void* xn, int32_t* idx, float* p, hipStream_t s) {
  return is_bf16 ? launch_router_norm_t<true>(x, g, eps, rw, bias, T, d, E, xn, idx, p, s)
                 : launch_router_norm_t<false>(x, g, eps, rw, bias, T, d, E, xn, idx, p, s);
}

}  // namespace gm
