// Gate-weighted combine of the Grok-1 MoE layer on gfx950.
//
// Page "Grok-1: 314B Total Parameters, 25B Active Per Token (MoE Explained)", section "How MoE Works in
// Practice": the layer output of a token is the sum over its selected experts of the expert output times that
// expert's router probability.  The down-projection may leave S partial sums per assignment (a split of the
// d_ff axis); they are added here in ascending order, so the result is deterministic.
//
// One workgroup of NT threads per (token, 4*NT-column block); each thread handles 4 consecutive outputs (16-byte
// loads and stores).  Small token counts use 64-thread workgroups so that the partial sums are read by enough
// workgroups to keep many loads in flight.
#include "common.h"
#include "launch.h"

namespace gm {

template <int NT>
__global__ __launch_bounds__(NT) void combine_kernel(const float* __restrict__ y, int S, int64_t split_stride,
                                                     const float* __restrict__ p, const int32_t* __restrict__ inv,
                                                     int d, float* __restrict__ out) {
  constexpr int COLS = 4 * NT;
  const int nblk = (d + COLS - 1) / COLS;
  const int t = blockIdx.x / nblk;
  const int c = (blockIdx.x - t * nblk) * COLS + threadIdx.x * 4;
  if (c >= d) return;
  const float p0 = p[2 * t], p1 = p[2 * t + 1];
  const float* y0 = y + int64_t(inv[2 * t]) * d + c;
  const float* y1 = y + int64_t(inv[2 * t + 1]) * d + c;
  f32x4_t a = *reinterpret_cast<const f32x4_t*>(y0);
  f32x4_t b = *reinterpret_cast<const f32x4_t*>(y1);
#pragma unroll 4
  for (int s = 1; s < S; ++s) {
    a += *reinterpret_cast<const f32x4_t*>(y0 + s * split_stride);
    b += *reinterpret_cast<const f32x4_t*>(y1 + s * split_stride);
  }
  f32x4_t o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = __fmaf_rn(p1, b[i], p0 * a[i]);
  *reinterpret_cast<f32x4_t*>(out + int64_t(t) * d + c) = o;
}

hipError_t launch_combine(const float* y, int S, const float* p, const int32_t* inv, int T, int d, float* out,
                          hipStream_t s) {
  const int64_t split_stride = int64_t(2) * T * d;
  if (int64_t(T) * ((d + 1023) / 1024) < 512) {
    const dim3 grid(unsigned((d + 255) / 256) * unsigned(T)), block(64);
    combine_kernel<64><<<grid, block, 0, s>>>(y, S, split_stride, p, inv, d, out);
  } else {
    const dim3 grid(unsigned((d + 1023) / 1024) * unsigned(T)), block(256);
    combine_kernel<256><<<grid, block, 0, s>>>(y, S, split_stride, p, inv, d, out);
  }
  return hipGetLastError();
}

// The post-MoE RMSNorm and the residual add of the layer ("Grok-1-BF16", section "Architecture": a norm after
// the MoE block; "... (MoE Explained)", section "Why JAX Instead of PyTorch": the block output is x plus the MoE
// branch): out[t] = x[t] + (o / sqrt(mean(o^2) + eps)) * g, with o the combined MoE output already in out.
// One workgroup per token: pass 1 forms the float64 sum of squares of o (each thread over its own columns in
// ascending order, then a fixed reduction tree), pass 2 rewrites each thread's own elements.
__global__ __launch_bounds__(256) void norm_residual_kernel(int d, const void* __restrict__ xres, bool bf16,
                                                            const void* __restrict__ g, double eps,
                                                            float* __restrict__ out) {
  __shared__ double ssq[4];
  const int t = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float* orow = out + int64_t(t) * d;
  double ss = 0.0;
#pragma unroll 4
  for (int c = threadIdx.x * 4; c < d; c += 1024) {
    const f32x4_t o = *reinterpret_cast<const f32x4_t*>(orow + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) ss = __fma_rn(double(o[i]), double(o[i]), ss);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if (lane == 0) ssq[wave] = ss;
  __syncthreads();
  const double rms = sqrt(((ssq[0] + ssq[1]) + (ssq[2] + ssq[3])) / double(d) + eps);
#pragma unroll 4
  for (int c = threadIdx.x * 4; c < d; c += 1024) {
    const f32x4_t o = *reinterpret_cast<const f32x4_t*>(orow + c);
    float xv[4], gv[4];
    if (bf16) {
      const u32x2_t xw = *reinterpret_cast<const u32x2_t*>(static_cast<const uint16_t*>(xres) + int64_t(t) * d + c);
      const u32x2_t gw = *reinterpret_cast<const u32x2_t*>(static_cast<const uint16_t*>(g) + c);
      xv[0] = bf16lo(xw[0]); xv[1] = bf16hi(xw[0]); xv[2] = bf16lo(xw[1]); xv[3] = bf16hi(xw[1]);
      gv[0] = bf16lo(gw[0]); gv[1] = bf16hi(gw[0]); gv[2] = bf16lo(gw[1]); gv[3] = bf16hi(gw[1]);
    } else {
      const f32x4_t xw = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(xres) + int64_t(t) * d + c);
      const f32x4_t gw = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(g) + c);
#pragma unroll
      for (int i = 0; i < 4; ++i) { xv[i] = xw[i]; gv[i] = gw[i]; }
    }
    f32x4_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = float(double(xv[i]) + (double(o[i]) / rms) * double(gv[i]));
    *reinterpret_cast<f32x4_t*>(orow + c) = r;
  }
}

// Combine (into out), then the norm and residual in place: two launches, so that the combine keeps its full
// width of workgroups.
hipError_t launch_combine_norm(const float* y, int S, const float* p, const int32_t* inv, int T, int d,
                               const void* xres, bool bf16, const void* g, double eps, float* out, hipStream_t s) {
  hipError_t e = launch_combine(y, S, p, inv, T, d, out, s);
  if (e != hipSuccess) return e;
  norm_residual_kernel<<<T, 256, 0, s>>>(d, xres, bf16, g, eps, out);
  return hipGetLastError();
}

}  // namespace gm
