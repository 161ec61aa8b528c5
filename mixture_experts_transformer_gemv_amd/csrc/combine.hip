// Gate-weighted combine of the Grok-1 MoE layer on gfx950.
//
// Page "Grok-1: 314B Total Parameters, 25B Active Per Token (MoE Explained)", section "How MoE Works in
// Practice": the layer output of a token is the sum over its selected experts of the expert output times that
// expert's router probability.  The down-projection may leave S partial sums per assignment (a split of the
// d_ff axis); they are added here in ascending order, so the result is deterministic.
//
// One workgroup per (token, 1024-column block); each thread handles 4 consecutive outputs (16-byte loads and stores).
#include "common.h"
#include "launch.h"

namespace gm {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, int S, int64_t split_stride,
                                                      const float* __restrict__ p, const int32_t* __restrict__ inv,
                                                      int d, float* __restrict__ out) {
  const int nblk = (d + 1023) >> 10;
  const int t = blockIdx.x / nblk;
  const int c = (blockIdx.x - t * nblk) * 1024 + threadIdx.x * 4;
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
  const dim3 grid(unsigned((d + 1023) / 1024) * unsigned(T)), block(256);
  combine_kernel<<<grid, block, 0, s>>>(y, S, split_stride, p, inv, d, out);
  return hipGetLastError();
}

}  // namespace gm
