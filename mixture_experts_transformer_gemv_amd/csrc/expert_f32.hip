// Expert matrix products of the fp32 Grok-1-style MoE layer on gfx950 (vector ALU, LDS tiles).
//
// Expert FFN, page "A functional bridge between openai/grok and xai-org/grok-1" (architecture diagram):
// y = (GELU(x W1) (*) (x Wv)) W2.  In the fp32 layer h = GELU(a) * b stays fp32.
//
// Grouped over the expert-sorted slots like the bf16 kernels: a workgroup of 256 threads computes a 64-row x
// 64-column tile (per matrix; NMAT = 2 computes the same columns of W1 and Wv), 4 x 4 outputs per thread,
// with 16-deep K steps staged through LDS.  Weights stored [E, in, out] are copied row by row; weights stored
// [E, out, in] (OUTIN) are read as 4 consecutive k of one column per thread and transposed into the same
// [k][column] LDS tile.
#include "common.h"
#include "launch.h"

namespace gm {

namespace {
constexpr int FBM = 64, FBN = 64, FBK = 16;
}

template <int NMAT, bool OUTIN>
__global__ __launch_bounds__(256) void f32_tiled_kernel(const float* __restrict__ A, const float* __restrict__ B0,
                                                        const float* __restrict__ B1,
                                                        const int32_t* __restrict__ counts,
                                                        const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ perm, int K, int N, int E,
                                                        float* __restrict__ out, int64_t split_stride) {
  int e, row0, rows;
  if (!find_row_tile(counts, offsets, E, FBM, blockIdx.x, &e, &row0, &rows)) return;
  __shared__ float As[FBK][FBM + 4];
  __shared__ float Bs[NMAT][FBK][FBN + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int nbase = blockIdx.y * FBN;
  // split blockIdx.z of gridDim.z covers k in [kbase, kbase + Ks) (NMAT = 1: partial sums, added by the combine)
  const int Ks = K / gridDim.z, kbase = blockIdx.z * Ks;
  out += blockIdx.z * split_stride;

  // A piece: row tid/4, k 4 (tid%4) .. +3
  const int ar = tid >> 2, ak = 4 * (tid & 3);
  const int arr = min(ar, rows - 1);
  const size_t arow = (NMAT == 2) ? size_t(perm[row0 + arr]) : size_t(row0 + arr);
  const float* a_src = A + arow * K + ak;
  // B piece: [in, out]: k row tid/16, columns 4 (tid%16) .. +3; [out, in]: column tid/4, k 4 (tid%4) .. +3
  const int bk = OUTIN ? 4 * (tid & 3) : tid >> 4, bn = OUTIN ? tid >> 2 : 4 * (tid & 15);
  const size_t b_off = OUTIN ? size_t(e) * K * N + size_t(nbase + bn) * K + bk
                             : size_t(e) * K * N + size_t(bk) * N + nbase + bn;

  float acc[NMAT][4][4];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[m][i][j] = 0.0f;

  for (int k0 = kbase; k0 < kbase + Ks; k0 += FBK) {
    const f32x4_t av = *reinterpret_cast<const f32x4_t*>(a_src + k0);
#pragma unroll
    for (int i = 0; i < 4; ++i) As[ak + i][ar] = av[i];
    if (OUTIN) {
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        const f32x4_t bv = *reinterpret_cast<const f32x4_t*>((m ? B1 : B0) + b_off + k0);
#pragma unroll
        for (int i = 0; i < 4; ++i) Bs[m][bk + i][bn] = bv[i];
      }
    } else {
      *reinterpret_cast<f32x4_t*>(&Bs[0][bk][bn]) = *reinterpret_cast<const f32x4_t*>(B0 + b_off + size_t(k0) * N);
      if (NMAT == 2)
        *reinterpret_cast<f32x4_t*>(&Bs[NMAT - 1][bk][bn]) =
            *reinterpret_cast<const f32x4_t*>(B1 + b_off + size_t(k0) * N);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FBK; ++kk) {
      float a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        float b[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = Bs[m][kk][tx * 4 + j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[m][i][j] = __fmaf_rn(a[i], b[j], acc[m][i][j]);
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = ty * 4 + i;
    if (r < rows) {
      f32x4_t o;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = (NMAT == 2) ? gelu_erf(acc[0][i][j]) * acc[NMAT - 1][i][j] : acc[0][i][j];
      *reinterpret_cast<f32x4_t*>(out + size_t(row0 + r) * N + nbase + tx * 4) = o;
    }
  }
}

hipError_t launch_up_f32(const float* x, const float* w1, const float* wv, bool outin, const int32_t* counts,
                         const int32_t* offsets, const int32_t* perm, int d, int f, int E, int slots, float* h,
                         hipStream_t s) {
  const dim3 grid(slots / FBM + E, f / FBN), block(256);
  if (outin) f32_tiled_kernel<2, true><<<grid, block, 0, s>>>(x, w1, wv, counts, offsets, perm, d, f, E, h, 0);
  else f32_tiled_kernel<2, false><<<grid, block, 0, s>>>(x, w1, wv, counts, offsets, perm, d, f, E, h, 0);
  return hipGetLastError();
}

hipError_t launch_down_f32(const float* h, const float* w2, bool outin, const int32_t* counts,
                           const int32_t* offsets, int d, int f, int E, int slots, int S, float* y, hipStream_t s) {
  if (S < 1 || f % (S * FBK) != 0) return hipErrorInvalidValue;
  const dim3 grid(slots / FBM + E, d / FBN, S), block(256);
  const int64_t stride = int64_t(slots) * d;
  if (outin)
    f32_tiled_kernel<1, true><<<grid, block, 0, s>>>(h, w2, nullptr, counts, offsets, nullptr, f, d, E, y, stride);
  else
    f32_tiled_kernel<1, false><<<grid, block, 0, s>>>(h, w2, nullptr, counts, offsets, nullptr, f, d, E, y, stride);
  return hipGetLastError();
}

}  // namespace gm
