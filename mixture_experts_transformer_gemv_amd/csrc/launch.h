// Internal launchers of the gfx950 kernels (host side).  Each returns hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gm {

// Layout of int8 scales [Es, G, N] ("Grok-1-BF16", section "Conversion Details": scales broadcast over groups):
// the scale of (expert e, group g, column n) is at e * estride + g * N + n (estride = G * N, or 0 when all
// experts share one scale tensor); a group is gsize consecutive input rows (gsize == K: one group).
struct ScaleLayout {
  int64_t estride;
  int gsize;
};

// Router: fp64 gate GEMV, softmax over E, top-2 (lower index first on ties).  is_bf16 selects the input type.
hipError_t launch_router(const void* x, const void* rw, const float* bias, int T, int d, int E, bool is_bf16,
                         int32_t* idx, float* p, hipStream_t s);

// Router with the pre-MoE RMSNorm in front: writes xn [T,d] (activation type) and routes on it.
hipError_t launch_router_norm(const void* x, const void* g, double eps, const void* rw, const float* bias, int T,
                              int d, int E, bool is_bf16, void* xn, int32_t* idx, float* p, hipStream_t s);

// Combine, then the post-MoE RMSNorm and the residual add: out = x + RMSNorm(combined, g, eps).
hipError_t launch_combine_norm(const float* y, int S, const float* p, const int32_t* inv, int T, int d,
                               const void* xres, bool bf16, const void* g, double eps, float* out, hipStream_t s);

// Histogram + scan + stable permutation of the k = 2 assignments per token (one workgroup).
hipError_t launch_bin(const int32_t* idx, int T, int E, int32_t* counts, int32_t* offsets, int32_t* perm,
                      int32_t* inv, hipStream_t s);
hipError_t launch_counts_out(int32_t* dst, const int32_t* src, int E, bool add, hipStream_t s);

// Combine: out[t] = sum_j p[t,j] * sum_s y[s, inv[t,j]].
hipError_t launch_combine(const float* y, int S, const float* p, const int32_t* inv, int T, int d, float* out,
                          hipStream_t s);

// Streaming (few tokens per expert) expert kernels: weights go HBM -> registers -> MFMA, no LDS tiling.
// mt = number of 16-row MFMA tiles held per pass (1 or 2).
// outin: weights stored [E, out, in] instead of [E, in, out].
// 4 if the streaming up-projection splits d over the waves of a workgroup (small f), else 1; the [in, out] and
// [out, in] streaming kernels split alike.
int up_stream_ksplit(int d, int f, int E);
// true if launch_up_stream runs the 64-column bf16 kernel for this shape (slots = k T)
bool up_stream_narrow(int d, int f, int E, int slots, bool int8, bool outin, int mt);
hipError_t launch_up_stream(const uint16_t* x, const void* w1, const void* wv, const uint16_t* s1,
                            const uint16_t* sv, ScaleLayout sl, bool outin, const int32_t* counts,
                            const int32_t* offsets, const int32_t* perm, int d, int f, int E, int slots, bool int8,
                            int mt, uint16_t* h, hipStream_t s);
hipError_t launch_down_stream(const uint16_t* h, const void* w2, const uint16_t* s2, ScaleLayout sl, bool outin,
                              const int32_t* counts, const int32_t* offsets, int d, int f, int E, int slots, int S,
                              bool int8, int mt, float* y, hipStream_t s);

// int8 [in, out] weights with one scale per column (scales at expert stride s_estride): the weight-streaming
// down-projection with the weights staged in per-wave LDS rings (deeper streams than registers allow).
hipError_t launch_down_stream_lds(const uint16_t* h, const void* w2, const uint16_t* s2, int64_t s_estride,
                                  const int32_t* counts, const int32_t* offsets, int d, int f, int E, int slots,
                                  int S, int mt, float* y, hipStream_t s);

// Streaming kernels for weights stored [E, out, in]: weight rows staged in LDS by direct copies of 256-byte
// pieces.  mt = 16-row token tiles per pass (1 or 2).  Usable when oi_stream_fits(K chunk, ...).
bool oi_stream_fits(int Kc, bool int8, ScaleLayout sl, int K);
int oi_up_blocks(int f, int E, int slots);
hipError_t launch_up_stream_oi(const uint16_t* x, const void* w1, const void* wv, const uint16_t* s1,
                               const uint16_t* sv, ScaleLayout sl, const int32_t* counts, const int32_t* offsets,
                               const int32_t* perm, int d, int f, int E, int slots, bool int8, int mt,
                               uint16_t* h, hipStream_t s);
hipError_t launch_down_stream_oi(const uint16_t* h, const void* w2, const uint16_t* s2, ScaleLayout sl,
                                 const int32_t* counts, const int32_t* offsets, int d, int f, int E, int slots,
                                 int S, bool int8, int mt, float* y, hipStream_t s);

// LDS-tiled grouped GEMMs (many tokens per expert): the direct-to-LDS kernels below for bf16 weights and for int8
// weights with one scale group in [in, out] storage; register-staged tiles for int8 with grouped scales or in
// [out, in] storage.
hipError_t launch_up_tiled(const uint16_t* x, const void* w1, const void* wv, const uint16_t* s1,
                           const uint16_t* sv, ScaleLayout sl, bool outin, const int32_t* counts,
                           const int32_t* offsets, const int32_t* perm, int d, int f, int E, int slots, bool int8,
                           uint16_t* h, hipStream_t s);
hipError_t launch_down_tiled(const uint16_t* h, const void* w2, const uint16_t* s2, ScaleLayout sl, bool outin,
                             const int32_t* counts, const int32_t* offsets, int d, int f, int E, int slots, int S,
                             bool int8, float* y, hipStream_t s);

// Grouped int8 scales on the direct-to-LDS tiles ([in, out] weights, K / gsize <= 8 groups along K; 128-row tiles).
bool tiled_dma_grouped_fits(int K, int gsize);
hipError_t launch_up_tiled_dma_grouped(const uint16_t* x, const void* w1, const void* wv, const uint16_t* s1,
                                       const uint16_t* sv, int64_t s_estride, int gsize, const int32_t* counts,
                                       const int32_t* offsets, const int32_t* perm, int d, int f, int E, int slots,
                                       uint16_t* h, hipStream_t s);
hipError_t launch_down_tiled_dma_grouped(const uint16_t* h, const void* w2, const uint16_t* s2, int64_t s_estride,
                                         int gsize, const int32_t* counts, const int32_t* offsets, int d, int f,
                                         int E, int slots, int S, float* y, hipStream_t s);
// Direct global -> LDS copies, LDS transpose reads for [in, out] weights (bf16, or int8 with per-column scales
// [Es, 1, N] at expert stride s_estride).
hipError_t launch_up_tiled_dma(const uint16_t* x, const void* w1, const void* wv, const uint16_t* s1,
                               const uint16_t* sv, int64_t s_estride, bool int8, bool outin, const int32_t* counts,
                               const int32_t* offsets, const int32_t* perm, int d, int f, int E, int slots,
                               uint16_t* h, hipStream_t s);
hipError_t launch_down_tiled_dma(const uint16_t* h, const void* w2, const uint16_t* s2, int64_t s_estride, bool int8,
                                 bool outin, const int32_t* counts, const int32_t* offsets, int d, int f, int E,
                                 int slots, int S, float* y, hipStream_t s);
// The up-projection's 256-row tiles for bf16 [in, out] weights in one persistent launch (one workgroup per CU;
// d / 32 >= 8).
hipError_t launch_up_persist(const uint16_t* x, const void* w1, const void* wv, const int32_t* counts,
                             const int32_t* perm, int d, int f, int E, int slots, uint16_t* h, hipStream_t s);

// fp32 layer (VALU, LDS tiles).
hipError_t launch_up_f32(const float* x, const float* w1, const float* wv, bool outin, const int32_t* counts,
                         const int32_t* offsets, const int32_t* perm, int d, int f, int E, int slots, float* h,
                         hipStream_t s);
hipError_t launch_down_f32(const float* h, const float* w2, bool outin, const int32_t* counts,
                           const int32_t* offsets, int d, int f, int E, int slots, int S, float* y, hipStream_t s);

// Tile scheduling shared by the grouped kernels: the m-th row tile (of height bm) over all experts in
// ascending expert order.  Returns false if m is past the last tile.  counts has E entries.
__device__ __forceinline__ bool find_row_tile(const int32_t* counts, const int32_t* offsets, int E, int bm, int m,
                                              int* e_out, int* row0_out, int* rows_out) {
  int base = 0;
  for (int e = 0; e < E; ++e) {
    const int n = counts[e];
    const int tiles = (n + bm - 1) / bm;
    if (m < base + tiles) {
      const int r = (m - base) * bm;
      *e_out = e;
      *row0_out = offsets[e] + r;
      *rows_out = min(bm, n - r);
      return true;
    }
    base += tiles;
  }
  return false;
}

}  // namespace gm
