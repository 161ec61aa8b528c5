// Token binning of the Grok-1 MoE layer on gfx950: per-expert histogram, exclusive prefix sum and a stable
// permutation of the 2T (token, selected expert) assignments, grouped by expert.
//
// Page "Grok-1: 314B Total Parameters, 25B Active Per Token (MoE Explained)", section "How MoE Works in
// Practice": each token is routed to a subset (two) of the experts.  Grouping the assignments by expert turns
// the per-token expert calls into one matrix product per expert.
//
// One workgroup of NT threads: 1024 (16 waves), or one wave for at most 64 tokens, where the barriers of 16
// waves cost more than the work.  Counts use LDS integer atomics (exact, order-free).  The scatter walks the
// tokens in chunks of NT in ascending order; within a chunk each wave ranks its lanes with a
// ballot and popcount, and waves are ordered by a scan over per-wave counts, so slots of one expert are in
// ascending token order.
#include "common.h"
#include "launch.h"

namespace gm {

template <int NT>
__global__ __launch_bounds__(NT) void bin_tokens_kernel(const int32_t* __restrict__ idx, int T, int E,
                                                          int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  __shared__ int s_cnt[64];
  __shared__ int s_base[64];
  constexpr int NW = NT / 64;
  __shared__ int s_wc[64][NW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < E) s_cnt[tid] = 0;
  __syncthreads();
  for (int t = tid; t < T; t += NT) {
    atomicAdd(&s_cnt[idx[2 * t]], 1);
    atomicAdd(&s_cnt[idx[2 * t + 1]], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int e = 0; e < E; ++e) {
      s_base[e] = run;
      offsets[e] = run;
      counts[e] = s_cnt[e];
      run += s_cnt[e];
    }
    offsets[E] = run;
  }
  __syncthreads();
  const uint64_t lt = (uint64_t(1) << lane) - 1;
  for (int c0 = 0; c0 < T; c0 += NT) {
    const int t = c0 + tid;
    const bool valid = t < T;
    const int e0 = valid ? idx[2 * t] : -1;
    const int e1 = valid ? idx[2 * t + 1] : -1;
    int r0 = 0, r1 = 0;
    for (int e = 0; e < E; ++e) {
      const uint64_t m = __ballot(e0 == e || e1 == e);
      if (lane == 0) s_wc[e][wave] = __popcll(m);
      if (e == e0) r0 = __popcll(m & lt);
      if (e == e1) r1 = __popcll(m & lt);
    }
    __syncthreads();
    if (valid) {
      int p0 = s_base[e0] + r0, p1 = s_base[e1] + r1;
      for (int w = 0; w < wave; ++w) {
        p0 += s_wc[e0][w];
        p1 += s_wc[e1][w];
      }
      perm[p0] = t;
      perm[p1] = t;
      inv[2 * t] = p0;
      inv[2 * t + 1] = p1;
    }
    __syncthreads();
    if (tid < E) {
      int s = 0;
      for (int w = 0; w < NW; ++w) s += s_wc[tid][w];
      s_base[tid] += s;
    }
    __syncthreads();
  }
}

hipError_t launch_bin(const int32_t* idx, int T, int E, int32_t* counts, int32_t* offsets, int32_t* perm,
                      int32_t* inv, hipStream_t s) {
  if (T <= 64)
    bin_tokens_kernel<64><<<1, 64, 0, s>>>(idx, T, E, counts, offsets, perm, inv);
  else
    bin_tokens_kernel<1024><<<1, 1024, 0, s>>>(idx, T, E, counts, offsets, perm, inv);
  return hipGetLastError();
}

// Per-expert counts of one pass written (add = 0) or added (add = 1) to the caller's array, E <= 64.
__global__ __launch_bounds__(64) void counts_out_kernel(int32_t* __restrict__ dst, const int32_t* __restrict__ src,
                                                        int E, int add) {
  const int e = threadIdx.x;
  if (e < E) dst[e] = add ? dst[e] + src[e] : src[e];
}

hipError_t launch_counts_out(int32_t* dst, const int32_t* src, int E, bool add, hipStream_t s) {
  counts_out_kernel<<<1, 64, 0, s>>>(dst, src, E, add ? 1 : 0);
  return hipGetLastError();
}

}  // namespace gm
