// Measurement probes of the practical ceilings of one MI355X (gfx950); contracts in include/grok_moe_probe.h.
//
// Streaming HBM read (default or nontemporal 16-byte loads), dense bf16 MFMA on register operands with a
// checkable result and the clock it ran at, and a clock sampler that runs beside other work.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/grok_moe_probe.h"

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

namespace {

template <bool NT>
__device__ __forceinline__ u32x4_t ld16(const u32x4_t* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

// UNROLL independent 16-byte loads in flight per lane per iteration (the layer's weight streams keep about 16).
template <bool NT, int UNROLL>
__global__ __launch_bounds__(256) void read_kernel(const u32x4_t* __restrict__ p, size_t n16, uint32_t* sink) {
  const size_t stride = size_t(gridDim.x) * 256;
  size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (; i + (UNROLL - 1) * stride < n16; i += UNROLL * stride) {
    u32x4_t v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) v[u] = ld16<NT>(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= ld16<NT>(p + i);
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x ^= __shfl_xor(x, m, 64);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = x;
}

__device__ __forceinline__ f32x16_t mfma(const u32x4_t& a, const u32x4_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}

// Operand pair of MFMA m (0..15) of a round: ORDER 0 (the layer's tile kernels): blocks (i, j) row by row, so A
// fragment i stays for 4 MFMAs while B changes; ORDER 1: both fragments change at every MFMA, (m & 3, (m/4 + m) & 3);
// ORDER 2: the pair (0, 0) for all 16 (the operands never change).
template <int ORDER>
__device__ __forceinline__ int pair_a(int m) { return ORDER == 0 ? m >> 2 : ORDER == 1 ? m & 3 : 0; }
template <int ORDER>
__device__ __forceinline__ int pair_b(int m) { return ORDER == 0 ? m & 3 : ORDER == 1 ? ((m >> 2) + m) & 3 : 0; }

template <int ORDER>
__global__ __launch_bounds__(256) void mfma_kernel(const u32x4_t* __restrict__ ops, int iters,
                                                   float* __restrict__ checksum, uint64_t* __restrict__ clocks) {
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  u32x4_t a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = ops[i * 64 + lane];
    b[i] = ops[(4 + i) * 64 + lane];
  }
  f32x16_t acc[16];
#pragma unroll
  for (int m = 0; m < 16; ++m)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[m][v] = 0.0f;
  const uint64_t c0 = clock64(), w0 = wall_clock64();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 16; ++m) acc[m] = mfma(a[pair_a<ORDER>(m)], b[pair_b<ORDER>(m)], acc[m]);
  }
  const uint64_t c1 = clock64(), w1 = wall_clock64();
  float s = 0.0f;
#pragma unroll
  for (int m = 0; m < 16; ++m)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[m][v];
  checksum[w * 64 + lane] = s;
  if (lane == 0) {
    clocks[4 * w + 0] = c0;
    clocks[4 * w + 1] = c1;
    clocks[4 * w + 2] = w0;
    clocks[4 * w + 3] = w1;
  }
}

__global__ __launch_bounds__(64) void clock_kernel(uint64_t ticks, uint64_t* out) {
  const uint64_t c0 = clock64(), w0 = wall_clock64();
  for (int i = 0; i < (1 << 20); ++i) {  // bounded: every workgroup ends
    __builtin_amdgcn_s_sleep(127);
    if (wall_clock64() - w0 >= ticks) break;
  }
  const uint64_t c1 = clock64(), w1 = wall_clock64();
  if (threadIdx.x == 0) {
    out[4 * blockIdx.x + 0] = c0;
    out[4 * blockIdx.x + 1] = c1;
    out[4 * blockIdx.x + 2] = w0;
    out[4 * blockIdx.x + 3] = w1;
  }
}

inline bool aligned16(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
inline int status(hipError_t e) { return e == hipSuccess ? 0 : -4; }

}  // namespace

#define PROBE_API __attribute__((visibility("default")))

extern "C" {

PROBE_API int grok_moe_probe_read(const void* buf, size_t bytes, int workgroups, int nontemporal, uint32_t* sink,
                        hipStream_t stream) {
  if (!aligned16(buf) || sink == nullptr || bytes % 16 != 0 || workgroups < 1 || workgroups > (1 << 20)) return -1;
  const u32x4_t* p = static_cast<const u32x4_t*>(buf);
  if (nontemporal) read_kernel<true, 16><<<workgroups, 256, 0, stream>>>(p, bytes / 16, sink);
  else read_kernel<false, 16><<<workgroups, 256, 0, stream>>>(p, bytes / 16, sink);
  return status(hipGetLastError());
}

PROBE_API int grok_moe_probe_mfma(const uint16_t* ops, int iters, int order, float* checksum, uint64_t* clocks,
                                  hipStream_t stream) {
  if (!aligned16(ops) || checksum == nullptr || clocks == nullptr || iters < 1 || order < 0 || order > 2) return -1;
  const u32x4_t* o = reinterpret_cast<const u32x4_t*>(ops);
  if (order == 0) mfma_kernel<0><<<256, 256, 0, stream>>>(o, iters, checksum, clocks);
  else if (order == 1) mfma_kernel<1><<<256, 256, 0, stream>>>(o, iters, checksum, clocks);
  else mfma_kernel<2><<<256, 256, 0, stream>>>(o, iters, checksum, clocks);
  return status(hipGetLastError());
}

PROBE_API int grok_moe_probe_clock(int workgroups, uint64_t ticks, uint64_t* out, hipStream_t stream) {
  if (out == nullptr || workgroups < 1 || workgroups > 1024) return -1;
  clock_kernel<<<workgroups, 64, 0, stream>>>(ticks, out);
  return status(hipGetLastError());
}

PROBE_API int grok_moe_probe_wall_clock_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
  return khz;
}

}  // extern "C"
