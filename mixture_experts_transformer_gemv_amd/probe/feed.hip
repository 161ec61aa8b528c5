// Probe of what feeding the MFMAs costs (gfx950); contract in include/grok_moe_probe.h.
//
// The K loop of the 256 x 256 prefill tiles without the layer around it: one workgroup of 4 waves per CU, each wave
// a 128 x 128 block of accumulators (4 x 4 blocks of v_mfma_f32_32x32x16_bf16, the order of the tile kernels), a
// 4-stage LDS ring of 32 KB stages, the operand fragments of each half K step read from LDS while the MFMAs of the
// other half run, one barrier per step between its halves.  With copies, every step also copies the stage of the
// step three ahead from global memory into the ring (8 direct-to-LDS copies of 1 KB per wave, the copy bytes per
// flop of the tile kernels), from a small source that stays in L2; without, the ring is filled once and the steps
// cycle through it.  The results are real: the caller checks the sums.
#include "../csrc/dma.h"

#include "../../include/grok_moe_probe.h"

namespace gm {
namespace {

constexpr int F_STAGE = 32768;  // bytes of one ring stage and of one source image
constexpr int F_FRAG = 1024;    // one operand fragment: 64 lanes x 16 bytes

// Fragments of a stage: A (wm, ks, i) at ((wm * 2 + ks) * 4 + i) * 1 KB, B (wn, ks, j) at 16 KB + the same with
// wn, j.  Lane l of a fragment holds row (A) or column (B) l & 31, k = 8 (l >> 5) .. +7 of its 32 x 16 operand.
__device__ __forceinline__ int frag_a(int wm, int ks, int i) { return ((wm * 2 + ks) * 4 + i) * F_FRAG; }
__device__ __forceinline__ int frag_b(int wn, int ks, int j) { return 16384 + ((wn * 2 + ks) * 4 + j) * F_FRAG; }

template <bool COPY>
__global__ __launch_bounds__(256) void feed_kernel(const uint8_t* __restrict__ src, int nimg, int iters,
                                                   float* __restrict__ checksum, uint64_t* __restrict__ clocks) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * F_STAGE];
  lds_u8* lds = (lds_u8*)smem;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // the wave's 8 copies of a stage: 1 KB chunks 8 wave .. 8 wave + 7 of the image, each to the same place in the
  // ring slot (lane l moves bytes 16 l .. +15 of its chunk)
  auto copy = [&](int step, int n) {
    const int img = step % nimg;  // step >= 0
    const int c = 8 * wave + n;
    g2lds16(src + size_t(img) * F_STAGE + size_t(c) * F_FRAG, uint32_t(lane) * 16u,
            lds0 + uint32_t(step & 3) * F_STAGE + uint32_t(c) * F_FRAG);
  };
  u32x4_t fa[2][4], fb[2][4];
  auto read = [&](int buf, int step, int ks, int p) {  // fragment p of half ks: 0..3 A blocks, 4..7 B blocks
    const lds_u8* st = lds + (step & 3) * F_STAGE + lane * 16;
    if (p < 4) fa[buf][p] = *(const __attribute__((address_space(3))) u32x4_t*)(st + frag_a(wm, ks, p));
    else fb[buf][p - 4] = *(const __attribute__((address_space(3))) u32x4_t*)(st + frag_b(wn, ks, p - 4));
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // prologue: stages 0, 1, 2 (with copies), or all four (without), then step 0's first fragments
#pragma unroll
  for (int s = 0; s < (COPY ? 3 : 4); ++s)
#pragma unroll
    for (int n = 0; n < 8; ++n) copy(s, n);
  if constexpr (COPY) wait_vm<16>();  // stage 0 landed
  else wait_vm<0>();
  lds_barrier();
  const uint64_t c0 = clock64(), w0 = wall_clock64();
#pragma unroll
  for (int p = 0; p < 8; ++p) read(0, 0, 0, p);

  for (int it = 0; it < iters; ++it) {
    // half 0: MFMAs of half 0 of step it; fragments of its half 1; the first 4 copies of step it + 3
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      acc[m >> 2][m & 3] = mfma32x32x16(fa[0][m >> 2], fb[0][m & 3], acc[m >> 2][m & 3]);
      if (m < 8) read(1, it, 1, m);
      if (COPY && (m & 3) == 0) copy(it + 3, m >> 2);
      __builtin_amdgcn_sched_barrier(0);
    }
    // step it + 1 landed: issued after its copies are step it + 2's 8 and step it + 3's first 4
    if constexpr (COPY) wait_vm<12>();
    lds_barrier();
    // half 1: MFMAs of half 1; fragments of half 0 of step it + 1; the last 4 copies of step it + 3
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      acc[m >> 2][m & 3] = mfma32x32x16(fa[1][m >> 2], fb[1][m & 3], acc[m >> 2][m & 3]);
      if (m < 8) read(0, it + 1, 0, m);
      if (COPY && (m & 3) == 0) copy(it + 3, 4 + (m >> 2));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  const uint64_t c1 = clock64(), w1 = wall_clock64();
  wait_vm<0>();  // no copy may land in LDS after the workgroup ends

  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) s += acc[i][j][v];
  const int w = blockIdx.x * 4 + wave;
  checksum[w * 64 + lane] = s;
  if (lane == 0) {
    clocks[4 * w + 0] = c0;
    clocks[4 * w + 1] = c1;
    clocks[4 * w + 2] = w0;
    clocks[4 * w + 3] = w1;
  }
}

}  // namespace
}  // namespace gm

extern "C" __attribute__((visibility("default"))) int grok_moe_probe_mfma_feed(const void* src, int64_t src_bytes,
                                                                               int iters, int copies, float* checksum,
                                                                               uint64_t* clocks, hipStream_t stream) {
  using namespace gm;
  if (src == nullptr || (reinterpret_cast<uintptr_t>(src) & 15) != 0 || checksum == nullptr || clocks == nullptr ||
      iters < 1 || iters > (1 << 30) || src_bytes % F_STAGE != 0 || src_bytes < 4 * F_STAGE ||
      src_bytes > (int64_t(1) << 30) || (copies != 0 && copies != 1))
    return -1;
  const int nimg = int(src_bytes / F_STAGE);
  const uint8_t* s = static_cast<const uint8_t*>(src);
  if (copies) feed_kernel<true><<<256, 256, 0, stream>>>(s, nimg, iters, checksum, clocks);
  else feed_kernel<false><<<256, 256, 0, stream>>>(s, nimg, iters, checksum, clocks);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
