// Weight-streaming down-projection for int8 weights stored [in, out] with one scale per column, staged in LDS,
// gfx950.
//
// Expert FFN, page "A functional bridge between openai/grok and xai-org/grok-1" (architecture diagram): y = h W2;
// int8 weights times bf16 scales, page "Grok-1-BF16", section "Conversion Details".
//
// Same work split as down_stream_kernel (expert_stream.hip): one wave per 128 columns of W2 over one of S chunks of
// the f axis, the token rows of the expert in passes of 16 MT, fp32 partial sums to y[S, slots, d].  What differs is
// the path of the weights: each wave copies its [32 k][128 column] int8 piece of every K step straight into a ring
// of NST private LDS stages (global_load_lds_dwordx4: no registers held by loads in flight), together with the
// step's activation rows, and reads the MFMA B operands back with one ds_read_b64_tr_b8 per 16 columns (8
// consecutive k of one column per lane, no register transpose).  With two waves per SIMD each wave keeps NST - 1
// K steps of weights in flight (12 KB at NST = 4, where the register-staged kernel holds one step of 4 KB), which
// measured 2% faster on MI355X at NST = 3 (int8 weights at T = 16 and 64; the same staging for the up-projection,
// one wave per SIMD with 3 steps of both matrices in flight, was 2-4% slower than its register-staged kernel).
// With 32-row passes (MT = 2) the four waves share each step's activation rows (SH below): a quarter of the
// activation copies, and the LDS that frees holds a fourth weight stage; measured on MI355X at T = 64 (Grok-1
// shape, three alternating runs on one board): 0.282 -> 0.264 ms, 5.8 -> 6.2 TB/s.  Each output element is the same
// MFMA over the same k in the same order as in the register-staged kernel, so the results are bit-identical.
//
// LDS stage (per wave): weights [32 k rows][128 B], the 16-byte chunk m of k row k in slot m ^ 2 ((k >> 1) & 3)
// (the transpose reads of a 16-lane group then touch distinct banks); activations [MT][64 lanes][16 B]: lane l's
// A operand of block mt (row 16 mt + (l & 15) of the pass, k chunk l >> 4) at 16 l, copied by lane l of the wave
// (SH: of wave mt) and read by lane l of every wave that uses it.
// Rows past the expert's end get an out-of-range buffer offset: zeros, as the register-staged kernel multiplies.
#include "chunks.h"
#include "common.h"
#include "dma.h"
#include "launch.h"

namespace gm {

namespace {
constexpr int L_W = 32 * 128;  // bytes of one step's weights per wave
constexpr uint32_t L_OOR = 0x80000000u;

// The waits and copies below carry a memory clobber: each wave reads back what it copied, with no barrier between,
// so the compiler must not move LDS reads across them.
template <int N> __device__ __forceinline__ void wait_vm_mem() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 0..63");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
__device__ __forceinline__ void g2lds16_nt_mem(const void* base, uint32_t voff, uint32_t dst) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" : : "v"(voff), "s"(base), "s"(dst) : "m0", "memory");
}
__device__ __forceinline__ void b2lds16_mem(const u32x4_t& rsrc, uint32_t soff, uint32_t voff, uint32_t dst) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               : : "v"(voff), "s"(rsrc), "s"(soff), "s"(dst) : "m0", "memory");
}
}  // namespace

// SH: the workgroup's 4 waves (same expert, same f chunk, four 128-column slices) share each step's activation
// rows instead of each copying them: wave w < MT copies block w into a ring of NST + 1 shared slots, and one
// workgroup barrier per step, after every wave's copies of the step have landed, makes them visible.  A step's
// shared slot is copied over two steps after it was read, once every wave has passed the barrier that follows
// its reads, so the copies are still issued NST - 1 steps ahead without waiting for the other waves.  Waves past
// the last column stay in the loop for the barriers (they stream a valid slice and store nothing).
template <int MT, int NST, bool SH>
__global__ __launch_bounds__(256, 2) void down_stream_lds_kernel(const uint16_t* __restrict__ h,
                                                                 const int8_t* __restrict__ w2,
                                                                 const uint16_t* __restrict__ s2, int64_t s_estride,
                                                                 const int32_t* __restrict__ counts,
                                                                 const int32_t* __restrict__ offsets, uint32_t h_bytes,
                                                                 int d, int f, int S, int64_t split_stride,
                                                                 float* __restrict__ y) {
  static_assert(!SH || MT == 2, "shared activation rows: waves 0 and 1 copy the two 16-row blocks");
  constexpr int STG = SH ? L_W : L_W + MT * 1024;  // bytes of one stage of a wave's ring
  constexpr int NSA = NST + 1;                        // SH: shared activation slots
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * NST * STG + (SH ? NSA * MT * 1024 : 0)];
  const int e = blockIdx.z;
  const int n_e = counts[e];
  if (n_e == 0) return;  // whole workgroup
  const int off = offsets[e];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (blockIdx.x * 4 * 128 >= d) return;  // whole workgroup
  const bool live = (blockIdx.x * 4 + wave) * 128 < d;
  if (!SH && !live) return;  // no workgroup barrier without SH
  const int n0 = live ? (blockIdx.x * 4 + wave) * 128 : d - 128;
  const bool acopy = !SH || wave < MT;  // SH: waves 0 .. MT - 1 copy the activation blocks
  constexpr int CPS = 4 + (SH ? 1 : MT);  // copies per wave and K step (SH: 4 for the waves that copy no activations)
  const int kbeg = down_chunk_begin(blockIdx.y, f, S), kend = down_chunk_begin(blockIdx.y + 1, f, S);
  const int nsteps = (kend - kbeg) / 32;
  float* ys = y + int64_t(blockIdx.y) * split_stride;
  const int g = lane >> 4, c16 = lane & 15;

  lds_u8* ring = (lds_u8*)(smem) + wave * NST * STG;
  const uint32_t ring0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ring));
  lds_u8* aring = (lds_u8*)(smem) + 4 * NST * STG;  // SH: the shared activation slots
  const uint32_t aring0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(aring));
  // weight copy c of a step: lane writes k row 8 c + lane / 8, slot lane & 7, which holds chunk (lane & 7) ^ sw
  const int8_t* wbase = w2 + size_t(e) * f * d + n0;
  uint32_t w_voff[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int k = 8 * c + (lane >> 3);
    w_voff[c] = uint32_t(k * d + 16 * ((lane & 7) ^ (2 * ((k >> 1) & 3))));
  }
  // B fragment j (columns n0 + 16 j .. +15) of group g: lane 2 r + q addresses k row 8 g + r, columns 16 j + 8 q
  uint32_t b_off[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int k = 8 * g + (c16 >> 1);
    b_off[j] = uint32_t(k * 128 + 16 * (j ^ (2 * ((k >> 1) & 3))) + 8 * (c16 & 1));
  }
  const u32x4_t h_rsrc = buffer_rsrc(h, h_bytes);
  // scales of the lane's 8 columns n0 + 16 j + c16
  float sc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) sc[j] = bf16f(s2[size_t(e) * s_estride + n0 + 16 * j + c16]);

  for (int mb = 0; mb < n_e; mb += 16 * MT) {
    f32x4_t acc[MT][8];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[mt][j] = f32x4_t{0, 0, 0, 0};
    uint32_t a_voff[MT];  // lane's activation row of block mt, k chunk g (bytes from h)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mb + 16 * mt + c16;
      a_voff[mt] = m < n_e ? (uint32_t(off + m) * uint32_t(f) + 8u * uint32_t(g)) * 2u : L_OOR;
    }
    // the copies of step s (past the last step: the last step again, into a stage nobody reads)
    auto copy_step = [&](int s) {
      const int slot = s % NST;
      const int k0 = kbeg + 32 * min(s, nsteps - 1);
      const uint32_t st = ring0 + uint32_t(slot * STG);
#pragma unroll
      for (int c = 0; c < 4; ++c) g2lds16_nt_mem(wbase + size_t(k0) * d, w_voff[c], st + uint32_t(c * 1024));
      if constexpr (SH) {
        if (acopy)
          b2lds16_mem(h_rsrc, uint32_t(k0) * 2u, wave == 0 ? a_voff[0] : a_voff[MT - 1],
                      aring0 + uint32_t((s % NSA) * MT * 1024 + wave * 1024));
      } else {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          b2lds16_mem(h_rsrc, uint32_t(k0) * 2u, a_voff[mt], st + uint32_t(L_W + mt * 1024));
      }
    };
    if (nsteps > 0) {
#pragma unroll
      for (int s = 0; s < NST - 1; ++s) copy_step(s);
      for (int s = 0; s < nsteps; ++s) {
        asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");  // the reads of step s - 1 are complete ...
        copy_step(s + NST - 1);  // ... before its stage is copied over (SH: the shared slot of step s - 2)
        if (!SH || acopy) wait_vm_mem<CPS * (NST - 1)>();  // step s landed
        else wait_vm_mem<4 * (NST - 1)>();
        if constexpr (SH) lds_barrier();  // ... for every wave: the shared activations of step s are complete
        const lds_u8* st = ring + (s % NST) * STG;
        const lds_u8* sa = SH ? aring + (s % NSA) * (MT * 1024) : st + L_W;
        u32x4_t a[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          a[mt] = *(const __attribute__((address_space(3))) u32x4_t*)(sa + mt * 1024 + 16 * lane);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const u32x4_t b = i8x8_to_bf16(lds_tr8(st + b_off[j]));  // exact: |q| <= 127
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[mt][j] = mfma16x16x32(a[mt], b, acc[mt][j]);
        }
      }
      wait_vm_mem<0>();  // the copies past the last step (the next pass reuses the stages)
      if constexpr (SH) lds_barrier();  // every wave's reads of this pass are complete
    }
    // y rows mb + 16 mt + 4 g + v, column n0 + 16 j + c16 (the MFMA result layout)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = mb + 16 * mt + 4 * g + v;
        if (live && m < n_e) {
          float* dst = ys + size_t(off + m) * d + n0 + c16;
#pragma unroll
          for (int j = 0; j < 8; ++j) dst[16 * j] = acc[mt][j][v] * sc[j];
        }
      }
  }
}

// int8 [in, out] weights with one scale per column (scales [Es, 1, d] at expert stride s_estride): the
// LDS-staged down-projection above, same grid and chunks as launch_down_stream.
hipError_t launch_down_stream_lds(const uint16_t* h, const void* w2, const uint16_t* s2, int64_t s_estride,
                                  const int32_t* counts, const int32_t* offsets, int d, int f, int E, int slots,
                                  int S, int mt, float* y, hipStream_t s) {
  const size_t hbytes = size_t(slots) * f * 2;
  if (hbytes >= (size_t(1) << 31) || size_t(31) * d + 128 >= (size_t(1) << 31) || d % 128 != 0 || f % 128 != 0)
    return hipErrorInvalidValue;
  const dim3 grid((d + 511) / 512, S, E), block(256);
  const int64_t stride = int64_t(slots) * d;
  const int8_t* w = static_cast<const int8_t*>(w2);
  if (mt == 1)
    down_stream_lds_kernel<1, 4, false><<<grid, block, 0, s>>>(h, w, s2, s_estride, counts, offsets, uint32_t(hbytes),
                                                               d, f, S, stride, y);
  else
    down_stream_lds_kernel<2, 4, true><<<grid, block, 0, s>>>(h, w, s2, s_estride, counts, offsets, uint32_t(hbytes),
                                                              d, f, S, stride, y);
  return hipGetLastError();
}

}  // namespace gm
