// LDS-tiled grouped GEMM with direct global -> LDS copies and LDS transpose reads (bf16 weights), gfx950.
//
// Expert FFN, page "A functional bridge between openai/grok and xai-org/grok-1" (architecture diagram):
// y = (GELU(x W1) (*) (x Wv)) W2.
//
// Tile shape, order and epilogue: tiles.h.  K steps of 32 in a 4-deep LDS ring (4 x 32 KB).  Both operands
// are copied straight from global memory into LDS with global_load_lds_dwordx4 (no registers, no VALU), 16
// bytes per lane:
//   * A tile [256 rows][32 k], 64-byte rows; the 16-byte k chunk c of row r sits in slot c ^ ((r >> 2) & 3);
//   * B tile [32 k][256 columns], 512-byte rows; the 8-column chunk c of row k sits in slot c ^ (4 (k & 3)).
// The XOR swizzles are chosen on the global side (which chunk each lane fetches), so that the MFMA operand
// reads below hit distinct LDS banks.  A fragments are 16-byte reads; the weights are stored [in, out]
// (columns contiguous), so their MFMA fragments (8 consecutive k of one column per lane) come from two
// ds_read_b64_tr_b16: within each 16-lane group, lane j receives element j % 4 of the 8 bytes addressed by lane
// 4 r + j / 4 (r = 0..3), i.e. 4 consecutive k of one column when four lanes address four consecutive k rows.
// One workgroup barrier per K step, placed between the step's two 16-deep halves: the first half of step kt+1
// is read from LDS while the second half of step kt is multiplied.
#include "common.h"
#include "launch.h"
#include "tiles.h"

// The copies are issued from inline assembly (they only set M0, no destination register).
#pragma clang diagnostic ignored "-Winline-asm"

namespace gm {

namespace {
using tile::BM;
using tile::BNT;
constexpr int BK = 32;                  // K per ring stage
constexpr int NSTAGE = 4;               // ring depth
constexpr int A_STAGE = BM * BK * 2;    // bytes
constexpr int B_STAGE = BK * BNT * 2;   // bytes
constexpr int STAGE = A_STAGE + B_STAGE;
}

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef short i16x4_t __attribute__((ext_vector_type(4)));

// 16-byte global -> LDS copy: lane i of the wave writes LDS bytes [dst + 16 i, dst + 16 i + 16); dst is
// wave-uniform.  Issued as inline assembly so that the compiler does not wait for every copy in flight before
// each LDS read (it cannot tell the ring stages apart); completion is awaited explicitly with vmcnt before the
// workgroup barrier of the stage.  No "memory" clobber: the barrier sequence below orders the LDS accesses.
__device__ __forceinline__ void g2lds16(const void* src, const lds_u8* dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst)));
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(m0) : "m0");
}

// LDS transpose read (see the header comment).
__device__ __forceinline__ u32x2_t lds_tr16(const lds_u8* p) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(p)));
}

// Wait until at most n copies issued by this wave are in flight (n = copies of the later stages).
__device__ __forceinline__ void wait_copies(int later_stages) {
  if (later_stages >= 2) asm volatile("s_waitcnt vmcnt(16)");
  else if (later_stages == 1) asm volatile("s_waitcnt vmcnt(8)");
  else asm volatile("s_waitcnt vmcnt(0)");
}

// Workgroup barrier ordering LDS accesses only (a __syncthreads would also wait for all copies in flight).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// A: x [*, K] (gathered through perm, NMAT = 2) or h [slots, K] (NMAT = 1), bf16.  B0/B1: bf16 weights
// [E, K, N] (B1 only for NMAT = 2).  out: h bf16 [slots, N] (NMAT = 2) or y f32 [slots, N] (NMAT = 1).
template <int NMAT>
__global__ __launch_bounds__(256) void tiled_dma_kernel(const uint16_t* __restrict__ A,
                                                        const uint16_t* __restrict__ B0,
                                                        const uint16_t* __restrict__ B1,
                                                        const int32_t* __restrict__ counts,
                                                        const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ perm, int K, int N, int E,
                                                        void* __restrict__ out) {
  constexpr int BNM = BNT / NMAT;  // columns per matrix
  int e, row0, rows, ntile;
  if (!tile::map_tile(counts, offsets, E, N / BNM, blockIdx.x, &e, &row0, &rows, &ntile)) return;  // whole WG

  __shared__ __attribute__((aligned(1024))) uint8_t smem[NSTAGE * STAGE];
  lds_u8* lds = (lds_u8*)(smem);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nbase = ntile * BNM;

  // ---- copy sources.  A: wave w copies rows 64 w + 16 i + lane/4 (i = 0..3), LDS slot lane & 3 of the row.
  const uint16_t* a_src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 64 * wave + 16 * i + (lane >> 2);
    const int rr = min(r, rows - 1);  // rows past the expert's end repeat a valid row; never stored
    const size_t arow = (NMAT == 2) ? size_t(perm[row0 + rr]) : size_t(row0 + rr);
    a_src[i] = A + arow * K + 8 * ((lane & 3) ^ ((r >> 2) & 3));
  }
  // B: wave w copies k rows 8 w + 2 i + lane/32 (i = 0..3), LDS slot lane & 31 of the 512-byte row.
  const uint16_t* b_src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = 8 * wave + 2 * i + (lane >> 5);
    const int c = (lane & 31) ^ (4 * (k & 3));
    const uint16_t* bm = (NMAT == 2 && c >= 16) ? B1 : B0;
    const int col = nbase + 8 * ((NMAT == 2) ? (c & 15) : c);
    b_src[i] = bm + size_t(e) * K * N + size_t(k) * N + col;
  }
  auto issue = [&](int stage, int k0) {
    const lds_u8* as = lds + stage * STAGE;
    const lds_u8* bs = as + A_STAGE;
#pragma unroll
    for (int i = 0; i < 4; ++i) g2lds16(a_src[i] + k0, as + (64 * wave + 16 * i) * (BK * 2));
#pragma unroll
    for (int i = 0; i < 4; ++i) g2lds16(b_src[i] + size_t(k0) * N, bs + (8 * wave + 2 * i) * (BNT * 2));
  };

  // ---- fragment addresses.  Waves 2 x 2: wave rows wm*128 .. +127, 4 column sub-tiles of 32.
  const int wm = wave >> 1, wn = wave & 1;
  int a_off[4][2];  // A row wm*128 + 32 i + (lane & 31), k chunk 2 ks + (lane >> 5)
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int r = wm * 128 + 32 * i + (lane & 31);
      a_off[i][ks] = r * (BK * 2) + 16 * ((2 * ks + (lane >> 5)) ^ ((r >> 2) & 3));
    }
  // B halves h: lane addresses k row 16 ks + 8 g + 4 h + (s >> 2) and columns col .. +3, where G = lane >> 4,
  // g = G >> 1, s = lane & 15 and col = (sub-tile base) + 16 (G & 1) + 4 (s & 3)
  int b_off[4][2][2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int colbase = (NMAT == 2) ? ((j >> 1) * 128 + wn * 64 + (j & 1) * 32) : (wn * 128 + j * 32);
    const int G = lane >> 4, s = lane & 15;
    const int col = colbase + 16 * (G & 1) + 4 * (s & 3);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = 16 * ks + 8 * (G >> 1) + 4 * h + (s >> 2);
        b_off[j][ks][h] = A_STAGE + k * (BNT * 2) + 16 * ((col >> 3) ^ (4 * (k & 3))) + 2 * (col & 7);
      }
  }
  auto frags = [&](const lds_u8* st, int ks, u32x4_t fa[4], u32x4_t fb[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = *(const __attribute__((address_space(3))) u32x4_t*)(st + a_off[i][ks]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x2_t lo = lds_tr16(st + b_off[j][ks][0]);
      const u32x2_t hi = lds_tr16(st + b_off[j][ks][1]);
      fb[j] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
    }
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  auto mma = [&](const u32x4_t fa[4], const u32x4_t fb[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma32x32x16(fa[i], fb[j], acc[i][j]);
  };

  // ---- main loop.  Copies issued so far are always stages 0 .. min(kt + NSTAGE - 2, KT - 1).
  const int KT = K / BK;
#pragma unroll
  for (int s = 0; s < NSTAGE - 1; ++s)
    if (s < KT) issue(s, s * BK);
  wait_copies(min(KT - 1, NSTAGE - 2));
  lds_barrier();
  u32x4_t fa0[4], fb0[4], fa1[4], fb1[4];
  frags(lds, 0, fa0, fb0);
  for (int kt = 0; kt < KT; ++kt) {
    const lds_u8* st = lds + (kt % NSTAGE) * STAGE;
    frags(st, 1, fa1, fb1);
    mma(fa0, fb0);
    wait_copies(min(KT - 1, kt + NSTAGE - 2) - (kt + 1));
    lds_barrier();  // stage kt+1 landed for every wave; every wave finished reading stage kt-1
    if (kt + NSTAGE - 1 < KT) issue((kt + NSTAGE - 1) % NSTAGE, (kt + NSTAGE - 1) * BK);
    if (kt + 1 < KT) frags(lds + ((kt + 1) % NSTAGE) * STAGE, 0, fa0, fb0);
    mma(fa1, fb1);
  }

  tile::store_tile<NMAT, false>(acc, wm, wn, lane, e, row0, rows, nbase, N, nullptr, nullptr, out);
}

hipError_t launch_up_tiled_dma(const uint16_t* x, const void* w1, const void* wv, const int32_t* counts,
                               const int32_t* offsets, const int32_t* perm, int d, int f, int E, int slots,
                               uint16_t* h, hipStream_t s) {
  const dim3 grid(tile::grid_tiles(slots, E, f / (BNT / 2))), block(256);
  tiled_dma_kernel<2><<<grid, block, 0, s>>>(x, static_cast<const uint16_t*>(w1), static_cast<const uint16_t*>(wv),
                                             counts, offsets, perm, d, f, E, h);
  return hipGetLastError();
}

hipError_t launch_down_tiled_dma(const uint16_t* h, const void* w2, const int32_t* counts, const int32_t* offsets,
                                 int d, int f, int E, int slots, float* y, hipStream_t s) {
  const dim3 grid(tile::grid_tiles(slots, E, d / BNT)), block(256);
  tiled_dma_kernel<1><<<grid, block, 0, s>>>(h, static_cast<const uint16_t*>(w2), nullptr, counts, offsets, nullptr,
                                             f, d, E, y);
  return hipGetLastError();
}

}  // namespace gm
