// LDS-tiled grouped GEMM with register-staged weight tiles (used for int8 weights), gfx950.
//
// Expert FFN, page "A functional bridge between openai/grok and xai-org/grok-1" (architecture diagram):
// y = (GELU(x W1) (*) (x Wv)) W2; int8 weights times per-(expert, output channel) bf16 scales, page
// "Grok-1-BF16", section "Conversion Details".
//
// Tile shape, order and epilogue: tiles.h.  K steps of 64, double-buffered in LDS (2 x 72 KB).  Weights are
// stored [in, out] while the MFMA wants 8 consecutive k per lane, so each thread loads an 8 (k) x 8 (n) block as
// eight row pieces, converts int8 to bf16 exactly (|q| <= 128 has at most 8 significant bits) while transposing
// it in registers, and writes eight 16-byte column pieces into the [n][k] LDS tile.  LDS rows are padded by 16
// bytes so that 16-byte MFMA operand reads of consecutive rows fall into distinct banks.  The per-channel scales
// multiply the fp32 accumulators in the epilogue.  bf16 weights take the direct-to-LDS kernel of
// expert_tiled_dma.hip instead.
#include "common.h"
#include "launch.h"
#include "tiles.h"

namespace gm {

namespace {
using tile::BM;
using tile::BNT;
constexpr int BK = 64;
constexpr int LDK = BK + 8;  // padded LDS row (bf16 elements)
}

template <bool INT8> struct BRow;
template <> struct BRow<false> {
  typedef u32x4_t T;
  static __device__ __forceinline__ T load(const void* base, size_t i) {
    return *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(base) + i);
  }
  static __device__ __forceinline__ void transpose(const T r[8], u32x4_t t[8]) { transpose8x8_bf16(r, t); }
};
template <> struct BRow<true> {
  typedef u32x2_t T;
  static __device__ __forceinline__ T load(const void* base, size_t i) {
    return *reinterpret_cast<const u32x2_t*>(static_cast<const int8_t*>(base) + i);
  }
  static __device__ __forceinline__ void transpose(const T r[8], u32x4_t t[8]) { transpose8x8_i8_to_bf16(r, t); }
};

// A: x [*, K] (gathered through perm, NMAT = 2) or h [slots, K] (NMAT = 1).  B0/B1: weights [E, K, N].
// out: h bf16 [slots, N] (NMAT = 2) or y f32 [slots, N] (NMAT = 1).
template <int NMAT, bool INT8>
__global__ __launch_bounds__(256) void tiled_reg_kernel(const uint16_t* __restrict__ A, const void* __restrict__ B0,
                                                    const void* __restrict__ B1, const uint16_t* __restrict__ sc0,
                                                    const uint16_t* __restrict__ sc1,
                                                    const int32_t* __restrict__ counts,
                                                    const int32_t* __restrict__ offsets,
                                                    const int32_t* __restrict__ perm, int K, int N, int E,
                                                    void* __restrict__ out) {
  typedef BRow<INT8> W;
  constexpr int BNM = BNT / NMAT;  // columns per matrix
  int e, row0, rows, ntile;
  if (!tile::map_tile<tile::Group<NMAT>::N>(counts, offsets, E, N / BNM, blockIdx.x, &e, &row0, &rows, &ntile)) return;  // whole workgroup

  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BNT * LDK];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nbase = ntile * BNM;

  // ---- global A pieces: 8 x 16 bytes per thread (rows tid/8 + 32 i, k piece tid % 8)
  const uint16_t* a_src[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = (tid >> 3) + 32 * i;
    const int rr = min(r, rows - 1);  // rows past the expert's end repeat a valid row; never stored
    const size_t arow = (NMAT == 2) ? size_t(perm[row0 + rr]) : size_t(row0 + rr);
    a_src[i] = A + arow * K + 8 * (tid & 7);
  }
  // ---- global B block: rows 8 kb .. +7 of the K step, columns gcol .. +7 of matrix `mat`
  const int kb = lane & 7, nb = lane >> 3;
  const int mat = (NMAT == 2) ? (wave >> 1) : 0;
  const int gcol = nbase + ((NMAT == 2) ? (wave & 1) * 64 : wave * 64) + nb * 8;
  const void* bmat = (NMAT == 2 && mat == 1) ? B1 : B0;
  const size_t b_base = size_t(e) * K * N + size_t(8 * kb) * N + gcol;
  const int b_lds_row = wave * 64 + nb * 8;  // first of the 8 LDS rows (columns) this thread writes

  u32x4_t ra[8];
  typename W::T rb[8];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) ra[i] = *reinterpret_cast<const u32x4_t*>(a_src[i] + k0);
#pragma unroll
    for (int r = 0; r < 8; ++r) rb[r] = W::load(bmat, b_base + size_t(k0 + r) * N);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<u32x4_t*>(&As[buf][((tid >> 3) + 32 * i) * LDK + 8 * (tid & 7)]) = ra[i];
    u32x4_t t[8];
    W::transpose(rb, t);
#pragma unroll
    for (int c = 0; c < 8; ++c) *reinterpret_cast<u32x4_t*>(&Bs[buf][(b_lds_row + c) * LDK + 8 * kb]) = t[c];
  };

  // ---- MFMA tiling: waves 2 x 2; wave rows wm*128 .. +127; 4 column sub-tiles of 32
  const int wm = wave >> 1, wn = wave & 1;
  int bsub[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) bsub[j] = (NMAT == 2) ? ((j >> 1) * 128 + wn * 64 + (j & 1) * 32) : (wn * 128 + j * 32);
  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int lr = lane & 31, lk = 8 * (lane >> 5);
  auto frags = [&](int buf, int ks, u32x4_t a[4], u32x4_t b[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[i] = *reinterpret_cast<const u32x4_t*>(&As[buf][(wm * 128 + i * 32 + lr) * LDK + ks + lk]);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const u32x4_t*>(&Bs[buf][(bsub[j] + lr) * LDK + ks + lk]);
  };

  // ---- main loop.  Step kt: the operand fragments of sub-step ks+1 are read from LDS while sub-step ks is
  // multiplied; the K step kt+1 (already in registers) is transposed and stored to the other LDS buffer, and
  // step kt+2 is fetched from global memory, all interleaved with the 64 MFMAs of step kt.  The body has no
  // branches (the prefetch past the last step re-reads it; it is never stored).
  const int KT = K / BK;
  gload(0);
  lstore(0);
  gload(min(1, KT - 1) * BK);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    u32x4_t fa[2][4], fb[2][4];
    frags(buf, 0, fa[0], fb[0]);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      if (ks + 1 < BK / 16) frags(buf, (ks + 1) * 16, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32x32x16(fa[ks & 1][i], fb[ks & 1][j], acc[i][j]);
    }
    lstore(buf ^ 1);
    gload(min(kt + 2, KT - 1) * BK);
    // interleave: 8 fragment reads, then MFMAs each followed by the remaining fragment reads, then by
    // transposes and LDS stores, then by the global loads of the step after next
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i < 24; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    __syncthreads();
  }

  tile::store_tile<NMAT, INT8>(acc, wm, wn, lane, e, row0, rows, nbase, N, sc0, sc1, out);
}

hipError_t launch_up_tiled(const uint16_t* x, const void* w1, const void* wv, const uint16_t* s1,
                           const uint16_t* sv, const int32_t* counts, const int32_t* offsets, const int32_t* perm,
                           int d, int f, int E, int slots, bool int8, uint16_t* h, hipStream_t s) {
  if (!int8) return launch_up_tiled_dma(x, w1, wv, counts, offsets, perm, d, f, E, slots, h, s);
  const dim3 grid(tile::grid_tiles(slots, E, f / (BNT / 2))), block(256);
  tiled_reg_kernel<2, true><<<grid, block, 0, s>>>(x, w1, wv, s1, sv, counts, offsets, perm, d, f, E, h);
  return hipGetLastError();
}

hipError_t launch_down_tiled(const uint16_t* h, const void* w2, const uint16_t* s2, const int32_t* counts,
                             const int32_t* offsets, int d, int f, int E, int slots, int S, bool int8, float* y,
                             hipStream_t s) {
  if (!int8) return launch_down_tiled_dma(h, w2, counts, offsets, d, f, E, slots, S, y, s);
  const dim3 grid(tile::grid_tiles(slots, E, d / BNT)), block(256);
  tiled_reg_kernel<1, true><<<grid, block, 0, s>>>(h, w2, nullptr, s2, nullptr, counts, offsets, nullptr, f, d, E, y);
  return hipGetLastError();
}

}  // namespace gm
