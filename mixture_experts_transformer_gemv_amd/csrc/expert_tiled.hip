// Expert matrix products of the Grok-1 MoE layer for many tokens per expert (prefill), gfx950.
//
// Expert FFN, page "A functional bridge between openai/grok and xai-org/grok-1" (architecture diagram):
// y = (GELU(x W1) (*) (x Wv)) W2; int8 weights times per-(expert, output channel) bf16 scales, page
// "Grok-1-BF16", section "Conversion Details".
//
// Grouped GEMM over the expert-sorted assignment slots.  A workgroup (4 waves) computes a 128-row x 256-column
// output tile with a 64-deep K step, double-buffered in LDS:
//   * up-projection (NMAT = 2): 128 columns of W1 and the same 128 columns of Wv; A rows are gathered from x
//     through the slot -> token permutation; the epilogue writes h = bf16(GELU(a) * b);
//   * down-projection (NMAT = 1): 256 columns of W2; A rows are consecutive slots of h; fp32 output.
// Weights are stored [in, out] (columns contiguous) while the MFMA wants 8 consecutive k per lane, so each
// thread loads an 8 (k) x 8 (n) block as eight row pieces, transposes it in registers (converting int8 to bf16
// exactly on the way) and writes eight 16-byte column pieces into the [n][k] LDS tile.  LDS rows are padded by
// 16 bytes so that the 16-byte MFMA operand reads of consecutive rows fall into distinct banks.
// MFMA 32x32x16 bf16; each wave holds a 64 x 128 accumulator tile (128 fp32 per lane).
#include "common.h"
#include "launch.h"

namespace gm {

namespace {
constexpr int BM = 128;  // rows per tile
constexpr int BNT = 256; // output columns per tile (all matrices)
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

// A: x [*, K] (GATHER through perm) or h [slots, K].  B0/B1: weights [E, K, N] (B1 only for NMAT = 2).
// out: h bf16 [slots, N] (NMAT = 2) or y f32 [slots, N] (NMAT = 1).
template <int NMAT, bool INT8>
__global__ __launch_bounds__(256) void tiled_kernel(const uint16_t* __restrict__ A, const void* __restrict__ B0,
                                                    const void* __restrict__ B1, const uint16_t* __restrict__ sc0,
                                                    const uint16_t* __restrict__ sc1,
                                                    const int32_t* __restrict__ counts,
                                                    const int32_t* __restrict__ offsets,
                                                    const int32_t* __restrict__ perm, int K, int N, int E,
                                                    void* __restrict__ out) {
  typedef BRow<INT8> W;
  int e, row0, rows;
  if (!find_row_tile(counts, offsets, E, BM, blockIdx.x, &e, &row0, &rows)) return;  // whole workgroup

  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BNT * LDK];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  constexpr int BNM = BNT / NMAT;  // columns per matrix
  const int nbase = blockIdx.y * BNM;

  // ---- global A pieces: 4 x 16 bytes per thread (rows tid/8 + 32 i, k piece tid % 8)
  const uint16_t* a_src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
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

  u32x4_t ra[4];
  typename W::T rb[8];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[i] = *reinterpret_cast<const u32x4_t*>(a_src[i] + k0);
#pragma unroll
    for (int r = 0; r < 8; ++r) rb[r] = W::load(bmat, b_base + size_t(k0 + r) * N);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4_t*>(&As[buf][((tid >> 3) + 32 * i) * LDK + 8 * (tid & 7)]) = ra[i];
    u32x4_t t[8];
    W::transpose(rb, t);
#pragma unroll
    for (int c = 0; c < 8; ++c) *reinterpret_cast<u32x4_t*>(&Bs[buf][(b_lds_row + c) * LDK + 8 * kb]) = t[c];
  };

  // ---- MFMA tiling: waves 2 x 2; wave rows wm*64 .. +63; 4 column sub-tiles of 32
  const int wm = wave >> 1, wn = wave & 1;
  int bsub[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) bsub[j] = (NMAT == 2) ? ((j >> 1) * 128 + wn * 64 + (j & 1) * 32) : (wn * 128 + j * 32);
  f32x16_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int lr = lane & 31, lk = 8 * (lane >> 5);
  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < BK; ks += 16) {
      u32x4_t a[2], b[4];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const u32x4_t*>(&As[buf][(wm * 64 + i * 32 + lr) * LDK + ks + lk]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const u32x4_t*>(&Bs[buf][(bsub[j] + lr) * LDK + ks + lk]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
    }
  };

  const int KT = K / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + 1 < KT) gload((kt + 1) * BK);
    compute(kt & 1);
    if (kt + 1 < KT) lstore((kt + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds column lr of each 32-wide sub-tile, rows (v&3) + 8(v>>2) + 4(lane>>5)
  const int rhalf = 4 * (lane >> 5);
  if (NMAT == 2) {
    uint16_t* h = static_cast<uint16_t*>(out);
#pragma unroll
    for (int jn = 0; jn < 2; ++jn) {
      const int n = nbase + wn * 64 + jn * 32 + lr;
      float s_a = 1.0f, s_b = 1.0f;
      if (INT8) { s_a = bf16f(sc0[size_t(e) * N + n]); s_b = bf16f(sc1[size_t(e) * N + n]); }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = wm * 64 + i * 32 + (v & 3) + 8 * (v >> 2) + rhalf;
          if (r < rows) {
            const float a = acc[i][jn][v] * s_a, b = acc[i][2 + jn][v] * s_b;
            h[size_t(row0 + r) * N + n] = uint16_t(f2bf(gelu_erf(a) * b));
          }
        }
      }
    }
  } else {
    float* y = static_cast<float*>(out);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = nbase + wn * 128 + j * 32 + lr;
      const float s = INT8 ? bf16f(sc0[size_t(e) * N + n]) : 1.0f;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = wm * 64 + i * 32 + (v & 3) + 8 * (v >> 2) + rhalf;
          if (r < rows) y[size_t(row0 + r) * N + n] = INT8 ? acc[i][j][v] * s : acc[i][j][v];
        }
      }
    }
  }
}

static inline int max_row_tiles(int slots, int E) { return slots / BM + E; }

hipError_t launch_up_tiled(const uint16_t* x, const void* w1, const void* wv, const uint16_t* s1,
                           const uint16_t* sv, const int32_t* counts, const int32_t* offsets, const int32_t* perm,
                           int d, int f, int E, int slots, bool int8, uint16_t* h, hipStream_t s) {
  const dim3 grid(max_row_tiles(slots, E), f / (BNT / 2)), block(256);
  if (int8) tiled_kernel<2, true><<<grid, block, 0, s>>>(x, w1, wv, s1, sv, counts, offsets, perm, d, f, E, h);
  else tiled_kernel<2, false><<<grid, block, 0, s>>>(x, w1, wv, s1, sv, counts, offsets, perm, d, f, E, h);
  return hipGetLastError();
}

hipError_t launch_down_tiled(const uint16_t* h, const void* w2, const uint16_t* s2, const int32_t* counts,
                             const int32_t* offsets, int d, int f, int E, int slots, bool int8, float* y,
                             hipStream_t s) {
  const dim3 grid(max_row_tiles(slots, E), d / BNT), block(256);
  if (int8) tiled_kernel<1, true><<<grid, block, 0, s>>>(h, w2, nullptr, s2, nullptr, counts, offsets, nullptr, f, d, E, y);
  else tiled_kernel<1, false><<<grid, block, 0, s>>>(h, w2, nullptr, s2, nullptr, counts, offsets, nullptr, f, d, E, y);
  return hipGetLastError();
}

}  // namespace gm
