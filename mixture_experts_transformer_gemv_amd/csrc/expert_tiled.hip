// LDS-tiled grouped GEMM with register-staged weight tiles (used for int8 weights), gfx950.
//
// Expert FFN, page "A functional bridge between openai/grok and xai-org/grok-1" (architecture diagram):
// y = (GELU(x W1) (*) (x Wv)) W2; int8 weights times bf16 scales broadcast over groups of input rows, page
// "Grok-1-BF16", section "Conversion Details".
//
// Tile shape, order and epilogue: tiles.h.  K steps of 64, double-buffered in LDS (2 x 72 KB).  Weights are
// stored [in, out] while the MFMA wants 8 consecutive k per lane, so each thread loads an 8 (k) x 8 (n) block as
// eight row pieces, converts int8 to bf16 exactly (|q| <= 128 has at most 8 significant bits) while transposing
// it in registers, and writes eight 16-byte column pieces into the [n][k] LDS tile.  LDS rows are padded by 16
// bytes so that 16-byte MFMA operand reads of consecutive rows fall into distinct banks.  With one scale group
// along K the per-channel scales multiply the fp32 accumulators in the epilogue.  With several (GROUPED) the
// accumulators are kept in units of the current group's scale: entering group g multiplies each column by
// s[g-1]/s[g], the epilogue multiplies by the last group's scale; a zero scale is replaced by one and the
// column's int8 values of that group are masked to zero while they are converted.  bf16 weights take the
// direct-to-LDS kernel of expert_tiled_dma.hip instead.  The GROUPED form uses 128-row tiles (64 x 128 per
// wave) so that the accumulators leave registers for the rescaling.  Weights stored [E, out, in] (OUTIN) are
// loaded as 8 consecutive k of each of the thread's 8 columns (eight lanes read 64 contiguous bytes of a row)
// and only converted, not transposed, before the same LDS stores.
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

// Row piece of an int8 weight block: 8 bytes = 8 columns (or, [out, in], 8 k of one column).
__device__ __forceinline__ u32x2_t load_i8x8(const void* base, size_t i) {
  return *reinterpret_cast<const u32x2_t*>(static_cast<const int8_t*>(base) + i);
}

// A: x [*, K] (gathered through perm, NMAT = 2) or h [slots, K] (NMAT = 1).  B0/B1: weights [E, K, N].
// out: h bf16 [slots, N] (NMAT = 2) or y f32 [slots, N] (NMAT = 1).
template <int NMAT, bool GROUPED, bool OUTIN>
__global__ __launch_bounds__(256) void tiled_reg_kernel(const uint16_t* __restrict__ A, const void* __restrict__ B0,
                                                    const void* __restrict__ B1, const uint16_t* __restrict__ sc0,
                                                    const uint16_t* __restrict__ sc1, ScaleLayout sl,
                                                    const int32_t* __restrict__ counts,
                                                    const int32_t* __restrict__ offsets,
                                                    const int32_t* __restrict__ perm, int K, int N, int E,
                                                    void* __restrict__ out) {
  constexpr int BNM = BNT / NMAT;       // columns per matrix
  constexpr int TBM = GROUPED ? 128 : BM;  // rows per tile
  constexpr int MI = TBM / 64;          // 32-row MFMA blocks per wave
  constexpr int NA = TBM / 32;          // 16-byte A pieces per thread and K step
  int e, row0, rows, ntile;
  if (!tile::map_tile<tile::Group<NMAT>::N, TBM>(counts, offsets, E, N / BNM, blockIdx.x, &e, &row0, &rows, &ntile))
    return;  // whole workgroup

  __shared__ __attribute__((aligned(16))) uint16_t As[2][TBM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BNT * LDK];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nbase = ntile * BNM;

  // ---- global A pieces: NA x 16 bytes per thread (rows tid/8 + 32 i, k piece tid % 8)
  const uint16_t* a_src[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
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
  // [in, out]: rows 8 kb .. +7 of the K step, 8 columns; [out, in]: column rows gcol .. +7, k 8 kb .. +7
  const size_t b_base = OUTIN ? size_t(e) * K * N + size_t(gcol) * K + 8 * kb
                              : size_t(e) * K * N + size_t(8 * kb) * N + gcol;
  const int b_lds_row = wave * 64 + nb * 8;  // first of the 8 LDS rows (columns) this thread writes

  // GROUPED: scales of the 8 columns of this thread's B block (group 0), and the byte mask of those with a
  // non-zero scale in the group of the K step held in rb
  const uint16_t* bscale = ((NMAT == 2 && mat == 1) ? sc1 : sc0) + size_t(e) * sl.estride + gcol;
  u32x2_t bmask = {~0u, ~0u};
  auto set_bmask = [&](int grp) {
    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(bscale + size_t(grp) * N);
    bmask = u32x2_t{0u, 0u};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t b = (w[c >> 1] >> (16 * (c & 1))) & 0xffffu;
      if (b & 0x7fffu) bmask[c >> 2] |= 0xffu << (8 * (c & 3));
    }
  };

  u32x4_t ra[NA];
  u32x2_t rb[8];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < NA; ++i) ra[i] = *reinterpret_cast<const u32x4_t*>(a_src[i] + k0);
#pragma unroll
    for (int r = 0; r < 8; ++r)
      rb[r] = OUTIN ? load_i8x8(bmat, b_base + size_t(r) * K + k0) : load_i8x8(bmat, b_base + size_t(k0 + r) * N);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NA; ++i)
      *reinterpret_cast<u32x4_t*>(&As[buf][((tid >> 3) + 32 * i) * LDK + 8 * (tid & 7)]) = ra[i];
    u32x4_t t[8];
    if constexpr (OUTIN) {  // rb[c] is column c: mask whole columns, convert without transposing
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        u32x2_t v = rb[c];
        if constexpr (GROUPED) {
          const uint32_t keep = ((bmask[c >> 2] >> (8 * (c & 3))) & 0xffu) ? ~0u : 0u;
          v &= u32x2_t{keep, keep};
        }
        t[c] = i8x8_to_bf16(v);
      }
    } else {
      if constexpr (GROUPED) {
#pragma unroll
        for (int r = 0; r < 8; ++r) rb[r] &= bmask;
      }
      transpose8x8_i8_to_bf16(rb, t);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) *reinterpret_cast<u32x4_t*>(&Bs[buf][(b_lds_row + c) * LDK + 8 * kb]) = t[c];
  };

  // ---- MFMA tiling: waves 2 x 2; wave rows wm*TBM/2 .. +TBM/2-1; 4 column sub-tiles of 32
  const int wm = wave >> 1, wn = wave & 1;
  int bsub[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) bsub[j] = (NMAT == 2) ? ((j >> 1) * 128 + wn * 64 + (j & 1) * 32) : (wn * 128 + j * 32);
  f32x16_t acc[MI][4];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int lr = lane & 31, lk = 8 * (lane >> 5);
  // the output column of each accumulator sub-tile held by this lane, as a pointer to its group-0 scale
  const uint16_t* jscale[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (NMAT == 2) jscale[j] = ((j >> 1) ? sc1 : sc0) + size_t(e) * sl.estride + nbase + wn * 64 + (j & 1) * 32 + lr;
    else jscale[j] = sc0 + size_t(e) * sl.estride + nbase + wn * 128 + j * 32 + lr;
  }
  float cur[4] = {1.0f, 1.0f, 1.0f, 1.0f};  // GROUPED: scale (zero -> one) of the group being accumulated
  auto group_scale = [&](int j, int grp) {
    const uint16_t b = jscale[j][size_t(grp) * N];
    return (b & 0x7fffu) ? bf16f(b) : 1.0f;
  };
  auto frags = [&](int buf, int ks, u32x4_t a[MI], u32x4_t b[4]) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
      a[i] = *reinterpret_cast<const u32x4_t*>(&As[buf][(wm * 32 * MI + i * 32 + lr) * LDK + ks + lk]);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const u32x4_t*>(&Bs[buf][(bsub[j] + lr) * LDK + ks + lk]);
  };

  // ---- main loop.  Step kt: the operand fragments of sub-step ks+1 are read from LDS while sub-step ks is
  // multiplied; the K step kt+1 (already in registers) is transposed and stored to the other LDS buffer, and
  // step kt+2 is fetched from global memory, all interleaved with the 64 MFMAs of step kt.  The body has no
  // branches (the prefetch past the last step re-reads it; it is never stored).
  const int KT = K / BK;
  const int gsteps = sl.gsize / BK;  // K steps per scale group (GROUPED)
  if constexpr (GROUPED) {
    set_bmask(0);
#pragma unroll
    for (int j = 0; j < 4; ++j) cur[j] = group_scale(j, 0);
  }
  gload(0);
  lstore(0);
  gload(min(1, KT - 1) * BK);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if constexpr (GROUPED) {
      if (kt > 0 && kt % gsteps == 0) {  // step kt opens group kt / gsteps: change the accumulators' unit
        const int grp = kt / gsteps;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float nv = group_scale(j, grp);
          const float r = cur[j] / nv;
          cur[j] = nv;
#pragma unroll
          for (int i = 0; i < MI; ++i) acc[i][j] *= r;
        }
      }
      if ((kt + 1) < KT && (kt + 1) % gsteps == 0) set_bmask((kt + 1) / gsteps);  // rb holds step kt + 1
    }
    u32x4_t fa[2][MI], fb[2][4];
    frags(buf, 0, fa[0], fb[0]);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      if (ks + 1 < BK / 16) frags(buf, (ks + 1) * 16, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32x32x16(fa[ks & 1][i], fb[ks & 1][j], acc[i][j]);
    }
    lstore(buf ^ 1);
    gload(min(kt + 2, KT - 1) * BK);
    // interleave: 8 fragment reads, then MFMAs each followed by the remaining fragment reads, then by
    // transposes and LDS stores, then by the global loads of the step after next (the GROUPED form is left to
    // the compiler's schedule)
    if constexpr (!GROUPED) {
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
    }
    __syncthreads();
  }

  // the scale of the last group (GROUPED) or of the only one, then the plain epilogue
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float sj = GROUPED ? cur[j] : bf16f(jscale[j][0]);
#pragma unroll
    for (int i = 0; i < MI; ++i) acc[i][j] *= sj;
  }
  tile::store_tile<NMAT, MI>(acc, wm, wn, lane, row0, rows, nbase, N, out);
}

hipError_t launch_up_tiled(const uint16_t* x, const void* w1, const void* wv, const uint16_t* s1,
                           const uint16_t* sv, ScaleLayout sl, bool outin, const int32_t* counts,
                           const int32_t* offsets, const int32_t* perm, int d, int f, int E, int slots, bool int8,
                           uint16_t* h, hipStream_t s) {
  const bool grouped = sl.gsize < d;
  if (!int8 || (!grouped && !outin))  // bf16, and int8 with one scale group from [in, out] storage: direct copies
    return launch_up_tiled_dma(x, w1, wv, s1, sv, sl.estride, int8, outin, counts, offsets, perm, d, f, E, slots,
                               h, s);
  if (grouped && !outin && tiled_dma_grouped_fits(d, sl.gsize))  // up to 8 scale groups: direct copies too
    return launch_up_tiled_dma_grouped(x, w1, wv, s1, sv, sl.estride, sl.gsize, counts, offsets, perm, d, f, E,
                                       slots, h, s);
  const dim3 grid(tile::grid_tiles(slots, E, f / (BNT / 2), grouped ? 128 : BM)), block(256);
#define GM_UPT(GR, OI) tiled_reg_kernel<2, GR, OI><<<grid, block, 0, s>>>(x, w1, wv, s1, sv, sl, counts, offsets, \
                                                                             perm, d, f, E, h)
  if (grouped) { if (outin) GM_UPT(true, true); else GM_UPT(true, false); }
  else { if (outin) GM_UPT(false, true); else GM_UPT(false, false); }
#undef GM_UPT
  return hipGetLastError();
}

hipError_t launch_down_tiled(const uint16_t* h, const void* w2, const uint16_t* s2, ScaleLayout sl, bool outin,
                             const int32_t* counts, const int32_t* offsets, int d, int f, int E, int slots, int S,
                             bool int8, float* y, hipStream_t s) {
  const bool grouped = sl.gsize < f;
  if (!int8 || (!grouped && !outin))
    return launch_down_tiled_dma(h, w2, s2, sl.estride, int8, outin, counts, offsets, d, f, E, slots, S, y, s);
  if (grouped && !outin && tiled_dma_grouped_fits(f, sl.gsize))
    return launch_down_tiled_dma_grouped(h, w2, s2, sl.estride, sl.gsize, counts, offsets, d, f, E, slots, S, y,
                                         s);
  const dim3 grid(tile::grid_tiles(slots, E, d / BNT, grouped ? 128 : BM)), block(256);
#define GM_DNT(GR, OI) tiled_reg_kernel<1, GR, OI><<<grid, block, 0, s>>>(h, w2, nullptr, s2, nullptr, sl, counts, \
                                                                             offsets, nullptr, f, d, E, y)
  if (grouped) { if (outin) GM_DNT(true, true); else GM_DNT(true, false); }
  else { if (outin) GM_DNT(false, true); else GM_DNT(false, false); }
#undef GM_DNT
  return hipGetLastError();
}

}  // namespace gm
