// Expert matrix products for few tokens per expert with the weights stored [E, out, in], gfx950.
//
// Expert FFN, page "A functional bridge between openai/grok and xai-org/grok-1" (architecture diagram):
// y = (GELU(x W1) (*) (x Wv)) W2.  [out, in] is the PyTorch layout the weights are converted to, page
// "Grok-1-BF16", section "Conversion Details"; int8 weights times bf16 scales grouped along the input axis.
//
// Bound by streaming the weights from HBM.  In [out, in] storage each output column is a contiguous row of K
// values, but the MFMA operand layout puts 16 different columns in the 16 lanes of a group, so operands loaded
// straight from memory touch 16 rows x 64 bytes per load (measured 4.9-5.2 TB/s on MI355X, against 5.9-6.0 TB/s
// for 8 rows x 128 bytes or 4 rows x 256 bytes).  So the weights go through LDS: per stage of 128 k every stored
// row contributes a 256-byte (bf16) or 128-byte (int8) piece, copied by global_load_lds_dwordx4 with 16 or 8 lanes
// on one row; the token rows of the stage are copied the same way; the MFMA operands are then 16-byte (int8:
// 8-byte) LDS reads.  16-byte chunk c of tile row r sits in slot c ^ (r & 15) (256-byte rows) or c ^ ((r >> 1) & 7)
// (128-byte rows), chosen on the global side, so both the copies and the operand reads are free of bank
// conflicts.
// The weight copies carry the nontemporal hint: each weight byte is read once per launch.
//
// A workgroup of 4 waves owns 64 output columns (16 per wave) of W1 and Wv (up) or of W2 (down: all spw chunks of
// the f axis, a partial sum stored per chunk, so that one ring streams every chunk) for all token
// rows of its expert (16 MT rows per pass), over a ring of NSTG stages with one workgroup barrier per stage.  The
// bf16 up-projection's workgroups take NB consecutive blocks of 64 columns as one stream of stages (the last stages
// of a block copy the first ones of the next), so a workgroup start, with its first copies' latency, comes once per
// NB blocks.
// Each (token, column) accumulates over k in 32-deep steps in ascending order, with the same lane-to-k
// assignment as the [in, out] kernels, so the results are bit-identical to theirs.
//
// Grouped int8 scales (group boundaries on stage boundaries): the accumulators are kept in units of the current
// group's scale (rescaled by s[g-1]/s[g] on entering group g, zero scales replaced by one with their columns'
// values masked); the scales of the wave's 16 columns are read with uniform (scalar) loads one group ahead.
#include "chunks.h"
#include "common.h"
#include "dma.h"
#include "launch.h"

namespace gm {

namespace {
constexpr int OI_COLS = 64;            // output columns (stored rows) per workgroup, 16 per wave
constexpr int OI_KS = 128;             // k per stage
constexpr int OI_AROW = OI_KS * 2;     // bytes of a token row per stage (bf16)
constexpr int OI_LDS = 144 * 1024;     // LDS budget of the ring
}

template <int NMAT, bool INT8, int MT>
struct OiCfg {
  static constexpr int ROWB = OI_KS * (INT8 ? 1 : 2);          // bytes of each stored row per stage
  static constexpr int WTILE = OI_COLS * ROWB;                 // one matrix's stage tile
  static constexpr int W_PER_WAVE = WTILE / 1024 / 4;          // 1 KB copies per wave and matrix (4 or 2)
  static constexpr int WROWS_PER_COPY = 1024 / ROWB;           // 4 or 8
  static constexpr int ABYTES = MT * 16 * OI_AROW;             // token tile per stage
  static constexpr int STAGE = NMAT * WTILE + ABYTES;
  // ring depth (measured on MI355X).  Up-projection: at most 4 stages; two workgroups per CU (80 KB each) where
  // that leaves at least 3 stages, else one workgroup with up to 144 KB (two resident rings keep more copies in
  // flight: int8 with grouped scales 0.65 -> 0.56 ms at T = 64), 3 stages for one 16-row tile (bf16 T = 8:
  // 0.953 -> 0.945 ms against 4; 2 stages on two workgroups per CU: 0.953).  Down-projection: 2 stages, so that 3-4
  // workgroups share a CU and the whole grid (one workgroup per 64 columns and expert, every chunk of f) runs
  // in one round (bf16 T = 8: 0.578 -> 0.549 ms against 4 stages over 6 rounds).
  static constexpr int NSTG2 = (80 * 1024 / STAGE) < 4 ? (80 * 1024 / STAGE) : 4;
  static constexpr int NSTG1 = MT == 1 ? 3 : 4;  // one workgroup per CU
  static constexpr int NSTG =
      NMAT == 1 ? 2 : (NSTG2 >= 3 ? NSTG2 : ((OI_LDS / STAGE) < NSTG1 ? (OI_LDS / STAGE) : NSTG1));
  static constexpr int A_PER_WAVE = ABYTES / 1024 / 4;         // = MT
  static constexpr int CPW = NMAT * W_PER_WAVE + A_PER_WAVE;   // copies per wave per stage
  static_assert(NSTG >= 2, "stage ring does not fit");
  // slot of 16-byte chunk c in tile row r
  static __device__ __forceinline__ int wslot(int c, int r) { return INT8 ? (c ^ ((r >> 1) & 7)) : (c ^ (r & 15)); }
};

// This lane's raw bf16 scale out of the 16 consecutive ones held in lo, hi (8 + 8, two per dword).
__device__ __forceinline__ uint32_t lane_scale_bits(const u32x4_t& lo, const u32x4_t& hi, int c16) {
  const int q = c16 >> 1;
  uint32_t w = lo[0];
  w = q == 1 ? lo[1] : w;
  w = q == 2 ? lo[2] : w;
  w = q == 3 ? lo[3] : w;
  w = q == 4 ? hi[0] : w;
  w = q == 5 ? hi[1] : w;
  w = q == 6 ? hi[2] : w;
  w = q == 7 ? hi[3] : w;
  return (w >> (16 * (c16 & 1))) & 0xffffu;
}

// A: x [*, K] (gathered through perm, NMAT = 2) or h [slots, K] (NMAT = 1), bf16.  W0/W1: weights [E, N, K]
// (bf16 or int8).  Scales [Es, G, N] (sl).  out: h bf16 [slots, N] (NMAT = 2) or y f32 [S, slots, N] (NMAT = 1,
// one workgroup row over all of K, stored as spw partial sums over the chunks of down_chunk_begin).  NMAT = 2: Kc = K,
// spw = 1.
// KS = 4 (up-projection): the sums over the four quarters of K are kept apart and added in ascending quarter order
// at the end, as the [in, out] kernel with its d axis split over 4 waves adds them (with grouped scales each
// quarter's sum is first brought to the unit of the last quarter, by the same fused multiply-adds).
template <int NMAT, bool INT8, bool GROUPED, int MT, int KS = 1, int NB = 1>
__global__ __launch_bounds__(256) void oi_stream_kernel(const uint16_t* __restrict__ A, const void* __restrict__ W0,
                                                        const void* __restrict__ W1, const uint16_t* __restrict__ sc0,
                                                        const uint16_t* __restrict__ sc1, ScaleLayout sl,
                                                        const int32_t* __restrict__ counts,
                                                        const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ perm, int K, int N, int Kc,
                                                        int spw, void* __restrict__ out, int64_t split_stride) {
  typedef OiCfg<NMAT, INT8, MT> C;
  static_assert(INT8 || !GROUPED, "grouped scales belong to int8 weights");
  static_assert(NB == 1 || (NMAT == 2 && !INT8 && KS == 1), "column blocks per workgroup: bf16 up-projection");
  constexpr int ESZ = INT8 ? 1 : 2;
  const int e = blockIdx.z;
  const int n_e = counts[e];
  if (n_e == 0) return;  // whole workgroup
  const int off = offsets[e];
  const int nbase = blockIdx.x * OI_COLS * NB;
  const int kbeg = NMAT == 1 ? 0 : blockIdx.y * Kc;
  const int NS = (NMAT == 1 ? K : Kc) / OI_KS;  // stages

  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::NSTG * C::STAGE];
  const lds_u8* lds = (const lds_u8*)(smem);
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c16 = lane & 15;

  // ---- weight copies: wave w copies tile rows 16 w .. +15 of each matrix, WROWS_PER_COPY rows per copy; lane
  // slot (lane % chunks per row) of row r receives the chunk stored there (wslot is an involution)
  const size_t wexp = size_t(e) * N * K * ESZ;  // bytes to expert e
  const uint8_t* wb0 = static_cast<const uint8_t*>(W0) + wexp;
  const uint8_t* wb1 = NMAT == 2 ? static_cast<const uint8_t*>(W1) + wexp : wb0;
  uint32_t w_voff[C::W_PER_WAVE];
#pragma unroll
  for (int i = 0; i < C::W_PER_WAVE; ++i) {
    constexpr int CPR = C::ROWB / 16;  // chunks per row
    const int r = 16 * wave + C::WROWS_PER_COPY * i + lane / CPR;
    w_voff[i] = uint32_t(nbase + r) * uint32_t(K * ESZ) + 16u * uint32_t(C::wslot(lane % CPR, r));
  }
  // the wave's operand reads: tile row 16 w + c16 (its column), and token row 16 mt + c16
  const int wrow = 16 * wave + c16;
  const uint16_t* s0w = INT8 ? sc0 + size_t(e) * sl.estride + nbase + 16 * wave : nullptr;  // wave's 16 columns
  const uint16_t* s1w = (INT8 && NMAT == 2) ? sc1 + size_t(e) * sl.estride + nbase + 16 * wave : nullptr;

  for (int mb = 0; mb < n_e; mb += 16 * MT) {
    // ---- token copies: copy q = wave * A_PER_WAVE + i covers token rows ROWS_PER_A_COPY q .. of the pass;
    // lane slot receives chunk slot ^ (row & 15); rows past the expert's end repeat a valid row (never stored)
    uint32_t a_voff[C::A_PER_WAVE];
#pragma unroll
    for (int i = 0; i < C::A_PER_WAVE; ++i) {
      const int q = wave * C::A_PER_WAVE + i;
      const int r = 4 * q + (lane >> 4), slot = lane & 15;  // 4 token rows of 256 bytes per copy
      const int rr = min(mb + r, n_e - 1);
      const uint32_t arow = (NMAT == 2) ? uint32_t(perm[off + rr]) : uint32_t(off + rr);
      a_voff[i] = arow * uint32_t(K * 2) + 16u * uint32_t(slot ^ (r & 15));
    }
    // stage fs of the workgroup's stream: stage fs % NS of column block fs / NS
    auto copy_stage = [&](int slot, int fs) {
      const uint32_t so = lds0 + uint32_t(slot * C::STAGE);
      const int blk = fs / NS;
      const int k0 = kbeg + (fs - blk * NS) * OI_KS;
      const size_t wo = (size_t(blk) * OI_COLS * K + size_t(k0)) * ESZ;
#pragma unroll
      for (int i = 0; i < C::W_PER_WAVE; ++i)
        g2lds16_nt(wb0 + wo, w_voff[i], so + uint32_t((16 * wave + C::WROWS_PER_COPY * i) * C::ROWB));
      if (NMAT == 2) {
#pragma unroll
        for (int i = 0; i < C::W_PER_WAVE; ++i)
          g2lds16_nt(wb1 + wo, w_voff[i],
                  so + uint32_t(C::WTILE + (16 * wave + C::WROWS_PER_COPY * i) * C::ROWB));
      }
#pragma unroll
      for (int i = 0; i < C::A_PER_WAVE; ++i)
        g2lds16(A + k0, a_voff[i], so + uint32_t(NMAT * C::WTILE + (wave * C::A_PER_WAVE + i) * 1024));
    };

    f32x4_t acc[NMAT][MT];
    f32x4_t part[KS == 1 ? 1 : KS - 1][NMAT][MT];  // KS = 4: sums of quarters 0 .. 2
    float cpart[KS > 1 && GROUPED ? KS - 1 : 1][NMAT];  // ... and their units (grouped scales)
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[m][mt] = f32x4_t{0, 0, 0, 0};

    // GROUPED: current group's scales of this lane's column (zero replaced by one), the keep masks of its int8
    // values, and the raw scales of the next group
    float cur[NMAT];
    uint32_t keep[NMAT];
    u32x4_t pend_lo[NMAT], pend_hi[NMAT];  // uniform loads: the 16 columns of the wave
    auto fetch_group = [&](int grp) {
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        const uint16_t* p = (m ? s1w : s0w) + size_t(grp) * N;
        pend_lo[m] = *reinterpret_cast<const u32x4_t*>(p);
        pend_hi[m] = *reinterpret_cast<const u32x4_t*>(p + 8);
      }
    };
    int gnext = kbeg, gi = GROUPED ? kbeg / sl.gsize : 0;
    float s_fix[NMAT];  // one scale group: the lane's column scales
    if (INT8) fetch_group(gi);
    if (INT8 && !GROUPED) {
#pragma unroll
      for (int m = 0; m < NMAT; ++m) s_fix[m] = bf16f(uint16_t(lane_scale_bits(pend_lo[m], pend_hi[m], c16)));
    }
    // results of the lane: column nbase + OI_COLS blk + wrow, token rows mb + 16 mt + 4 g + v; NMAT = 1 stores
    // chunk `split`
    auto store = [&](int split, int blk) {
      const int n = nbase + OI_COLS * blk + wrow;
      float s_m[NMAT];
#pragma unroll
      for (int m = 0; m < NMAT; ++m) s_m[m] = GROUPED ? cur[m] : (INT8 ? s_fix[m] : 1.0f);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = mb + 16 * mt + 4 * g + v;
          if (row < n_e) {
            if constexpr (NMAT == 2) {
              float a = acc[0][mt][v], b = acc[1][mt][v];
              if (INT8) { a *= s_m[0]; b *= s_m[1]; }
              static_cast<uint16_t*>(out)[size_t(off + row) * N + n] = uint16_t(f2bf(gelu_erf(a) * b));
            } else {
              const float y = INT8 ? acc[0][mt][v] * s_m[0] : acc[0][mt][v];
              (static_cast<float*>(out) + split * split_stride)[size_t(off + row) * N + n] = y;
            }
          }
        }
    };

    int chunk = 0, cnext = down_chunk_begin(1, K, spw);  // NMAT = 1: the chunk being summed and its end
    // ---- prologue: stages 0 .. NSTG-2 (past the end: the last stage again, into slots never read)
    const int FS = NB * NS;  // stages of the stream
#pragma unroll
    for (int s = 0; s < C::NSTG - 1; ++s) copy_stage(s, min(s, FS - 1));

    for (int fs = 0; fs < FS; ++fs) {
      const int s = fs % NS;               // stage within the column block
      wait_vm<(C::NSTG - 2) * C::CPW>();  // this wave's copies of stage fs landed
      lds_barrier();                       // ... every wave's; every wave finished reading stage fs - 1
      if constexpr (NB > 1) {
        if (s == 0 && fs > 0) {
          // the previous block's results (the stores add to the vector memory count: the copy waits only get
          // stronger)
          store(0, fs / NS - 1);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[0][mt] = acc[1][mt] = f32x4_t{0, 0, 0, 0};
        }
      }
      copy_stage((fs + C::NSTG - 1) % C::NSTG, min(fs + C::NSTG - 1, FS - 1));
      const int k0 = kbeg + s * OI_KS;
      if constexpr (KS > 1) {
        if (s > 0 && s % (NS / KS) == 0) {  // stage s opens quarter q: keep the sum of quarter q - 1 apart
          const int q = s / (NS / KS);
#pragma unroll
          for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
              for (int qq = 0; qq < KS - 1; ++qq)
                if (qq == q - 1) part[qq][m][mt] = acc[m][mt];
              acc[m][mt] = f32x4_t{0, 0, 0, 0};
            }
          if constexpr (GROUPED) {
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
              for (int qq = 0; qq < KS - 1; ++qq)
                if (qq == q - 1) cpart[qq][m] = cur[m];
          }
        }
      }
      if (GROUPED && k0 == gnext) {  // stage s opens group gi
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
          const uint32_t bits = lane_scale_bits(pend_lo[m], pend_hi[m], c16);
          const bool z = (bits & 0x7fffu) == 0;
          const float nv = z ? 1.0f : bf16f(uint16_t(bits));
          keep[m] = z ? 0u : ~0u;
          if (k0 != kbeg) {
            const float r = cur[m] / nv;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[m][mt] *= r;
          }
          cur[m] = nv;
        }
        ++gi;
        gnext = gi * sl.gsize;
        if (gnext < kbeg + NS * OI_KS) fetch_group(gi);
      }
      const lds_u8* st = lds + (fs % C::NSTG) * C::STAGE;
#pragma unroll
      for (int t = 0; t < OI_KS / 32; ++t) {
        u32x4_t a[MT], b[NMAT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int chunk = 4 * t + g;
          a[mt] = *(const __attribute__((address_space(3))) u32x4_t*)(
              st + NMAT * C::WTILE + (16 * mt + c16) * OI_AROW + 16 * (chunk ^ c16));
        }
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
          const lds_u8* wt = st + m * C::WTILE + wrow * C::ROWB;
          if constexpr (INT8) {
            u32x2_t v = *(const __attribute__((address_space(3))) u32x2_t*)(
                wt + 16 * C::wslot(2 * t + (g >> 1), wrow) + 8 * (g & 1));
            if (GROUPED) v &= u32x2_t{keep[m], keep[m]};
            b[m] = i8x8_to_bf16(v);
          } else {
            b[m] = *(const __attribute__((address_space(3))) u32x4_t*)(wt + 16 * C::wslot(4 * t + g, wrow));
          }
        }
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[m][mt] = mfma16x16x32(a[mt], b[m], acc[m][mt]);
      }
      if (NMAT == 1 && s + 1 < NS && (s + 1) * OI_KS == cnext) {  // end of a chunk that is not the last
        store(chunk, 0);
        cnext = down_chunk_begin(++chunk + 1, K, spw);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[0][mt] = f32x4_t{0, 0, 0, 0};
      }
    }
    wait_vm<0>();   // the copies past the end
    lds_barrier();  // every wave done with the ring before the next pass refills it
    if constexpr (KS > 1 && GROUPED) {  // fma(q2, c2 / u, fma(q1, c1 / u, q0 * (c0 / u))) + q3, u = unit of q3
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        const float u = cur[m];
        const float r[3] = {cpart[0][m] / u, cpart[1][m] / u, cpart[2][m] / u};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            float t = part[0][m][mt][v] * r[0];
            t = __builtin_fmaf(part[1][m][mt][v], r[1], t);
            t = __builtin_fmaf(part[2][m][mt][v], r[2], t);
            acc[m][mt][v] = t + acc[m][mt][v];
          }
      }
    } else if constexpr (KS > 1) {  // ((q0 + q1) + q2) + q3
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[m][mt] = ((part[0][m][mt] + part[1][m][mt]) + part[2][m][mt]) + acc[m][mt];
    }
    store(NMAT == 1 ? spw - 1 : 0, NB - 1);
  }
}

// Kernel eligibility: stages of 128 k must tile each K chunk and each scale group.
bool oi_stream_fits(int Kc, bool int8, ScaleLayout sl, int K) {
  if (Kc % OI_KS != 0) return false;
  if (int8 && sl.gsize < K && sl.gsize % OI_KS != 0) return false;
  return true;
}

template <int NMAT, bool INT8, bool GROUPED>
static void launch_oi_mt(int mt, dim3 grid, hipStream_t s, const uint16_t* A, const void* W0, const void* W1,
                         const uint16_t* sc0, const uint16_t* sc1, ScaleLayout sl, const int32_t* counts,
                         const int32_t* offsets, const int32_t* perm, int K, int N, int Kc, int spw, void* out,
                         int64_t split_stride) {
  const dim3 block(256);
  if (mt == 1)
    oi_stream_kernel<NMAT, INT8, GROUPED, 1><<<grid, block, 0, s>>>(A, W0, W1, sc0, sc1, sl, counts, offsets, perm,
                                                                    K, N, Kc, spw, out, split_stride);
  else
    oi_stream_kernel<NMAT, INT8, GROUPED, 2><<<grid, block, 0, s>>>(A, W0, W1, sc0, sc1, sl, counts, offsets, perm,
                                                                    K, N, Kc, spw, out, split_stride);
}

// Column blocks of 64 per workgroup of the bf16 up-projection: 8 where f splits into whole 512-column ranges and
// the experts that can be hit hold at least 512 of them, else 1.  Measured on MI355X at Grok-1 shape, up-projection
// ms with 1 -> 8 blocks: T = 4 0.482 -> 0.471, T = 8 0.937 -> 0.917, T = 16 0.942 -> 0.924, T = 64 0.959 -> 0.941
// (2 or 4 blocks in between); fewer tokens keep 1 (T = 2 with 4 blocks: 0.350 -> 0.376).
int oi_up_blocks(int f, int E, int slots) {
  const int64_t hit = slots < E ? slots : E;
  return (f % (OI_COLS * 8) == 0 && hit * (f / (OI_COLS * 8)) >= 512) ? 8 : 1;
}

hipError_t launch_up_stream_oi(const uint16_t* x, const void* w1, const void* wv, const uint16_t* s1,
                               const uint16_t* sv, ScaleLayout sl, const int32_t* counts, const int32_t* offsets,
                               const int32_t* perm, int d, int f, int E, int slots, bool int8, int mt,
                               uint16_t* h, hipStream_t s) {
  const dim3 grid(f / OI_COLS, 1, E);  // one chunk: the whole d axis
  const bool grouped = int8 && sl.gsize < d;
  if (up_stream_ksplit(d, f, E) == 4) {  // the [in, out] kernel splits d: sum the same quarters
    const dim3 block(256);
#define GM_OI4(I8, GR, MT) oi_stream_kernel<2, I8, GR, MT, 4><<<grid, block, 0, s>>>(x, w1, wv, s1, sv, sl, counts, \
                                                                                    offsets, perm, d, f, d, 1, h, 0)
#define GM_OI4_MT(I8, GR) do { if (mt == 1) GM_OI4(I8, GR, 1); else GM_OI4(I8, GR, 2); } while (0)
    if (grouped) GM_OI4_MT(true, true);
    else if (int8) GM_OI4_MT(true, false);
    else GM_OI4_MT(false, false);
#undef GM_OI4_MT
#undef GM_OI4
    return hipGetLastError();
  }
  if (grouped)
    launch_oi_mt<2, true, true>(mt, grid, s, x, w1, wv, s1, sv, sl, counts, offsets, perm, d, f, d, 1, h, 0);
  else if (int8)
    launch_oi_mt<2, true, false>(mt, grid, s, x, w1, wv, s1, sv, sl, counts, offsets, perm, d, f, d, 1, h, 0);
  else {
    const int nb = oi_up_blocks(f, E, slots);
    const dim3 gridb(f / (OI_COLS * nb), 1, E), block(256);
#define GM_OIB(MT, NB) oi_stream_kernel<2, false, false, MT, 1, NB><<<gridb, block, 0, s>>>(x, w1, wv, s1, sv, sl, \
                                                                                        counts, offsets, perm, d, f, d, 1, h, 0)
#define GM_OIB_NB(MT) do { if (nb == 8) GM_OIB(MT, 8); else GM_OIB(MT, 1); } while (0)
    if (mt == 1) GM_OIB_NB(1);
    else GM_OIB_NB(2);
#undef GM_OIB_NB
#undef GM_OIB
  }
  return hipGetLastError();
}

hipError_t launch_down_stream_oi(const uint16_t* h, const void* w2, const uint16_t* s2, ScaleLayout sl,
                                 const int32_t* counts, const int32_t* offsets, int d, int f, int E, int slots,
                                 int S, bool int8, int mt, float* y, hipStream_t s) {
  const int spw = S;  // chunks per workgroup: all of them (partial sums still stored per chunk)
  const dim3 grid(d / OI_COLS, 1, E);
  const int64_t stride = int64_t(slots) * d;
  const bool grouped = int8 && sl.gsize < f;
  const int Kc = f;
  if (grouped)
    launch_oi_mt<1, true, true>(mt, grid, s, h, w2, nullptr, s2, nullptr, sl, counts, offsets, nullptr, f, d, Kc,
                                spw, y, stride);
  else if (int8)
    launch_oi_mt<1, true, false>(mt, grid, s, h, w2, nullptr, s2, nullptr, sl, counts, offsets, nullptr, f, d, Kc,
                                 spw, y, stride);
  else
    launch_oi_mt<1, false, false>(mt, grid, s, h, w2, nullptr, s2, nullptr, sl, counts, offsets, nullptr, f, d, Kc,
                                  spw, y, stride);
  return hipGetLastError();
}

}  // namespace gm
