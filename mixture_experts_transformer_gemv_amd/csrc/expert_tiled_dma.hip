// LDS-tiled grouped GEMM with direct global -> LDS copies and LDS transpose reads (bf16 weights), gfx950.
//
// Expert FFN, page "A functional bridge between openai/grok and xai-org/grok-1" (architecture diagram):
// y = (GELU(x W1) (*) (x Wv)) W2.
//
// Tile shape and order: tiles.h.  K steps of 32 in a 4-deep LDS ring (4 x 32 KB).  Both operands are copied
// straight from global memory into LDS with global_load_lds_dwordx4 (no registers, no VALU), 16 bytes per lane,
// addressed as a wave-uniform base plus a per-lane 32-bit offset:
//   * A (activations): copied per pair of K steps, [256 rows][64 k] with 128-byte rows (full cache lines), rows
//     0..127 in the A region of the pair's first ring slot and 128..255 in that of its second; the 16-byte k chunk
//     c of row r sits in slot c ^ ((r >> 1) & 7).  Even steps copy the activations of the pair two steps ahead.
//     With grouped int8 scales per K step instead: [256 rows][32 k], 64-byte rows, chunk c of row r in slot
//     c ^ ((r >> 2) & 3);
//   * weights as two [32 k][128 column] sub-tiles (up: W1 and Wv; down: two halves of the W2 columns) with
//     256-byte rows; the 8-column chunk c of row k sits in slot c ^ (4 (k & 3)).
// The XOR swizzles are chosen on the global side (which chunk each lane fetches) so that the MFMA operand reads
// hit distinct LDS banks.  A fragments are 16-byte reads; the weights are stored [in, out] (columns contiguous),
// so their MFMA fragments (8 consecutive k of one column per lane) come from two ds_read_b64_tr_b16: within each
// 16-lane group, lane j receives element j % 4 of the 8 bytes addressed by lane 4 r + j / 4 (r = 0..3), i.e. 4
// consecutive k of one column when four lanes address four consecutive k rows.
// Weights stored [E, out, in] (OUTIN) are K-contiguous like A, so their fragments are plain 16-byte reads; but
// copying them per 32-k step would fetch 64-byte row pieces, half of each 128-byte line at a time (measured: twice
// the HBM traffic and 64-byte row pieces read ~15% slower).  So their tile is copied per pair of K steps,
// [256 weight rows][64 k] with 128-byte rows (16-byte chunk c of row r in slot c ^ ((r >> 1) & 7)), into one of
// three pair slots beside a 4-deep ring of A stages (4 x 16 KB + 3 x 32 KB = 160 KB); a pair's copies are issued
// during the steps four and three steps ahead of it (half-step 1 of the even one, both half-steps of the odd one),
// so that they are spread over the half-steps the activation copies leave free.
// Schedule: one workgroup barrier per K step, between its two 16-deep halves; every MFMA is followed by at most
// one LDS fragment read or one copy (pinned with sched_barrier), so the copies (half of step kt+3 after the
// barrier, the other half in the next half-step) and the fragments of the next half-step are issued in the
// shadow of the 32-cycle MFMAs.  The down-projection may split K over gridDim.y workgroups (fp32 partial sums,
// added by the combine) so that its smaller number of tiles still fills the chip.  Up-projection epilogue: the
// GELU product tile is staged in the idle ring and written as 16-byte row pieces.
// Tile heights: the body is compiled for 256, 192 and 128 rows (4, 3 or 2 row blocks of 32 per wave; every copy,
// fragment and epilogue loop scales with the height).  The 256-row tiles run in one launch (for the bf16 [in, out]
// up-projection the persistent kernel of expert_persist.hip); small experts and the short last tiles of large ones
// run in a second launch (tiles.h gives the rules), whose 128-row tiles read each weight byte once and copy it with
// the nontemporal hint.
#include "common.h"
#include "dma.h"
#include "launch.h"
#include "tiles.h"

namespace gm {

namespace {
using tile::BM;
using tile::BNT;
constexpr int BK = 32;                  // K per ring stage
constexpr int NSTAGE = 4;               // ring depth
constexpr int A_STAGE = BM * BK * 2;    // bytes: [256 rows][32 k]
template <bool INT8> constexpr int b_sub() { return BK * 128 * (INT8 ? 1 : 2); }  // bytes: [32 k][128 col]
constexpr int B_PAIR = BM * 2 * BK * 2;  // bytes: [256 weight rows][64 k] ([out, in] weights)
constexpr int NPAIR = 3;                // pair slots
}

// A: x [*, K] (gathered through perm, NMAT = 2) or h [slots, K] (NMAT = 1), bf16, a_bytes bytes in all (< 2^31).
// B0/B1: weights [E, K, N] (bf16, or int8 if INT8), or bf16 [E, N, K] if OUTIN (B1 only for NMAT = 2).  INT8:
// per-column bf16 scales s0 (of B0), s1 (of B1) at expert stride s_estride.  out: h bf16 [slots, N] (NMAT = 2)
// or y f32 [slots, N] (NMAT = 1).
// LDS bytes of one tile body
template <int NMAT, bool OUTIN, bool INT8, int TBM>
constexpr int tile_lds_bytes() {
  return OUTIN ? NSTAGE * TBM * BK * 2 + NPAIR * B_PAIR : NSTAGE * (TBM * BK * 2 + 2 * b_sub<INT8>());
}
// Grouped int8 scales: at most this many groups along K, their scales for the tile's 256 output columns kept as
// fp32 in LDS beside the ring (GROUPED tiles only).
constexpr int kDmaMaxGroups = 8;
constexpr int kScaleTableBytes = kDmaMaxGroups * BNT * 4;

// One output tile: expert e, assignment rows row0 .. row0 + rows - 1 (rows <= TBM), column tile ntile; lds holds
// tile_lds_bytes() bytes (plus kScaleTableBytes if GROUPED).  B_NT: nontemporal weight copies (for launches that
// read each weight byte once).  GROUPED (int8, [in, out], 128-row tiles): int8 scales in groups of gsize rows of
// K (at most kDmaMaxGroups groups); otherwise one scale per column, or none for bf16.
template <int NMAT, bool OUTIN, bool INT8, int TBM, bool B_NT = (TBM == 128), bool GROUPED = false,
          bool TRACE = false>
__device__ __forceinline__ void tiled_dma_tile(const uint16_t* __restrict__ A, const void* __restrict__ B0,
                                                        const void* __restrict__ B1,
                                                        const uint16_t* __restrict__ s0,
                                                        const uint16_t* __restrict__ s1, int64_t s_estride,
                                                        const int32_t* __restrict__ counts,
                                                        const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ perm, uint32_t a_bytes, int K,
                                                        int N, void* __restrict__ out, int64_t split_stride, int e,
                                                        int row0, int rows, int ntile, lds_u8* lds, int gsize = 0,
                                                        uint64_t* trace = nullptr) {
  static_assert(!(OUTIN && INT8), "int8 weights are tiled from [E, K, N] storage");
  static_assert(TBM == 256 || TBM == 192 || TBM == 128, "tiles of 256, 192 or 128 rows");
  static_assert(!GROUPED || (INT8 && !OUTIN && TBM == 128), "grouped scales: int8 [in, out] weights, 128-row tiles");
  static_assert(!OUTIN || !GROUPED, "[out, in] tiles copy their activations per K-step pair");
  constexpr int BNM = BNT / NMAT;  // columns per matrix
  constexpr int MI = TBM / 64;     // row blocks of 32 per wave (waves 2 x 2: TBM / 2 rows each)
  constexpr int AP = TBM / 64;     // 1 KB activation copies per wave and K step
  constexpr int NMF = 4 * MI;      // MFMAs per wave and half-step
  constexpr int A_STG = TBM * BK * 2;  // bytes: [TBM rows][32 k]
  constexpr int B_SUB = b_sub<INT8>();
  constexpr int STAGE = A_STG + 2 * B_SUB;
  constexpr int WB = INT8 ? 1 : 2;             // bytes per weight
  constexpr int BCOPIES = INT8 ? 2 : 4;        // 1 KB weight copies per wave and K step ([in, out])
  constexpr int CPS = AP + BCOPIES;            // copies per wave and K step ([out, in]: AP + 4)
  constexpr int A_STRIDE = OUTIN ? A_STG : STAGE;  // between ring slots of A
  // The activations are copied per pair of K steps, 128 contiguous bytes (64 k) of each row per copy, so that a
  // copy instruction reads 8 full 128-byte lines instead of 16 half lines (the vector memory path is the K loop's
  // limit; measured on MI355X at Grok-1 shape, bit-identical: prefill down-projection 5.55 -> 5.32 ms, int8
  // weights at T = 8192 18.45 -> 17.88 ms per layer, [out, in] weights 17.5 -> 16.9 ms; with grouped int8 scales
  // 7.15 -> 7.24 ms at T = 2048, so those keep per-step copies).  The pair's TBM rows x 128 bytes fill the A
  // regions of the ring slots of its two steps: rows 0..TBM/2-1 in the first, the rest in the second.
  constexpr bool PAIRA = !GROUPED;
  constexpr int APP = 2 * AP;                   // 1 KB activation copies per wave and step pair
  // Launches whose tiles read each weight byte once (one 128-row tile per expert and column tile) copy the weights
  // with the nontemporal hint; tiles that share weight columns through the caches keep the default policy.
  auto copy_b = [](const void* base, uint32_t voff, uint32_t dst) {
    if constexpr (B_NT) g2lds16_nt(base, voff, dst);
    else g2lds16(base, voff, dst);
  };
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nbase = ntile * BNM;
  // split blockIdx.y of gridDim.y covers k in [ksplit * Ks, (ksplit + 1) * Ks)
  const int Ks = K / gridDim.y;
  const int kbase = blockIdx.y * Ks;

  // ---- copies.  A: wave w, piece i copies rows (TBM/4) w + 16 i + lane/4; lane's slot (lane & 3) of the 64-byte row
  // holds k chunk (lane & 3) ^ ((row >> 2) & 3).  Byte offsets from A (32 bits).  Rows past the expert's end (the
  // tail tile) get an out-of-range offset, so their copies write zeros: those rows are never stored, and
  // multiplying zeros takes markedly less power than multiplying data.
  // PAIRA: piece i copies rows (TBM/4) w + 8 i + lane/8; lane's slot (lane & 7) of the 128-byte row holds k chunk
  // (lane & 7) ^ ((row >> 1) & 7).
  const u32x4_t a_rsrc = buffer_rsrc(A, a_bytes);
  constexpr int NAV = PAIRA ? APP : AP;
  uint32_t a_voff[NAV];
#pragma unroll
  for (int i = 0; i < NAV; ++i) {
    const int r = PAIRA ? (TBM / 4) * wave + 8 * i + (lane >> 3) : (TBM / 4) * wave + 16 * i + (lane >> 2);
    if (r < rows) {
      const uint32_t arow = (NMAT == 2) ? uint32_t(perm[row0 + r]) : uint32_t(row0 + r);
      const uint32_t chunk = PAIRA ? uint32_t((lane & 7) ^ ((r >> 1) & 7)) : uint32_t((lane & 3) ^ ((r >> 2) & 3));
      a_voff[i] = (arow * uint32_t(K) + 8u * chunk) * 2u;
    } else {
      a_voff[i] = 0x80000000u;
    }
  }
  // B: weight sub-tile sub = wave >> 1 (NMAT = 2: W1 / Wv columns nbase..+127; NMAT = 1: W2 columns
  // nbase + 128 sub ..+127).  bf16: piece i copies k rows 16 (wave & 1) + 4 i + lane/16, lane's slot (lane & 15)
  // of the 256-byte row holds column chunk (lane & 15) ^ (4 (k & 3)).  int8: piece i copies k rows
  // 16 (wave & 1) + 8 i + lane/8, lane's slot (lane & 7) of the 128-byte row holds 16-column chunk
  // (lane & 7) ^ (2 ((k >> 1) & 3)) (the transpose reads below then touch distinct banks).
  const int sub = wave >> 1;
  const uint16_t* bmat = static_cast<const uint16_t*>((NMAT == 2 && sub == 1) ? B1 : B0);  // int8: bytes
  const size_t b_elem = size_t(e) * K * N + size_t(16 * (wave & 1)) * N + nbase + ((NMAT == 1) ? 128 * sub : 0);
  const uint16_t* b_base = bmat + b_elem;                                              // bf16
  const uint8_t* b_base8 = reinterpret_cast<const uint8_t*>(bmat) + b_elem;           // int8
  const uint32_t b_voff =
      INT8 ? uint32_t((lane >> 3) * N + 16 * ((lane & 7) ^ (2 * ((lane >> 4) & 3))))
           : uint32_t(((lane >> 4) * N + 8 * ((lane & 15) ^ (4 * ((lane >> 4) & 3)))) * 2);
  const uint32_t a_dst = lds0 + uint32_t((TBM / 4) * wave) * (BK * 2);
  const uint32_t b_dst = lds0 + A_STG + uint32_t(sub) * B_SUB + uint32_t(16 * (wave & 1)) * (128 * WB);
  // OUTIN: the weight tile of K-step pair q is [256 weight rows][64 k] (NMAT = 2: rows 0..127 are W1 rows
  // nbase.., 128..255 the same Wv rows; NMAT = 1: W2 rows nbase..); wave w copies tile rows 64 w .. +63, copy c
  // (0..7) rows 8 c + lane/8, lane's slot (lane & 7) of the 128-byte row holding chunk (lane & 7) ^ ((row >> 1) & 7)
  const uint16_t* bt_base = bmat + size_t(e) * K * N;
  uint32_t bp_voff[OUTIN ? 8 : 1];
  if constexpr (OUTIN) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int r = 64 * wave + 8 * c + (lane >> 3);
      const int wrow = nbase + ((NMAT == 2) ? (r & 127) : r);
      bp_voff[c] = (uint32_t(wrow) * uint32_t(K) + 8u * uint32_t((lane & 7) ^ ((r >> 1) & 7))) * 2u;
    }
  }
  const uint32_t bp_dst = lds0 + NSTAGE * A_STG + uint32_t(64 * wave) * 128;
  // piece n of the copies of K step kt into ring slot stage (n < AP: A piece n; else B piece n - AP, [in, out])
  auto copy_piece = [&](int stage, int kt, int n) {
    const uint32_t so = uint32_t(stage) * A_STRIDE;
    if (n < AP)
      b2lds16(a_rsrc, uint32_t(kbase + kt * BK) * 2u, a_voff[n], a_dst + so + uint32_t(16 * n) * (BK * 2));
    else if (INT8)  // 8 weight rows of 128 bytes per piece
      copy_b(b_base8 + size_t(kbase + kt * BK) * N + size_t(8 * (n - AP)) * N, b_voff,
              b_dst + so + uint32_t(8 * (n - AP)) * 128);
    else  // 4 weight rows of 256 bytes per piece
      copy_b(b_base + size_t(kbase + kt * BK) * N + size_t(4 * (n - AP)) * N, b_voff,
              b_dst + so + uint32_t(4 * (n - AP)) * 256);
  };
  // PAIRA: activation piece i of the step pair kd, kd + 1 (kd even) into the A regions of ring slots kd % NSTAGE
  // (rows 0..TBM/2-1) and (kd + 1) % NSTAGE; weight piece n of step kt into ring slot stage
  // (kd: the pair's first step, which places it in the ring; ks: the step its data is read from)
  auto copy_apair = [&](int kd, int ks, int i) {
    const uint32_t dst = lds0 + uint32_t(((kd + (wave >> 1)) % NSTAGE) * A_STRIDE) +
                         uint32_t((TBM / 4) * (wave & 1) + 8 * i) * 128u;
    b2lds16(a_rsrc, uint32_t(kbase + ks * BK) * 2u, a_voff[i], dst);
  };
  auto copy_bpiece = [&](int stage, int kt, int n) { copy_piece(stage, kt, AP + n); };
  // OUTIN: copy c of K-step pair q into pair slot q % 3 (past the end: the last pair again, into a free slot)
  auto copy_pair = [&](int q, int c) {
    const int qd = min(q, (Ks / BK) / 2 - 1);
    copy_b(bt_base + size_t(kbase + qd * 2 * BK), bp_voff[c],
            bp_dst + uint32_t((q % NPAIR) * B_PAIR) + uint32_t(c * 1024));
  };

  // ---- fragments.  Waves 2 x 2: wave rows wm*TBM/2 .. +TBM/2-1 (MI blocks of 32), 4 column sub-tiles of 32.
  const int wm = wave >> 1, wn = wave & 1;
  int a_off[MI][2];  // A row wm*TBM/2 + 32 i + (lane & 31), k chunk 2 ks + (lane >> 5)
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int r = wm * (TBM / 2) + 32 * i + (lane & 31);
      a_off[i][ks] = r * (BK * 2) + 16 * ((2 * ks + (lane >> 5)) ^ ((r >> 2) & 3));
    }
  // PAIRA: row 32 i + (lane & 31) of the wave's A region (that of the pair's first step for wm = 0, second for
  // wm = 1), k chunk 4 (kt & 1) + 2 ks + (lane >> 5) of its 8; the block adds 32 i rows (4 KB) and leaves the
  // swizzle unchanged, so one base offset per (kt & 1, ks)
  int a_offp[2][2];
#pragma unroll
  for (int hp = 0; hp < 2; ++hp)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int r = lane & 31;
      a_offp[hp][ks] = r * 128 + 16 * ((4 * hp + 2 * ks + (lane >> 5)) ^ ((r >> 1) & 7));
    }
  // B halves h: lane addresses k row 16 ks + 8 g + 4 h + (s >> 2) and columns col .. +3 of its sub-tile, where
  // G = lane >> 4, g = G >> 1, s = lane & 15 and col = (sub-tile column base) + 16 (G & 1) + 4 (s & 3)
  int b_off[4][2][2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int bsub = (NMAT == 2) ? (j >> 1) : wn;
    const int lc = (NMAT == 2) ? (wn * 64 + (j & 1) * 32) : (j * 32);
    const int G = lane >> 4, s = lane & 15;
    const int col = lc + 16 * (G & 1) + 4 * (s & 3);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = 16 * ks + 8 * (G >> 1) + 4 * h + (s >> 2);
        b_off[j][ks][h] = A_STG + bsub * B_SUB + k * 256 + 16 * ((col >> 3) ^ (4 * (k & 3))) + 2 * (col & 7);
      }
  }
  // INT8: one 8-bit transpose read per fragment (ds_read_b64_tr_b8: within each 16-lane group, lane j receives
  // byte j % 8 of the 8 bytes addressed by lane 2 r + j / 8, r = 0..7).  Lane 2 r + q of group G addresses k row
  // 16 ks + 8 (G >> 1) + r and columns col8 .. +7, col8 = (sub-tile column base) + 16 (G & 1) + 8 q, so lane j
  // receives k rows 16 ks + 8 (G >> 1) .. +7 of column (sub-tile column base) + 16 (G & 1) + j: its MFMA operand.
  int b8_off[4][2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int bsub = (NMAT == 2) ? (j >> 1) : wn;
    const int lc = (NMAT == 2) ? (wn * 64 + (j & 1) * 32) : (j * 32);
    const int G = lane >> 4, s = lane & 15;
    const int col8 = lc + 16 * (G & 1) + 8 * (s & 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int k = 16 * ks + 8 * (G >> 1) + (s >> 1);
      b8_off[j][ks] = A_STG + bsub * B_SUB + k * 128 + 16 * ((col8 >> 4) ^ (2 * ((k >> 1) & 3))) + (col8 & 15);
    }
  }
  // OUTIN: weight fragment j of half-step ks of the pair's step p2 (0, 1) is the 16-byte read of tile row (its
  // column), k chunk 4 p2 + 2 ks + (lane >> 5) of the 128-byte row
  int bt_off[4][2][2];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int p2 = 0; p2 < 2; ++p2) {
        const int r = ((NMAT == 2) ? ((j >> 1) * 128 + wn * 64 + (j & 1) * 32) : (wn * 128 + j * 32)) + (lane & 31);
        bt_off[j][ks][p2] = r * 128 + 16 * ((4 * p2 + 2 * ks + (lane >> 5)) ^ ((r >> 1) & 7));
      }
  // fragment piece p of half-step ks from ring slot st, in the order the MFMAs consume them:
  // A0, B0 (two halves), B1, B2, B3, A1, A2, A3 (OUTIN, INT8: A0, B0, B1, B2, B3, A1, A2, A3, one read each)
  constexpr int NPIECE = (OUTIN || INT8) ? 4 + MI : 8 + MI;
  constexpr int NSLOT = NMF > NPIECE ? NMF : NPIECE;  // instruction slots per half-step (one MFMA each, if any)
  u32x4_t fa[2][MI], fb[2][4];
  u32x2_t bh[2][4][2];
  u32x2_t b8[2][4];
  // st: the step's A slot (and, [in, out], its weight sub-tiles); sb, p2: OUTIN pair slot and step within it;
  // sa (PAIRA): the wave's A region of the step's pair, p2 the step within the pair
  auto a_read = [&](int buf, int i, const lds_u8* st, const lds_u8* sa, int p2, int ks) {
    if constexpr (PAIRA)
      fa[buf][i] = *(const __attribute__((address_space(3))) u32x4_t*)(sa + a_offp[p2][ks] + i * 32 * 128);
    else
      fa[buf][i] = *(const __attribute__((address_space(3))) u32x4_t*)(st + a_off[i][ks]);
  };
  auto read_piece = [&](int buf, const lds_u8* st, const lds_u8* sb, const lds_u8* sa, int p2, int ks, int p) {
    if (OUTIN) {
      if (p == 0) a_read(buf, 0, st, sa, p2, ks);
      else if (p <= 4)
        fb[buf][p - 1] = *(const __attribute__((address_space(3))) u32x4_t*)(sb + bt_off[p - 1][ks][p2]);
      else a_read(buf, p - 4, st, sa, p2, ks);
    } else if (INT8) {
      if (p == 0) a_read(buf, 0, st, sa, p2, ks);
      else if (p <= 4) b8[buf][p - 1] = lds_tr8(st + b8_off[p - 1][ks]);
      else a_read(buf, p - 4, st, sa, p2, ks);
    } else if (p == 0) a_read(buf, 0, st, sa, p2, ks);
    else if (p <= 8) {
      const int j = (p - 1) >> 1, h = (p - 1) & 1;
      bh[buf][j][h] = lds_tr16(st + b_off[j][ks][h]);
    } else {
      a_read(buf, p - 8, st, sa, p2, ks);
    }
  };
  // keep (GROUPED): bit j clear masks the int8 values of fragment j's column (a zero scale in the step's group)
  auto join_b = [&](int buf, uint32_t keep) {
    if (OUTIN) return;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (INT8) {
        u32x2_t v = b8[buf][j];
        if constexpr (GROUPED) {
          const uint32_t m = ((keep >> j) & 1u) ? ~0u : 0u;
          v &= u32x2_t{m, m};
        }
        fb[buf][j] = i8x8_to_bf16(v);  // exact: |q| <= 127 has 8 significant bits
      } else {
        fb[buf][j] = u32x4_t{bh[buf][j][0][0], bh[buf][j][0][1], bh[buf][j][1][0], bh[buf][j][1][1]};
      }
    }
  };

  f32x16_t acc[MI][4];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // GROUPED: the accumulators are kept in units of the current group's scale.  The scales of the tile's columns
  // for every group are staged in an LDS table before the copies start (tile column c: NMAT = 2: W1 columns
  // 0..127, Wv 128..255; NMAT = 1: W2 columns); the lane's accumulator column of sub-tile j is tcol[j].  Entering
  // group g multiplies column j by cur[j] / s[g] (zero scales replaced by one, their int8 values masked to zero);
  // the epilogue multiplies by the last group's scale, so the result is sum_g s[g] * P[g].
  const int G = GROUPED ? K / gsize : 1;
  __attribute__((address_space(3))) float* tbl =
      (__attribute__((address_space(3))) float*)(lds + tile_lds_bytes<NMAT, OUTIN, INT8, TBM>());
  int tcol[4];
  float cur[4] = {1.0f, 1.0f, 1.0f, 1.0f};
  uint32_t keep_cur = 0xfu, keep_next = 0xfu;
  int gnext = 0;  // first K row of the next group
  auto group_scale = [&](int g, int j) { return tbl[g * BNT + tcol[j]]; };
  auto group_keep = [&](int g) {
    uint32_t k = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) k |= (group_scale(g, j) != 0.0f ? 1u : 0u) << j;
    return k;
  };
  if constexpr (GROUPED) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      tcol[j] = NMAT == 2 ? ((j >> 1) * 128 + wn * 64 + (j & 1) * 32 + (lane & 31)) : (wn * 128 + j * 32 + (lane & 31));
    // thread tid writes tile column tid for every group (ordinary loads, finished before the copies start)
    const uint16_t* sp = (NMAT == 2 && tid >= 128 ? s1 : s0) + e * s_estride + nbase + (NMAT == 2 ? (tid & 127) : tid);
    for (int g = 0; g < G; ++g) tbl[g * BNT + tid] = bf16f(sp[size_t(g) * N]);
  }

  // ---- main loop.  Step kt: half-step 0 multiplies fragments buffer 0 while the 12 fragment pieces of
  // half-step 1 are read; then the wave waits for its copies of step kt+1 and joins the barrier; half-step 1
  // multiplies buffer 1 while half-step 0 of step kt+1 is read.  Each MFMA is followed by at most one LDS read and
  // at most one copy, in a fixed order.  Ring slot kt - 1 was last read before the barrier of step kt - 1, so the
  // CPS copies of step kt + 3 (into that slot) are spread evenly over both half-steps of step kt: one copy every
  // NSLOT / (CPS / 2) MFMAs.  Issued in bursts, the copies of a workgroup (16 KB within a few MFMAs) outrun what the
  // vector memory path takes in, and the waves stall at issue with the MFMA pipes idle (measured on MI355X: MFMA
  // density of the K loop 0.83 with the copies bunched around the barrier, 0.94-0.98 with no copies at all).
  // Copies past the last step re-read the last step into a ring slot that is never read again, so every step
  // issues CPS copies and the wait count is constant.
  // PAIRA: an even step kt issues the activations of the pair kt + 2, kt + 3 in half-step 0 and the weights of
  // step kt + 3 in half-step 1; an odd step the weights of step kt + 3, half in each half-step (so the wait count
  // alternates between the parities); the prologue issues the weights of step 0, the activations of pair 0 and
  // the weights of steps 1 and 2.
  // OUTIN: as PAIRA for the activations; the weight copies of pair q are issued in half-step 1 of step 2 q - 4
  // (copies 0..3) and in both half-steps of step 2 q - 3 (4, 5 and 6, 7), so every half-step but the one with the
  // activation copies issues some, and the pair has landed two steps before it is read; the prologue issues the
  // weights of pairs 0 and 1 and the activations of pair 0.  (Copying the weights of pair q at the end of half-step
  // 0 of steps 2 q - 3 and 2 q - 2, in one burst with the activations on even steps, ran the [out, in] prefill
  // down-projection 6.13 -> 6.59 ms; this order 6.21 -> 5.77 ms, measured on MI355X.)
  const int KT = Ks / BK;
  const lds_u8* bpairs = lds + NSTAGE * A_STG;
  // PAIRA: the wave's A region of step kt
  auto a_region = [&](int kt) { return lds + (((kt & ~1) + wm) % NSTAGE) * A_STRIDE; };
  // zeros in the A slots of rows past the expert's end, in every ring stage (written by this lane only; the
  // out-of-range copies leave them zero)
  if (rows < TBM) {
    if constexpr (PAIRA) {
#pragma unroll
      for (int i = 0; i < APP; ++i)
        if (a_voff[i] == 0x80000000u)
#pragma unroll
          for (int pp = 0; pp < NSTAGE; pp += 2)  // the pairs' first slots: 0 and 2
            *(__attribute__((address_space(3))) u32x4_t*)(lds + ((pp + (wave >> 1)) % NSTAGE) * A_STRIDE +
                                                          ((TBM / 4) * (wave & 1) + 8 * i) * 128 + 16 * lane) =
                u32x4_t{0u, 0u, 0u, 0u};
    } else {
#pragma unroll
      for (int i = 0; i < AP; ++i)
        if (a_voff[i] == 0x80000000u)
#pragma unroll
          for (int st = 0; st < NSTAGE; ++st)
            *(__attribute__((address_space(3))) u32x4_t*)(lds + (a_dst - lds0) + st * A_STRIDE + 16 * i * (BK * 2) +
                                                          16 * lane) = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  if constexpr (OUTIN) {
    // the weights of pair 0, the activations of pair 0, the first half of the weights of pair 1 (the steady
    // state's order)
#pragma unroll
    for (int c = 0; c < 8; ++c) copy_pair(0, c);
#pragma unroll
    for (int i = 0; i < APP; ++i) copy_apair(0, 0, i);
#pragma unroll
    for (int c = 0; c < 8; ++c) copy_pair(1, c);
    wait_vm<8>();  // pair 0 landed
  } else if constexpr (PAIRA) {
    // the weights of step 0, the activations of steps 0 and 1, the weights of steps 1 and 2 (the steady state's
    // order)
#pragma unroll
    for (int n = 0; n < BCOPIES; ++n) copy_bpiece(0, 0, n);
#pragma unroll
    for (int i = 0; i < APP; ++i) copy_apair(0, 0, i);
#pragma unroll
    for (int st = 1; st < NSTAGE - 1; ++st)
#pragma unroll
      for (int n = 0; n < BCOPIES; ++n) copy_bpiece(st, min(st, KT - 1), n);
    wait_vm<2 * BCOPIES>();  // step 0 landed (its weights and the activations of steps 0 and 1)
  } else {
#pragma unroll
    for (int s = 0; s < NSTAGE - 1; ++s)
#pragma unroll
      for (int n = 0; n < CPS; ++n) copy_piece(s, min(s, KT - 1), n);
    wait_vm<CPS * (NSTAGE - 2)>();  // step 0 landed (steps 1, 2 may be in flight)
  }
  lds_barrier();
  if (TRACE && tid == 0) trace[2] = clock64();  // prologue done
  if constexpr (GROUPED) {  // the group of step 0 (kbase is a multiple of gsize or inside a group)
    const int g0 = kbase / gsize;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float v = group_scale(g0, j);
      cur[j] = v != 0.0f ? v : 1.0f;
    }
    keep_cur = group_keep(g0);
    keep_next = g0 + 1 < G ? group_keep(g0 + 1) : keep_cur;
    gnext = (g0 + 1) * gsize;
  }
#pragma unroll
  for (int p = 0; p < NPIECE; ++p) read_piece(0, lds, bpairs, a_region(0), 0, 0, p);
  join_b(0, keep_cur);
  // One K step; P is the step's parity (kt & 1), a compile-time constant so that the [out, in] forms index their
  // pair-slot offset arrays with constants (a runtime index turns each into a chain of selects).
  auto kstep = [&](int kt, auto parity) {
    constexpr int P = decltype(parity)::value;
    if constexpr (GROUPED) {
      if (kbase + kt * BK == gnext) {  // step kt opens group g: change the accumulators' unit
        const int g = gnext / gsize;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float v = group_scale(g, j);
          const float nv = v != 0.0f ? v : 1.0f;
          const float r = cur[j] / nv;
          cur[j] = nv;
#pragma unroll
          for (int i = 0; i < MI; ++i) acc[i][j] *= r;
        }
        keep_cur = keep_next;
        keep_next = g + 1 < G ? group_keep(g + 1) : keep_cur;
        gnext += gsize;
      }
    }
    const lds_u8* st = lds + (kt % NSTAGE) * A_STRIDE;
    const lds_u8* sb = bpairs + ((kt >> 1) % NPAIR) * B_PAIR;
    const lds_u8* sa = a_region(kt);
    // [in, out]: the copies of step kt+3 into slot (kt+3) % NSTAGE, C0 of them in half-step 0 and the rest in
    // half-step 1, at evenly spaced MFMA slots.  OUTIN: four copies of pair (kt + 3) / 2 in the last 4 slots of
    // half-step 0, the activation copies of step kt+3 in the first AP slots of half-step 1.
    constexpr int C0 = (CPS + 1) / 2, C1 = CPS - C0;
    const int cstage = (kt + NSTAGE - 1) % NSTAGE, ck = min(kt + NSTAGE - 1, KT - 1);
#pragma unroll
    for (int m = 0; m < NSLOT; ++m) {
      if (m < NMF) acc[m >> 2][m & 3] = mfma32x32x16(fa[0][m >> 2], fb[0][m & 3], acc[m >> 2][m & 3]);
      if (m < NPIECE) read_piece(1, st, sb, sa, P, 1, m);
      if constexpr (OUTIN) {
        if constexpr (P == 0) {  // the activations of the pair kt + 2, kt + 3 (past the end: the last pair again)
#pragma unroll
          for (int c = 0; c < APP; ++c)
            if (m == (c * NSLOT) / APP) copy_apair(kt + 2, min(kt + 2, KT - 2), c);
        } else {  // the second half of the weights of pair (kt + 3) / 2: copies 4, 5 here, 6, 7 in half-step 1
#pragma unroll
          for (int c = 0; c < 2; ++c)
            if (m == (c * NSLOT) / 2) copy_pair((kt + 3) >> 1, 4 + c);
        }
      } else if constexpr (PAIRA) {
        if constexpr (P == 0) {  // the activations of the pair kt + 2, kt + 3 (past the end: the last pair again)
#pragma unroll
          for (int c = 0; c < APP; ++c)
            if (m == (c * NSLOT) / APP) copy_apair(kt + 2, min(kt + 2, KT - 2), c);
        } else {
#pragma unroll
          for (int c = 0; c < BCOPIES / 2; ++c)
            if (m == (c * NSLOT) / (BCOPIES / 2)) copy_bpiece(cstage, ck, c);
        }
      } else {
#pragma unroll
        for (int c = 0; c < C0; ++c)
          if (m == (c * NSLOT) / C0) copy_piece(cstage, ck, c);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    join_b(1, keep_cur);
    // step kt+1 landed (the copies of step kt+2 and the first C0 of step kt+3 may be in flight)
    // PAIRA: issued after the last copy step kt + 1 needs are, for kt even, the odd step kt - 1's weights and this
    // step's activations, for kt odd, the even step kt - 1's weights and the first half of this step's
    // OUTIN: issued after the activations of the pair kt + 1 belongs to (the last copy it needs: its weights came
    // earlier) are, for kt even (pair kt / 2), the weights of step kt - 2 (4), step kt - 1 (4) and this step's
    // activations; for kt odd (pair (kt + 1) / 2), the weights of step kt - 1 (4) and half-step 0 of this step (2)
    if constexpr (OUTIN) wait_vm<P == 0 ? APP + 8 : 6>();
    else if constexpr (PAIRA) wait_vm<P == 0 ? BCOPIES + APP : BCOPIES + BCOPIES / 2>();
    else wait_vm<CPS * (NSTAGE - 3) + C0>();
    lds_barrier();  // ... for every wave; every wave finished reading step kt
    const lds_u8* nst = lds + ((kt + 1) % NSTAGE) * A_STRIDE;
    const lds_u8* nsb = bpairs + (((kt + 1) >> 1) % NPAIR) * B_PAIR;
    const lds_u8* nsa = a_region(kt + 1);
#pragma unroll
    for (int m = 0; m < NSLOT; ++m) {
      if (m < NMF) acc[m >> 2][m & 3] = mfma32x32x16(fa[1][m >> 2], fb[1][m & 3], acc[m >> 2][m & 3]);
      if constexpr (OUTIN) {
        if constexpr (P == 0) {  // the first half of the weights of pair kt / 2 + 2
#pragma unroll
          for (int c = 0; c < 4; ++c)
            if (m == (c * NSLOT) / 4) copy_pair((kt >> 1) + 2, c);
        } else {
#pragma unroll
          for (int c = 0; c < 2; ++c)
            if (m == (c * NSLOT) / 2) copy_pair((kt + 3) >> 1, 6 + c);
        }
      } else if constexpr (PAIRA) {
        constexpr int NB1 = P == 0 ? BCOPIES : BCOPIES / 2, B1 = P == 0 ? 0 : BCOPIES / 2;
#pragma unroll
        for (int c = 0; c < NB1; ++c)
          if (m == (c * NSLOT) / NB1) copy_bpiece(cstage, ck, B1 + c);
      } else {
#pragma unroll
        for (int c = 0; c < C1; ++c)
          if (m == (c * NSLOT) / C1) copy_piece(cstage, ck, C0 + c);
      }
      if (m < NPIECE) read_piece(0, nst, nsb, nsa, 1 - P, 0, m);
      __builtin_amdgcn_sched_barrier(0);
    }
    join_b(0, (GROUPED && kbase + (kt + 1) * BK == gnext) ? keep_next : keep_cur);  // fragments of step kt+1
  };
  if constexpr (OUTIN || PAIRA) {
    for (int kt = 0; kt < KT; kt += 2) {  // KT is even: K steps come in pairs
      kstep(kt, std::integral_constant<int, 0>{});
      kstep(kt + 1, std::integral_constant<int, 1>{});
    }
  } else {
    for (int kt = 0; kt < KT; ++kt) kstep(kt, std::integral_constant<int, 0>{});  // parity unused
  }
  asm volatile("s_waitcnt vmcnt(0)");
  if (TRACE && tid == 0) trace[3] = clock64();  // K loop done

  if constexpr (NMAT == 2) {
    // h tile [TBM rows][128 columns] bf16 staged in the (now idle) ring, then written as 16-byte row pieces
    lds_barrier();
    __attribute__((address_space(3))) uint16_t* ht = (__attribute__((address_space(3))) uint16_t*)(lds);
    const int lr = lane & 31, rhalf = 4 * (lane >> 5);
#pragma unroll
    for (int jn = 0; jn < 2; ++jn) {
      const int c = wn * 64 + jn * 32 + lr;
      // int8: the column's scales multiply the fp32 accumulators before the GELU product
      const float sa = GROUPED ? cur[jn] : (INT8 ? bf16f(s0[e * s_estride + nbase + c]) : 1.0f);
      const float sb = GROUPED ? cur[2 + jn] : (INT8 ? bf16f(s1[e * s_estride + nbase + c]) : 1.0f);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int v = 0; v < 16; v += 2) {  // rows r and r + 1 of the column: one packed conversion
          const int r = wm * (TBM / 2) + i * 32 + (v & 3) + 8 * (v >> 2) + rhalf;
          float hv[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const float a = INT8 ? acc[i][jn][v + u] * sa : acc[i][jn][v + u];
            const float b = INT8 ? acc[i][2 + jn][v + u] * sb : acc[i][2 + jn][v + u];
            hv[u] = gelu_erf(a) * b;
          }
          const uint32_t pk = pack_bf16(hv[0], hv[1]);
          ht[r * 128 + c] = uint16_t(pk);
          ht[(r + 1) * 128 + c] = uint16_t(pk >> 16);
        }
    }
    lds_barrier();
    uint16_t* h = static_cast<uint16_t*>(out);
#pragma unroll
    for (int q = 0; q < TBM / 16; ++q) {
      const int chunk = q * 256 + tid;          // 16-byte chunk: row chunk / 16, columns 8 (chunk % 16) ..
      const int r = chunk >> 4, c8 = (chunk & 15) * 8;
      if (r < rows)
        *reinterpret_cast<u32x4_t*>(h + size_t(row0 + r) * N + nbase + c8) =
            *(const __attribute__((address_space(3))) u32x4_t*)(ht + r * 128 + c8);
    }
  } else {
    if constexpr (INT8) {  // the column's scale multiplies the fp32 accumulators
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float sc = GROUPED ? cur[j] : bf16f(s0[e * s_estride + nbase + wn * 128 + j * 32 + (lane & 31)]);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[i][j][v] *= sc;
      }
    }
    tile::store_tile<NMAT, MI>(acc, wm, wn, lane, row0, rows, nbase, N,
                           static_cast<float*>(out) + blockIdx.y * split_stride);
  }
  if (TRACE && tid == 0) {  // epilogue stores issued
    trace[4] = clock64();
    trace[6] = wall_clock64();
  }
}

// The grouped GEMM: workgroup blockIdx.x takes the tile map_tile gives it among the row tiles R of TBM rows, in the
// XCD-aware order.  The up-projection (NMAT = 2) gives the experts that 192-row tiles pad less to those.
template <int NMAT, bool OUTIN, bool INT8, int TBM, tile::Rows R>
__global__ __launch_bounds__(256) void tiled_dma_kernel(const uint16_t* __restrict__ A, const void* __restrict__ B0,
                                                        const void* __restrict__ B1,
                                                        const uint16_t* __restrict__ s0,
                                                        const uint16_t* __restrict__ s1, int64_t s_estride,
                                                        const int32_t* __restrict__ counts,
                                                        const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ perm, uint32_t a_bytes, int K,
                                                        int N, int E, void* __restrict__ out,
                                                        int64_t split_stride) {
  int e, row0, rows, ntile;
  if (!tile::map_tile<tile::Group<NMAT>::N, TBM, R, NMAT == 2>(counts, offsets, E, N / (BNT / NMAT), blockIdx.x,
                                                               &e, &row0, &rows, &ntile))
    return;  // whole workgroup
  __shared__ __attribute__((aligned(1024))) uint8_t smem[tile_lds_bytes<NMAT, OUTIN, INT8, TBM>()];
  tiled_dma_tile<NMAT, OUTIN, INT8, TBM>(A, B0, B1, s0, s1, s_estride, counts, offsets, perm, a_bytes, K, N, out,
                                         split_stride, e, row0, rows, ntile, (lds_u8*)(smem));
}

#ifdef GROK_MOE_TILE_TRACE
// Timestamps of every tile of the 256-row launch (built into the measurement probes only): record b (workgroup
// blockIdx.y * gridDim.x + blockIdx.x) holds [0] the hardware ids (HW_ID | XCC_ID << 32), shader-clock counter at
// [1] start, [2] prologue done, [3] K loop done, [4] epilogue stores issued, constant-rate counter at [5] start and
// [6] end, and [7] the tile (expert | row0 << 8 | rows << 32 | column tile << 44), or ~0 for a workgroup without one.
template <int NMAT>
__global__ __launch_bounds__(256) void tiled_dma_trace_kernel(const uint16_t* __restrict__ A,
                                                              const void* __restrict__ B0,
                                                              const void* __restrict__ B1,
                                                              const int32_t* __restrict__ counts,
                                                              const int32_t* __restrict__ offsets,
                                                              const int32_t* __restrict__ perm, uint32_t a_bytes,
                                                              int K, int N, int E, void* __restrict__ out,
                                                              int64_t split_stride, uint64_t* __restrict__ trace) {
  const uint64_t c0 = clock64(), w0 = wall_clock64();
  uint64_t* rec = trace + 8 * (size_t(blockIdx.y) * gridDim.x + blockIdx.x);
  int e, row0, rows, ntile;
  const bool has = tile::map_tile<tile::Group<NMAT>::N, 256, tile::Rows::Main, NMAT == 2>(
      counts, offsets, E, N / (BNT / NMAT), blockIdx.x, &e, &row0, &rows, &ntile);
  if (threadIdx.x == 0) {
    const uint32_t hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);    // HW_ID
    const uint32_t xcc = __builtin_amdgcn_s_getreg((31 << 11) | 20);  // XCC_ID
    rec[0] = uint64_t(hw) | (uint64_t(xcc) << 32);
    rec[1] = c0;
    rec[5] = w0;
    rec[7] = has ? (uint64_t(e) | (uint64_t(row0) << 8) | (uint64_t(rows) << 32) | (uint64_t(ntile) << 44))
                 : ~uint64_t(0);
  }
  if (!has) return;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[tile_lds_bytes<NMAT, false, false, 256>()];
  tiled_dma_tile<NMAT, false, false, 256, false, false, true>(A, B0, B1, nullptr, nullptr, 0, counts, offsets, perm,
                                                              a_bytes, K, N, out, split_stride, e, row0, rows, ntile,
                                                              (lds_u8*)(smem), 0, rec);
}
#endif

// The up-projection's second launch: the 192-row tiles (tile::Rows::Mid) and the 128-row tiles (tile::Rows::Tail)
// in one grid, each workgroup running the body of its tile's height (one launch fewer than a launch per height:
// an empty launch of the upper-bound grid costs ~70 us at prefill size, measured on MI355X).
template <bool OUTIN, bool INT8>
__global__ __launch_bounds__(256) void tiled_dma_small_kernel(const uint16_t* __restrict__ A,
                                                              const void* __restrict__ B0,
                                                              const void* __restrict__ B1,
                                                              const uint16_t* __restrict__ s0,
                                                              const uint16_t* __restrict__ s1, int64_t s_estride,
                                                              const int32_t* __restrict__ counts,
                                                              const int32_t* __restrict__ offsets,
                                                              const int32_t* __restrict__ perm, uint32_t a_bytes,
                                                              int K, int N, int E, void* __restrict__ out) {
  bool mid;
  int e, row0, rows, ntile;
  if (!tile::map_small_tile<tile::Group<2>::N>(counts, offsets, E, N / (BNT / 2), blockIdx.x, &mid, &e, &row0, &rows,
                                               &ntile))
    return;  // whole workgroup
  __shared__ __attribute__((aligned(1024))) uint8_t smem[tile_lds_bytes<2, OUTIN, INT8, 192>()];
  if (mid)
    tiled_dma_tile<2, OUTIN, INT8, 192>(A, B0, B1, s0, s1, s_estride, counts, offsets, perm, a_bytes, K, N, out, 0,
                                        e, row0, rows, ntile, (lds_u8*)(smem));
  else
    tiled_dma_tile<2, OUTIN, INT8, 128>(A, B0, B1, s0, s1, s_estride, counts, offsets, perm, a_bytes, K, N, out, 0,
                                        e, row0, rows, ntile, (lds_u8*)(smem));
}

// int8 weights ([in, out]) with grouped scales (at most kDmaMaxGroups groups along K): 128-row tiles of every
// expert in one launch, in the XCD-aware order, so an expert's row tiles share its weight columns in L2 (default
// copies).  128 rows leave the registers the group rescaling needs (256-row tiles spill there).
template <int NMAT>
__global__ __launch_bounds__(256) void tiled_dma_grouped_kernel(const uint16_t* __restrict__ A,
                                                                const void* __restrict__ B0,
                                                                const void* __restrict__ B1,
                                                                const uint16_t* __restrict__ s0,
                                                                const uint16_t* __restrict__ s1, int64_t s_estride,
                                                                const int32_t* __restrict__ counts,
                                                                const int32_t* __restrict__ offsets,
                                                                const int32_t* __restrict__ perm, uint32_t a_bytes,
                                                                int K, int N, int E, void* __restrict__ out,
                                                                int64_t split_stride, int gsize) {
  int e, row0, rows, ntile;
  if (!tile::map_tile<tile::Group<NMAT>::N, 128, tile::Rows::All>(counts, offsets, E, N / (BNT / NMAT), blockIdx.x,
                                                                  &e, &row0, &rows, &ntile))
    return;  // whole workgroup
  __shared__ __attribute__((aligned(1024))) uint8_t smem[tile_lds_bytes<NMAT, false, true, 128>() + kScaleTableBytes];
  tiled_dma_tile<NMAT, false, true, 128, false, true>(A, B0, B1, s0, s1, s_estride, counts, offsets, perm, a_bytes, K,
                                                      N, out, split_stride, e, row0, rows, ntile, (lds_u8*)(smem),
                                                      gsize);
}

bool tiled_dma_grouped_fits(int K, int gsize) {
  return gsize > 0 && gsize % BK == 0 && K % gsize == 0 && K / gsize <= kDmaMaxGroups;
}

hipError_t launch_up_tiled_dma_grouped(const uint16_t* x, const void* w1, const void* wv, const uint16_t* s1,
                                       const uint16_t* sv, int64_t s_estride, int gsize, const int32_t* counts,
                                       const int32_t* offsets, const int32_t* perm, int d, int f, int E, int slots,
                                       uint16_t* h, hipStream_t s) {
  const int NT = f / (BNT / 2);
  const dim3 grid(tile::grid_tiles(slots, E, NT, 128)), block(256);
  const size_t xbytes = size_t(slots / 2) * d;  // x: [slots / 2 tokens, d] bf16
  if (2 * xbytes >= (size_t(1) << 31) || size_t(2) * slots * f >= (size_t(1) << 31) ||
      !tiled_dma_grouped_fits(d, gsize) || d % (2 * BK) != 0)  // whole K-step pairs
    return hipErrorInvalidValue;
  tiled_dma_grouped_kernel<2><<<grid, block, 0, s>>>(x, w1, wv, s1, sv, s_estride, counts, offsets, perm,
                                                     uint32_t(2 * xbytes), d, f, E, h, 0, gsize);
  return hipGetLastError();
}

hipError_t launch_down_tiled_dma_grouped(const uint16_t* h, const void* w2, const uint16_t* s2, int64_t s_estride,
                                         int gsize, const int32_t* counts, const int32_t* offsets, int d, int f,
                                         int E, int slots, int S, float* y, hipStream_t s) {
  const int NT = d / BNT;
  const dim3 grid(tile::grid_tiles(slots, E, NT, 128), S), block(256);
  const size_t hbytes = size_t(slots) * f * 2;  // h: [slots, f]
  if (hbytes >= (size_t(1) << 31) || !tiled_dma_grouped_fits(f, gsize) || f % (2 * BK * S) != 0)
    return hipErrorInvalidValue;  // whole K-step pairs in every split
  tiled_dma_grouped_kernel<1><<<grid, block, 0, s>>>(h, w2, nullptr, s2, nullptr, s_estride, counts, offsets,
                                                     nullptr, uint32_t(hbytes), f, d, E, y, int64_t(slots) * d,
                                                     gsize);
  return hipGetLastError();
}

// Launches: the 256-row tiles (tile::Rows::Main); then, for the up-projection, the 192-row tiles of experts with up
// to tile::kMidMax slots that they pad less (tile::Rows::Mid) together with at most one 128-row tile per expert and
// column tile (tile::Rows::Tail: an expert with at most 128 slots, or the short last tile of a large expert); for
// the down-projection the 128-row tiles alone.  The device decides from the counts; the grids are upper bounds and
// a workgroup without a tile exits at once.
static unsigned tail_tiles(int E, int NT) { return (unsigned(E) * unsigned(NT) + 7u) & ~7u; }
static unsigned small_tiles(int slots, int E, int NT) {
  const unsigned per_expert = unsigned(tile::kMidMax / 192), bound = unsigned(slots / 192 + E);
  const unsigned b1 = (per_expert * unsigned(E) < bound ? per_expert * unsigned(E) : bound) * unsigned(NT);
  return 8u * ((b1 + 7u) / 8u) + tail_tiles(E, NT);
}

hipError_t launch_up_tiled_dma(const uint16_t* x, const void* w1, const void* wv, const uint16_t* s1,
                               const uint16_t* sv, int64_t s_estride, bool int8, bool outin, const int32_t* counts,
                               const int32_t* offsets, const int32_t* perm, int d, int f, int E, int slots,
                               uint16_t* h, hipStream_t s) {
  const int NT = f / (BNT / 2);
  const dim3 grid(tile::grid_tiles(slots, E, NT)), grid_s(small_tiles(slots, E, NT)), block(256);
  const size_t xbytes = size_t(slots / 2) * d * 2;  // x: [slots / 2 tokens, d] (two slots per token)
  if (xbytes >= (size_t(1) << 31) || size_t(2) * slots * f >= (size_t(1) << 31)) return hipErrorInvalidValue;
  if (int8 && outin) return hipErrorInvalidValue;
  if (d % (2 * BK) != 0) return hipErrorInvalidValue;  // whole K-step pairs
  const uint32_t xb = uint32_t(xbytes);
#define GM_UPD(OI, I8)                                                                                           \
  do {                                                                                                         \
    tiled_dma_kernel<2, OI, I8, 256, tile::Rows::Main><<<grid, block, 0, s>>>(x, w1, wv, s1, sv, s_estride,       \
                                                                               counts, offsets, perm, xb, d, f, E, h, 0); \
    tiled_dma_small_kernel<OI, I8><<<grid_s, block, 0, s>>>(x, w1, wv, s1, sv, s_estride, counts, offsets, perm,  \
                                                             xb, d, f, E, h);                                   \
  } while (0)
  if (int8) {
    GM_UPD(false, true);
  } else if (outin) {
    GM_UPD(true, false);
  } else if (d / BK >= 8 && d % (2 * BK) == 0) {  // bf16 [in, out]: the persistent form of the 256-row launch
    const hipError_t err = launch_up_persist(x, w1, wv, counts, perm, d, f, E, slots, h, s);
    if (err != hipSuccess) return err;
    tiled_dma_small_kernel<false, false><<<grid_s, block, 0, s>>>(x, w1, wv, s1, sv, s_estride, counts, offsets, perm,
                                                                  xb, d, f, E, h);
  } else {
    GM_UPD(false, false);
  }
#undef GM_UPD
  return hipGetLastError();
}

hipError_t launch_down_tiled_dma(const uint16_t* h, const void* w2, const uint16_t* s2, int64_t s_estride, bool int8,
                                 bool outin, const int32_t* counts, const int32_t* offsets, int d, int f, int E,
                                 int slots, int S, float* y, hipStream_t s) {
  const int NT = d / BNT;
  const dim3 grid(tile::grid_tiles(slots, E, NT), S), grid_t(tail_tiles(E, NT), S), block(256);
  const int64_t stride = int64_t(slots) * d;
  const size_t hbytes = size_t(slots) * f * 2;  // h: [slots, f]
  if (hbytes >= (size_t(1) << 31)) return hipErrorInvalidValue;
  if (int8 && outin) return hipErrorInvalidValue;
  if (f % (2 * BK * S) != 0) return hipErrorInvalidValue;  // whole K-step pairs in every split
  const uint32_t hb = uint32_t(hbytes);
#define GM_DND(OI, I8)                                                                                           \
  do {                                                                                                         \
    tiled_dma_kernel<1, OI, I8, 256, tile::Rows::Main><<<grid, block, 0, s>>>(h, w2, nullptr, s2, nullptr,        \
                                                                               s_estride, counts, offsets, nullptr, \
                                                                               hb, f, d, E, y, stride);           \
    tiled_dma_kernel<1, OI, I8, 128, tile::Rows::Tail><<<grid_t, block, 0, s>>>(h, w2, nullptr, s2, nullptr,      \
                                                                                s_estride, counts, offsets, nullptr, \
                                                                                hb, f, d, E, y, stride);          \
  } while (0)
  if (int8) GM_DND(false, true);
  else if (outin) GM_DND(true, false);
  else GM_DND(false, false);
#undef GM_DND
  return hipGetLastError();
}

}  // namespace gm
