// Tile scheduling and epilogue shared by the two LDS-tiled grouped-GEMM kernels (gfx950).
//
// Expert FFN, page "A functional bridge between openai/grok and xai-org/grok-1" (architecture diagram):
// y = (GELU(x W1) (*) (x Wv)) W2.
//
// A workgroup of 4 waves computes a 256-row x 256-column output tile of the expert-sorted assignment slots:
//   * up-projection (NMAT = 2): 128 columns of W1 and the same 128 columns of Wv; h = bf16(GELU(a) * b);
//   * down-projection (NMAT = 1): 256 columns of W2; fp32 output.
// Each wave holds a 128 x 128 accumulator tile as 4 x 4 MFMA 32x32 blocks (256 fp32 per lane).  Shorter tiles (192
// or 128 rows: 96 or 64 x 128 per wave) serve small experts and short last tiles (Rows below), and the
// register-staged int8 kernel with grouped scales, which needs accumulator registers for its rescaling.
#pragma once

#include "common.h"

namespace gm {
namespace tile {

constexpr int BM = 256;   // rows per tile
constexpr int BNT = 256;  // output columns per tile (all matrices)
// Column tiles per group in the tile order: the up-projection streams W1|Wv (6.4 GB) while its token rows fit
// in the 256 MB last-level cache, so it favours weight reuse (4); the down-projection's rows (h, 1.07 GB at
// T = 8192) do not fit, so it favours row reuse (8).  Measured on MI355X.
template <int NMAT> struct Group { static constexpr int N = NMAT == 2 ? 4 : 8; };

// Which row tiles of an expert with n assignment slots a launch covers:
//   All:  ceil(n / TBM) tiles of TBM rows (the last one partly filled);
//   Main: 256-row tiles of the other experts (below), except a last tile of at most 128 rows when the expert has
//         at least kSplitFull full tiles;
//   Mid:  192-row tiles of the experts with 128 < n <= kMidMax slots that 192-row tiles pad less than 256-row ones
//         (n in (128, 192], (256, 384] or (512, 576]), if MID (else those experts stay in Main);
//   Tail: one 128-row tile per expert: the whole expert if it has at most 128 slots, else that split-off last tile.
// Main, Mid and Tail together cover every row once.  Smaller tiles spend less MFMA work on padding rows, which
// decides small experts (batches of a few hundred tokens, the small experts of skewed routing).  A tail split off a
// large expert runs in a later launch and reads the expert's weight columns again, without the row sharing of the
// 256-row launch, so only experts with many full tiles (which read them many times anyway) give up their tail
// (measured on MI355X).  The down-projection runs without Mid: its launches hold few rounds of tiles, and the
// partly idle last round of one more launch cost more than the 192-row tiles saved (measured on MI355X).
enum class Rows { All, Main, Mid, Tail };
constexpr int kSplitFull = 4;
constexpr int kMidMax = 576;

__device__ __forceinline__ bool mid_expert(int n) {
  return n > 128 && n <= kMidMax && (n + 191) / 192 * 192 < (n + 255) / 256 * 256;
}

template <Rows R, int TBM, bool MID = true>
__device__ __forceinline__ int row_tiles(int n) {
  const bool small = n > 0 && n <= 128;
  const bool mid = MID && mid_expert(n);
  const bool split = n / 256 >= kSplitFull && n % 256 != 0 && n % 256 <= 128;
  if constexpr (R == Rows::All) return (n + TBM - 1) / TBM;
  else if constexpr (R == Rows::Main) return (small || mid) ? 0 : (n + 255) / 256 - (split ? 1 : 0);
  else if constexpr (R == Rows::Mid) return mid ? (n + 191) / 192 : 0;
  else return (small || split) ? 1 : 0;
}

// first row (relative to the expert's first slot) and valid rows of row tile m
template <Rows R, int TBM>
__device__ __forceinline__ void tile_rows(int n, int m, int* r0, int* rows) {
  if constexpr (R == Rows::Tail) {  // n <= 128, or the last n % 256 <= 128 slots
    *r0 = n - n % 256;
    *rows = n % 256;
  } else {
    *r0 = m * TBM;
    *rows = min(TBM, n - m * TBM);
  }
}

// Tile L (in the order below) among the row tiles R of TBM rows: (expert, first row slot, valid rows, column tile).
// Order: expert -> group of NGROUP column tiles -> row tile -> column tile.
// The expert's first slot is the running sum of the counts before it (offsets[e] as the binning step writes it),
// so that no dependent load of offsets sits in the tile's prologue.
template <int NGROUP, Rows R, int TBM, bool MID>
__device__ __forceinline__ bool locate(const int32_t* counts, const int32_t* offsets, int E, int NT, int L,
                                       int* e_out, int* row0_out, int* rows_out, int* nt_out) {
  (void)offsets;
  int first = 0;
  for (int e = 0; e < E; ++e) {
    const int n = counts[e];
    const int mt = row_tiles<R, TBM, MID>(n);
    const int te = mt * NT;
    if (L < te) {
      const int ng = L / (mt * NGROUP);
      const int gsz = min(NGROUP, NT - ng * NGROUP);
      const int rem = L - ng * mt * NGROUP;
      const int m = rem / gsz;
      *nt_out = ng * NGROUP + (rem - m * gsz);
      *e_out = e;
      int r0, rows;
      tile_rows<R, TBM>(n, m, &r0, &rows);
      *row0_out = first + r0;
      *rows_out = rows;
      return true;
    }
    L -= te;
    first += n;
  }
  return false;
}

// Map workgroup p to (expert, first row slot, valid rows, column tile) for the row tiles R of TBM rows; false if p
// has no tile.
// Workgroup p runs on XCD p % 8 (round-robin dispatch).  Each XCD gets a contiguous range of tiles in the order of
// locate(), so the ~32 tiles resident on one XCD share their A rows (NGROUP ways) and their weight columns
// (32 / NGROUP ways) in that XCD's L2.
template <int NGROUP, int TBM = BM, Rows R = Rows::All, bool MID = true>
__device__ __forceinline__ bool map_tile(const int32_t* counts, const int32_t* offsets, int E, int NT, int p,
                                         int* e_out, int* row0_out, int* rows_out, int* nt_out) {
  int total = 0;
  for (int e = 0; e < E; ++e) total += row_tiles<R, TBM, MID>(counts[e]);
  total *= NT;
  const int chunk = (total + 7) >> 3;
  const int q = p >> 3;
  if (q >= chunk) return false;
  const int L = (p & 7) * chunk + q;
  if (L >= total) return false;
  return locate<NGROUP, R, TBM, MID>(counts, offsets, E, NT, L, e_out, row0_out, rows_out, nt_out);
}

// Map workgroup p of one launch over the Mid (192-row) and Tail (128-row) tiles: each XCD takes its contiguous
// eighth of the Mid tiles first, then of the Tail tiles.  *mid tells which.  Host grid: 8 (ceil(B1 / 8) +
// ceil(B2 / 8)) workgroups for upper bounds B1, B2 of the two tile counts.
template <int NGROUP>
__device__ __forceinline__ bool map_small_tile(const int32_t* counts, const int32_t* offsets, int E, int NT, int p,
                                               bool* mid, int* e_out, int* row0_out, int* rows_out, int* nt_out) {
  int t1 = 0, t2 = 0;
  for (int e = 0; e < E; ++e) {
    t1 += row_tiles<Rows::Mid, 192>(counts[e]);
    t2 += row_tiles<Rows::Tail, 128>(counts[e]);
  }
  t1 *= NT;
  t2 *= NT;
  const int x = p & 7, c1 = (t1 + 7) >> 3, c2 = (t2 + 7) >> 3;
  int q = p >> 3;
  *mid = q < c1;
  if (*mid) {
    const int L = x * c1 + q;
    return L < t1 && locate<NGROUP, Rows::Mid, 192, true>(counts, offsets, E, NT, L, e_out, row0_out, rows_out,
                                                           nt_out);
  }
  q -= c1;
  if (q >= c2) return false;
  const int L = x * c2 + q;
  return L < t2 && locate<NGROUP, Rows::Tail, 128, true>(counts, offsets, E, NT, L, e_out, row0_out, rows_out,
                                                          nt_out);
}

// Upper bound of the number of tiles, rounded to a multiple of 8 (the grid); the exact count depends on the
// per-expert counts, which only the device knows.
static inline unsigned grid_tiles(int slots, int E, int NT, int bm = BM) {
  const unsigned g = unsigned(slots / bm + E) * unsigned(NT);
  return (g + 7u) & ~7u;
}

// Epilogue.  acc[i][j] (i < MI row blocks of 32): wave (wm, wn) rows wm*32*MI + 32 i .., column sub-tile j
// (NMAT = 2: j = 0,1 are W1 columns wn*64 + 32 j, j = 2,3 the same Wv columns; NMAT = 1: columns wn*128 + 32 j).
// Lane holds column (lane & 31) of each sub-tile, rows (v & 3) + 8 (v >> 2) + 4 (lane >> 5) of each 32-row block.
// NMAT = 2 writes h = bf16(GELU(a) * b) to h [slots, N]; NMAT = 1 writes the fp32 accumulators to y [slots, N].
// Any scale has been applied to acc already.
template <int NMAT, int MI = 4>
__device__ __forceinline__ void store_tile(const f32x16_t (&acc)[MI][4], int wm, int wn, int lane, int row0, int rows,
                                           int nbase, int N, void* out) {
  const int lr = lane & 31, rhalf = 4 * (lane >> 5);
  if (NMAT == 2) {
    uint16_t* h = static_cast<uint16_t*>(out);
#pragma unroll
    for (int jn = 0; jn < 2; ++jn) {
      const int n = nbase + wn * 64 + jn * 32 + lr;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = wm * 32 * MI + i * 32 + (v & 3) + 8 * (v >> 2) + rhalf;
          if (r < rows) h[size_t(row0 + r) * N + n] = uint16_t(f2bf(gelu_erf(acc[i][jn][v]) * acc[i][2 + jn][v]));
        }
      }
    }
  } else {
    float* y = static_cast<float*>(out);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = nbase + wn * 128 + j * 32 + lr;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = wm * 32 * MI + i * 32 + (v & 3) + 8 * (v >> 2) + rhalf;
          if (r < rows) y[size_t(row0 + r) * N + n] = acc[i][j][v];
        }
      }
    }
  }
}

}  // namespace tile
}  // namespace gm
