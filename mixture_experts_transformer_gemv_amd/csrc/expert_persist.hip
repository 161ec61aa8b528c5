// Persistent form of the 256-row up-projection tiles (bf16 weights stored [in, out]), gfx950.
//
// Expert FFN, page "A functional bridge between openai/grok and xai-org/grok-1" (architecture diagram):
// h = GELU(x W1) (*) (x Wv), per assignment slot, rounded once to bf16.
//
// The tile body is that of expert_tiled_dma.hip (256 x 256 output tiles of W1|Wv columns, 32-deep K steps in a
// 4-deep LDS ring filled by direct global -> LDS copies, LDS transpose reads of the weights, one barrier per K
// step, copies spread over both half-steps).  What differs:
//   * the activations are copied for two K steps at once: each token row contributes 128 contiguous bytes (64 k)
//     per copy, so a copy instruction reads 8 full 128-byte lines instead of 16 half lines (the prefill
//     up-projection ran 10.76 -> 10.08 ms on MI355X with the per-step 64-byte pieces replaced, bit-identical).
//     The step pair's 256 rows x 128 bytes fill the activation regions (16 KB each) of the two ring slots of its
//     steps: rows 0..127 in the first, 128..255 in the second.  Even steps copy the activations of the pair two
//     steps ahead; every step copies the weights of the step three ahead;
//   * one workgroup per CU walks the tiles of its XCD (tile i, i + W, i + 2 W, ... of the XCD's contiguous range
//     in the order of tiles.h, W = workgroups per XCD), and the K steps of consecutive tiles form one stream: the
//     last four K steps of a tile copy the weights of the next tile's first three steps and the activations of its
//     first step pair (in the ring slots that follow), so a tile starts with its first steps already in LDS, and
//     the GELU epilogue of one tile runs while the next tile's first copies are in flight;
//   * the epilogue stages the h tile in the ring slot of the tile's last K step (free: the next tile's first
//     copies take the other three slots) and in 32 KB beside the ring;
//   * the activation row map (perm) of the tile after next is loaded during the epilogue, so its copy offsets are
//     ready when its copies start.
// The copy waits count vector memory operations in issue order, so every epilogue issues the same number of them:
// 8 row-map loads (of row 0 when there is no tile after next) and 16 stores of 16 bytes per lane (buffer stores;
// rows past the expert's end get an out-of-range offset and are dropped).  The first tile starts with the same
// number of loads and dropped stores.  Workgroups never wait for each other.
#include "common.h"
#include "dma.h"
#include "launch.h"
#include "tiles.h"

namespace gm {

namespace {
constexpr int PBK = 32;                       // K per ring stage
constexpr int P_A = 128 * 2 * PBK * 2;        // bytes: a slot's activation region [128 rows][64 k of a step pair]
constexpr int P_B = PBK * 128 * 2;            // bytes: one weight sub-tile [32 k][128 columns]
constexpr int P_STAGE = P_A + 2 * P_B;        // 32 KB
constexpr int P_EXTRA = 128 * 128 * 2;        // rows 128..255 of the staged h tile
constexpr int P_LDS = 4 * P_STAGE + P_EXTRA;  // 160 KB
constexpr int P_AP = 8;                       // activation copies per wave and step pair (8 rows x 128 bytes each)
constexpr int P_BP = 4;                       // weight copies per wave and step (4 rows x 256 bytes each)
constexpr int P_NPIECE = 12, P_NSLOT = 16;
constexpr int P_EPI = P_AP + 16;              // vector memory operations of one epilogue
// copy waits (operations issued after the last one a step needs, see kstep): even and odd steps
constexpr int P_WEVEN = P_BP + P_AP, P_WODD = P_BP + P_BP / 2;
constexpr uint32_t P_OOR = 0x80000000u;       // out-of-range buffer offset (x and h are < 2^31 bytes)

// One accumulator register read into a VGPR where it is used.  (Left to the compiler, the epilogue copies all 256
// accumulators out of the AGPRs at once and spills.)  The caller keeps the MFMA result hazard: wait states between
// the last MFMA and the first read.
__device__ __forceinline__ float agpr_read(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}

struct PTile {
  int e, row0, rows, ntile;
};

// Copy parameters of one tile: activation offsets of the lane's 4 pieces, the wave's weight sub-tile base, and the
// K of step s (k0 + s * kst; kst = 0 repeats one step: the copies past the last tile re-read a step nobody reads).
struct PCopy {
  uint32_t av[P_AP];
  const uint16_t* bb;
  int k0, kst;
};
}  // namespace

// TRACE (built into the measurement probes only): each tile's timestamps go to trace[8 L .. 8 L + 7] for its tile
// index L in the order of tiles.h: [0] HW_ID | XCC_ID << 32, shader-clock counter at [1] the tile's start (for a
// workgroup's first tile: the kernel's start, so that [2] - [1] is its prologue), [2] the start of its K loop,
// [3] K loop done, [4] epilogue stores issued, constant-rate counter at [5] start (as [1]) and [6] end, [7] expert |
// row0 << 8 | rows << 32 | column tile << 44.  One 64-byte buffer store per wave and epilogue (wave 0's four lanes
// write, every other lane's offset is out of range), counted with the epilogue's other operations.
template <bool TRACE>
__global__ __launch_bounds__(256) void tiled_up_persist_kernel(const uint16_t* __restrict__ A,
                                                               const uint16_t* __restrict__ W1,
                                                               const uint16_t* __restrict__ Wv,
                                                               const int32_t* __restrict__ counts,
                                                               const int32_t* __restrict__ perm, uint32_t a_bytes,
                                                               int K, int N, int E, uint16_t* __restrict__ h,
                                                               uint32_t h_bytes, uint64_t* __restrict__ trace,
                                                               uint32_t trace_bytes) {
  constexpr int NG = tile::Group<2>::N;
  constexpr int EPI = P_EPI + (TRACE ? 1 : 0);  // vector memory operations of one epilogue
  uint64_t tc_start = TRACE ? clock64() : 0, tw_start = TRACE ? wall_clock64() : 0;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[P_LDS];
  lds_u8* lds = (lds_u8*)smem;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int NT = N / 128;
  const int KT = K / PBK;

  // ---- this workgroup's tiles: XCD x = blockIdx.x % 8 owns tiles [x chunk, (x + 1) chunk) of the 256-row launch
  int total = 0;
  for (int e = 0; e < E; ++e) total += tile::row_tiles<tile::Rows::Main, 256, true>(counts[e]);
  total *= NT;
  const int chunk = (total + 7) >> 3;
  const int x = blockIdx.x & 7, W = gridDim.x >> 3;
  const int qend = min(chunk, total - x * chunk);  // tiles of this XCD
  auto tile_at = [&](int q, PTile& t) {
    tile::locate<NG, tile::Rows::Main, 256, true>(counts, nullptr, E, NT, x * chunk + q, &t.e, &t.row0, &t.rows,
                                                  &t.ntile);
  };
  int q = blockIdx.x >> 3;
  if (q >= qend) return;  // whole workgroup

  // ---- copies (as expert_tiled_dma.hip, 256-row tiles, [in, out] bf16 weights)
  const u32x4_t a_rsrc = buffer_rsrc(A, a_bytes);
  const int sub = wave >> 1;
  const uint16_t* bmat = sub ? Wv : W1;
  const uint32_t b_voff = uint32_t(((lane >> 4) * N + 8 * ((lane & 15) ^ (4 * ((lane >> 4) & 3)))) * 2);
  const uint32_t b_dst = lds0 + P_A + uint32_t(sub) * P_B + uint32_t(16 * (wave & 1)) * 256;
  // activation row of the lane's piece i of a step pair: tile row 64 wave + 8 i + lane / 8; its 16-byte chunk
  // lane % 8 of the row's 128 bytes (64 k) holds k chunk (lane % 8) ^ ((row >> 1) & 7)
  auto piece_row = [&](int i) { return 64 * wave + 8 * i + (lane >> 3); };
  auto make_copy = [&](const PTile& t, const int32_t (&pv)[P_AP], PCopy& c) {
#pragma unroll
    for (int i = 0; i < P_AP; ++i) {
      const int r = piece_row(i);
      c.av[i] = r < t.rows ? (uint32_t(pv[i]) * uint32_t(K) + 8u * uint32_t((lane & 7) ^ ((r >> 1) & 7))) * 2u : P_OOR;
    }
    c.bb = bmat + size_t(t.e) * K * N + size_t(16 * (wave & 1)) * N + t.ntile * 128;
    c.k0 = 0;
    c.kst = PBK;
  };
  // the lane's 8 row-map entries of tile t (row 0 of the map if there is no tile: the loads always happen)
  auto load_rows = [&](bool has, const PTile& t, int32_t (&pv)[P_AP]) {
#pragma unroll
    for (int i = 0; i < P_AP; ++i) {
      const int r = min(piece_row(i), t.rows - 1);
      pv[i] = perm[has ? t.row0 + r : 0];
    }
  };
  // activation piece i of the step pair s, s + 1 of tile c (s even): rows 0..127 of the tile into the activation
  // region of ring slot `slot`, rows 128..255 into that of the slot after it
  auto copy_a = [&](const PCopy& c, int slot, int s, int i) {
    const uint32_t dst = lds0 + uint32_t((slot + (wave >> 1)) & 3) * P_STAGE + uint32_t(64 * (wave & 1) + 8 * i) * 128u;
    b2lds16(a_rsrc, uint32_t(c.k0 + s * c.kst) * 2u, c.av[i], dst);
  };
  // weight piece n of step s of tile c into ring slot `slot`
  auto copy_b = [&](const PCopy& c, int slot, int s, int n) {
    const int k = c.k0 + s * c.kst;
    g2lds16(c.bb + size_t(k) * N + size_t(4 * n) * N, b_voff, b_dst + uint32_t(slot & 3) * P_STAGE + uint32_t(4 * n) * 256);
  };

  // ---- fragments (waves 2 x 2: rows wm * 128 .. +127 as 4 blocks of 32, 4 column sub-tiles of 32)
  const int wm = wave >> 1, wn = wave & 1;
  // A fragment (block i, half ks) of step kt: row 32 i + (lane & 31) of the wave's activation region (the slot of
  // the step pair's first step, or the slot after it for wm = 1), k chunk 4 (kt & 1) + 2 ks + (lane >> 5) of the
  // row's 8, at chunk position (that ^ ((row >> 1) & 7)); the block only adds 32 i rows and the swizzle depends on
  // lane & 31 alone, so one base offset per (kt & 1, ks).
  int a_base[2][2];
#pragma unroll
  for (int hp = 0; hp < 2; ++hp)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int r = lane & 31;
      a_base[hp][ks] = r * 128 + 16 * ((4 * hp + 2 * ks + (lane >> 5)) ^ ((r >> 1) & 7));
    }
  int r0 = 0;  // ring slot of the current tile's step 0
  // the wave's activation region for step kt
  auto a_region = [&](int kt) { return lds + ((r0 + (kt & ~1) + wm) & 3) * P_STAGE; };
  // B halves hh of sub-tile j, half-step ks: lane addresses k row 16 ks + 8 (G >> 1) + 4 hh + (s >> 2) and columns
  // col .. +3 (G = lane >> 4, s = lane & 15, col = wn * 64 + 32 (j & 1) + 16 (G & 1) + 4 (s & 3), sub-tile j >> 1).
  // k & 3 = (s >> 2) & 3 for every ks, hh, so ks and hh only add whole rows: one base per j & 1.
  int b_base[2];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int G = lane >> 4, s = lane & 15;
    const int col = wn * 64 + jj * 32 + 16 * (G & 1) + 4 * (s & 3);
    const int k = 8 * (G >> 1) + (s >> 2);
    b_base[jj] = P_A + k * 256 + 16 * ((col >> 3) ^ (4 * (k & 3))) + 2 * (col & 7);
  }
  u32x4_t fa[2][4], fb[2][4];
  u32x2_t bh[2][4][2];
  // piece p of the fragments of half ks of a step: p = 0, 9, 10, 11 the A blocks 0..3 from the wave's activation
  // region ast (hp = the step's parity), p = 1..8 the B halves from the step's slot st
  auto read_piece = [&](int buf, const lds_u8* st, const lds_u8* ast, int hp, int ks, int p) {
    if (p == 0) {
      fa[buf][0] = *(const __attribute__((address_space(3))) u32x4_t*)(ast + a_base[hp][ks]);
    } else if (p <= 8) {
      const int j = (p - 1) >> 1, hh = (p - 1) & 1;
      bh[buf][j][hh] = lds_tr16(st + b_base[j & 1] + (j >> 1) * P_B + (16 * ks + 4 * hh) * 256);
    } else {
      const int i = p - 8;
      fa[buf][i] = *(const __attribute__((address_space(3))) u32x4_t*)(ast + a_base[hp][ks] + i * 32 * 128);
    }
  };
  auto join_b = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      fb[buf][j] = u32x4_t{bh[buf][j][0][0], bh[buf][j][0][1], bh[buf][j][1][0], bh[buf][j][1][1]};
  };
  f32x16_t acc[4][4];
  const f32x16_t zero16 = {};

  // One K step kt of the tile whose step 0 sits in ring slot r0.  Copies: an even step issues the activations of
  // the step pair kt + 2, kt + 3 (8 pieces, half-step 0: pair ca's steps sa, sa + 1) and the weights of step kt + 3
  // (4 pieces, half-step 1: step sb of tile cb); an odd step the weights of step kt + 3 (2 pieces per half-step).
  // Before half-step 1 the copies step kt + 1 needs have landed: issued after the last of them are, for kt even,
  // the odd step kt - 1's 4 and this step's first 8 (P_WEVEN), for kt odd, step kt - 1's last 4 and this step's
  // first 2 (P_WODD).  EX: vector memory operations issued among those (an epilogue's, for a tile's step 0).
  // FIRST: the tile's first step (accumulators start from zero).
  auto kstep = [&](int kt, const PCopy& ca, int sa, const PCopy& cb, int sb, auto even, auto ex, auto first) {
    constexpr bool EVEN = decltype(even)::value;
    constexpr int EX = decltype(ex)::value;
    constexpr bool FIRST = decltype(first)::value;
    static_assert(EVEN || EX == 0, "an epilogue precedes even steps only");
    const lds_u8* st = lds + ((r0 + kt) & 3) * P_STAGE;
    const lds_u8* ast = a_region(kt);
    const int bslot = r0 + kt + 3, aslot = r0 + kt + 2;
#pragma unroll
    for (int m = 0; m < P_NSLOT; ++m) {
      acc[m >> 2][m & 3] = mfma32x32x16(fa[0][m >> 2], fb[0][m & 3], FIRST ? zero16 : acc[m >> 2][m & 3]);
      if (m < P_NPIECE) read_piece(1, st, ast, EVEN ? 0 : 1, 1, m);
      if (EVEN && (m & 1) == 0) copy_a(ca, aslot, sa, m >> 1);
      if (!EVEN && (m & 7) == 0) copy_b(cb, bslot, sb, m >> 3);
      __builtin_amdgcn_sched_barrier(0);
    }
    join_b(1);
    wait_vm<(EVEN ? P_WEVEN : P_WODD) + EX>();  // step kt + 1 landed
    lds_barrier();
    const lds_u8* nst = lds + ((r0 + kt + 1) & 3) * P_STAGE;
    const lds_u8* nast = a_region(kt + 1);
#pragma unroll
    for (int m = 0; m < P_NSLOT; ++m) {
      acc[m >> 2][m & 3] = mfma32x32x16(fa[1][m >> 2], fb[1][m & 3], acc[m >> 2][m & 3]);
      if (EVEN && (m & 3) == 0) copy_b(cb, bslot, sb, m >> 2);
      if (!EVEN && (m & 7) == 0) copy_b(cb, bslot, sb, 2 + (m >> 3));
      if (m < P_NPIECE) read_piece(0, nst, nast, EVEN ? 1 : 0, 0, m);
      __builtin_amdgcn_sched_barrier(0);
    }
    join_b(0);
  };

  // ---- h stores: 16-byte buffer stores; an offset at or past h_bytes (rows past the tile's end) is dropped
  const __amdgpu_buffer_rsrc_t h_rsrc = __builtin_amdgcn_make_buffer_rsrc(h, (short)0, int(h_bytes), 0x00020000);
  auto store_h = [&](uint32_t voff, u32x4_t v) { __builtin_amdgcn_raw_buffer_store_b128(v, h_rsrc, int(voff), 0, 0); };

  // ---- first tile: its row map, then the copies of its first three steps in the order of the steady state (the
  // weights of step 0, the activations of steps 0 and 1, the weights of steps 1 and 2), the row map of the next
  // tile and 16 dropped stores, so that the wait counts of every tile are those of the steady state
  PTile cur, nxt;
  tile_at(q, cur);
  nxt = cur;
  int32_t pv[P_AP];
  load_rows(true, cur, pv);
  PCopy cc, nc;
  make_copy(cur, pv, cc);
#pragma unroll
  for (int n = 0; n < P_BP; ++n) copy_b(cc, 0, 0, n);
#pragma unroll
  for (int i = 0; i < P_AP; ++i) copy_a(cc, 0, 0, i);
#pragma unroll
  for (int s = 1; s < 3; ++s)
#pragma unroll
    for (int n = 0; n < P_BP; ++n) copy_b(cc, s, s, n);
  bool has_next = q + W < qend;
  if (has_next) tile_at(q + W, nxt);
  load_rows(has_next, nxt, pv);
#pragma unroll
  for (int i = 0; i < EPI - P_AP; ++i) store_h(P_OOR + 16u * uint32_t(i), u32x4_t{0u, 0u, 0u, 0u});  // distinct: all issued
  wait_vm<2 * P_BP + EPI>();  // step 0 landed (its weights and the activations of steps 0 and 1)
  lds_barrier();
  const __amdgpu_buffer_rsrc_t t_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(TRACE ? trace : nullptr, (short)0, int(TRACE ? trace_bytes : 0), 0x00020000);

  for (;;) {
    // fragments of step 0, half 0 (landed and visible: the wait and barrier before)
    const lds_u8* st0 = lds + r0 * P_STAGE;
    const lds_u8* ast0 = a_region(0);
    const uint64_t tc_loop = TRACE ? clock64() : 0;
#pragma unroll
    for (int p = 0; p < P_NPIECE; ++p) read_piece(0, st0, ast0, 0, 0, p);
    join_b(0);
    using even_t = std::true_type;
    using odd_t = std::false_type;
    using ex0 = std::integral_constant<int, 0>;
    kstep(0, cc, 2, cc, 3, even_t{}, std::integral_constant<int, EPI>{}, std::true_type{});
    kstep(1, cc, 0, cc, 4, odd_t{}, ex0{}, std::false_type{});
    for (int kt = 2; kt < KT - 4; kt += 2) {
      kstep(kt, cc, kt + 2, cc, kt + 3, even_t{}, ex0{}, std::false_type{});
      kstep(kt + 1, cc, 0, cc, kt + 4, odd_t{}, ex0{}, std::false_type{});
    }
    kstep(KT - 4, cc, KT - 2, cc, KT - 1, even_t{}, ex0{}, std::false_type{});
    // the next tile's copy offsets (its row map was loaded during the last epilogue and has landed: the waits
    // above cover every operation issued before the copies of step 3); past the last tile, the current tile's
    // last step pair again
    if (has_next) {
      make_copy(nxt, pv, nc);
    } else {
      nc = cc;
      nc.k0 = (KT - 2) * PBK;
      nc.kst = 0;
    }
    kstep(KT - 3, nc, 0, nc, 0, odd_t{}, ex0{}, std::false_type{});
    kstep(KT - 2, nc, 0, nc, 1, even_t{}, ex0{}, std::false_type{});
    kstep(KT - 1, nc, 0, nc, 2, odd_t{}, ex0{}, std::false_type{});
    const uint64_t tc_kdone = TRACE ? clock64() : 0;

    // ---- epilogue: the row map of the tile after next, then the GELU product staged in LDS and stored.  32 wait
    // states after the last MFMA before its accumulators are read.
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7");
    const int qn2 = q + 2 * W;
    const bool has_next2 = has_next && qn2 < qend;
    PTile nxt2 = nxt;
    if (has_next2) tile_at(qn2, nxt2);
    load_rows(has_next2, nxt2, pv);
    // staging: rows wm * 128 .. +127 of the tile; wm = 0 in the ring slot of the last K step, wm = 1 beside the
    // ring.  Every wave passed the barrier of the last K step, after which nobody reads that slot.
    const int xslot = (r0 + KT - 1) & 3;
    __attribute__((address_space(3))) uint16_t* ht0 = (__attribute__((address_space(3))) uint16_t*)(lds + xslot * P_STAGE);
    __attribute__((address_space(3))) uint16_t* ht1 = (__attribute__((address_space(3))) uint16_t*)(lds + 4 * P_STAGE);
    {
      __attribute__((address_space(3))) uint16_t* ht = wm ? ht1 : ht0;
      const int lr = lane & 31, rhalf = 4 * (lane >> 5);
#pragma unroll
      for (int jn = 0; jn < 2; ++jn) {
        const int c = wn * 64 + jn * 32 + lr;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int v = 0; v < 16; v += 2) {  // rows r and r + 1 of the column: one packed conversion
            const int r = i * 32 + (v & 3) + 8 * (v >> 2) + rhalf;  // row within the wave's 128
            const float a0 = agpr_read(acc[i][jn][v]), b0 = agpr_read(acc[i][2 + jn][v]);
            const float a1 = agpr_read(acc[i][jn][v + 1]), b1 = agpr_read(acc[i][2 + jn][v + 1]);
            const uint32_t pk = pack_bf16(gelu_erf(a0) * b0, gelu_erf(a1) * b1);
            ht[r * 128 + c] = uint16_t(pk);
            ht[(r + 1) * 128 + c] = uint16_t(pk >> 16);
          }
      }
    }
    lds_barrier();
    const int nbase = cur.ntile * 128;
#pragma unroll
    for (int qq = 0; qq < 16; ++qq) {
      const int chunk16 = qq * 256 + tid;  // 16-byte chunk: tile row chunk16 / 16, columns 8 (chunk16 % 16) ..
      const int r = chunk16 >> 4, c8 = (chunk16 & 15) * 8;
      const __attribute__((address_space(3))) uint16_t* src = (qq < 8 ? ht0 + r * 128 : ht1 + (r - 128) * 128) + c8;
      const u32x4_t v = *(const __attribute__((address_space(3))) u32x4_t*)(src);
      const uint32_t voff = r < cur.rows ? (uint32_t(cur.row0 + r) * uint32_t(N) + uint32_t(nbase + c8)) * 2u : P_OOR;
      store_h(voff, v);
    }
    if constexpr (TRACE) {
      const uint64_t tc_epi = clock64(), tw_end = wall_clock64();
      const uint64_t hw = uint64_t(__builtin_amdgcn_s_getreg((31 << 11) | 4)) |
                          (uint64_t(__builtin_amdgcn_s_getreg((31 << 11) | 20)) << 32);
      const uint64_t code = uint64_t(cur.e) | (uint64_t(cur.row0) << 8) | (uint64_t(cur.rows) << 32) |
                            (uint64_t(cur.ntile) << 44);
      const uint64_t w[8] = {hw, tc_start, tc_loop, tc_kdone, tc_epi, tw_start, tw_end, code};
      const int i = lane & 3;
      uint64_t lo = w[0], hi = w[1];
#pragma unroll
      for (int k = 1; k < 4; ++k)
        if (i == k) { lo = w[2 * k]; hi = w[2 * k + 1]; }
      const uint32_t toff = (wave == 0 && lane < 4) ? uint32_t(x * chunk + q) * 64u + 16u * uint32_t(i) : P_OOR;
      __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{uint32_t(lo), uint32_t(lo >> 32), uint32_t(hi), uint32_t(hi >> 32)},
                                             t_rsrc, int(toff), 0, 0);
      tc_start = clock64();
      tw_start = wall_clock64();
    }
    lds_barrier();  // every wave read its staged rows: the next tile may copy into that slot
    if (!has_next) break;
    r0 = (r0 + KT) & 3;
    q += W;
    cur = nxt;
    cc = nc;
    has_next = has_next2;
    nxt = nxt2;
  }
}

// The up-projection's 256-row tiles with the persistent kernel above: one workgroup per CU (a multiple of 8, so
// that workgroup i runs on XCD i % 8).  Requires bf16 [in, out] weights, K = d a multiple of 64 (whole step pairs)
// with at least 8 K steps, and x and h below 2^31 bytes (checked here).
hipError_t launch_up_persist(const uint16_t* x, const void* w1, const void* wv, const int32_t* counts,
                             const int32_t* perm, int d, int f, int E, int slots, uint16_t* h, hipStream_t s) {
  int dev = 0, cus = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return err;
  const int wg = (cus / 8) * 8;
  if (wg < 8 || d % (2 * PBK) != 0 || d / PBK < 8) return hipErrorInvalidValue;
  const size_t xbytes = size_t(slots / 2) * d * 2, hbytes = size_t(slots) * f * 2;
  if (xbytes >= (size_t(1) << 31) || hbytes >= (size_t(1) << 31)) return hipErrorInvalidValue;
  tiled_up_persist_kernel<false><<<dim3(wg), dim3(256), 0, s>>>(x, static_cast<const uint16_t*>(w1),
                                                               static_cast<const uint16_t*>(wv), counts, perm,
                                                               uint32_t(xbytes), d, f, E, h, uint32_t(hbytes),
                                                               nullptr, 0u);
  return hipGetLastError();
}

}  // namespace gm
