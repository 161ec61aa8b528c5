// Expert matrix products of the Grok-1 MoE layer for few tokens per expert (decode-sized batches), gfx950.
//
// Expert FFN, page "A functional bridge between openai/grok and xai-org/grok-1" (architecture diagram):
// y = (GELU(x W1) (*) (x Wv)) W2.  int8 weights times bf16 scales broadcast over groups of input rows, page
// "Grok-1-BF16", section "Conversion Details".
//
// With at most a few dozen tokens per expert the products are bound by streaming the weights from HBM: every
// weight is used by at most 2 * 16 tokens.  So the weights go straight from HBM into registers, without LDS
// staging.  Each lane loads an 8 (k) x 8 (n) block as eight 16-byte row pieces (8-byte for int8), transposes
// it in registers (v_perm_b32; int8 values are converted to bf16 exactly on the way) so that it holds 8 k
// values for each of 8 columns, and feeds 8 MFMAs 16x16x32 against the same A fragment (16 token rows).
// Lane l covers columns n0 + 8 (l & 15) .. +7 and k rows 8 (l >> 4) .. +7 of each 32-deep step, so a wave
// owns 128 columns; the four 16-lane groups read four different row blocks of 256 contiguous bytes.
//
// Weights stored [E, out, in] (OUTIN; the PyTorch layout of "Grok-1-BF16", section "Conversion Details") need no
// transpose: each of the lane's 8 columns is a row of the stored matrix, whose 8 consecutive k are one 16-byte
// (int8: 8-byte) load, already the MFMA operand (int8 converted to bf16).  For one column the four 16-lane
// groups read 64 contiguous bytes of the row; the next 32-deep step reads the next 64.
//
// Up-projection: one wave per 128 columns of both W1 and Wv over the whole d axis (GELU needs the full sum; for bf16
// 16-row tiles with enough experts hit, up_stream_narrow_kernel below takes 64 columns per wave);
// h = bf16(GELU(a) * b) is written for the valid token rows.  Down-projection: one wave per 128 columns of W2
// over one of S chunks of the f axis; fp32 partial sums go to y[S, slots, d] and are added by the combine.
//
// The int8 [in, out] down-projection with one scale group stages its weights in LDS instead
// (expert_stream_lds.hip).
//
// int8 scales: with one group along the input axis the scale multiplies the fp32 accumulator once, in the
// epilogue.  With several groups (GROUPED) the accumulator is kept in units of the current group's scale: on
// entering group g it is multiplied by s[g-1]/s[g] for each column, the MFMAs then add that group's integer
// products, and the epilogue multiplies by the last group's scale, so that the result is sum_g s[g] * P[g].
// A zero scale is replaced by one and that group's int8 values of the column are masked to zero, which gives
// the same sum.  This costs one rounding per group boundary, far below the bf16 rounding of h.
#include "chunks.h"
#include "common.h"
#include "launch.h"

namespace gm {

// Weight rows are read once per launch: nontemporal loads (low cache retention) stream them faster from HBM.
template <bool INT8> struct WRow;
template <> struct WRow<false> {  // bf16: 16 bytes = 8 columns
  typedef u32x4_t T;
  static __device__ __forceinline__ T load(const void* base, size_t i) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(base) + i));
  }
  static __device__ __forceinline__ void transpose(const T r[8], u32x4_t t[8]) { transpose8x8_bf16(r, t); }
};
template <> struct WRow<true> {  // int8: 8 bytes = 8 columns
  typedef u32x2_t T;
  static __device__ __forceinline__ T load(const void* base, size_t i) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(static_cast<const int8_t*>(base) + i));
  }
  static __device__ __forceinline__ void transpose(const T r[8], u32x4_t t[8]) { transpose8x8_i8_to_bf16(r, t); }
};

// 8 scales (bf16) of consecutive columns -> float.
__device__ __forceinline__ void unpack_scales8(const u32x4_t& w, float o[8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) { o[2 * j] = bf16lo(w[j]); o[2 * j + 1] = bf16hi(w[j]); }
}
__device__ __forceinline__ u32x4_t load_raw8(const uint16_t* s) { return *reinterpret_cast<const u32x4_t*>(s); }
__device__ __forceinline__ void load_scales8(const uint16_t* s, float o[8]) { unpack_scales8(load_raw8(s), o); }

template <bool INT8, int MT>
struct UpStep {
  typename WRow<INT8>::T b1[8], b2[8];
  u32x4_t a[MT];
};

// Scales of a group for the 8 columns of a lane: the values with zero replaced by one, and a byte mask (per
// int8 column of a row piece) that keeps the columns whose scale is not zero.
__device__ __forceinline__ void group_scales8(const u32x4_t& raw, float o[8], u32x2_t& mask) {
  unpack_scales8(raw, o);
  mask = u32x2_t{0u, 0u};
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    if (__float_as_uint(o[c]) & 0x7fffffffu) mask[c >> 2] |= 0xffu << (8 * (c & 3));
    else o[c] = 1.0f;
  }
}

// The lane's weight block as 8 MFMA operands t[c] (8 consecutive k of column c), its int8 columns masked by
// the byte mask m (byte c for column c) if MASKED.  [in, out] storage: r[i] is row i (8 columns) and is
// transposed; [out, in] storage (OUTIN): r[c] is column c (8 k) and is only converted.
template <bool INT8, bool MASKED, bool OUTIN>
__device__ __forceinline__ void block_operands(const typename WRow<INT8>::T r[8], const u32x2_t& m, u32x4_t t[8]) {
  if constexpr (OUTIN) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      if constexpr (INT8) {
        u32x2_t v = r[c];
        if constexpr (MASKED) {
          const uint32_t keep = ((m[c >> 2] >> (8 * (c & 3))) & 0xffu) ? ~0u : 0u;
          v &= u32x2_t{keep, keep};
        }
        t[c] = i8x8_to_bf16(v);
      } else {
        t[c] = r[c];
      }
    }
  } else if constexpr (MASKED) {
    typename WRow<INT8>::T b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = r[i] & m;
    WRow<INT8>::transpose(b, t);
  } else {
    WRow<INT8>::transpose(r, t);
  }
}

// KS = 4 (small f: fewer workgroups than CUs): the 4 waves of a workgroup take the same 128 columns and one
// quarter of the d axis each; the partial sums meet in LDS and are added in ascending quarter order before the
// GELU product (the [out, in] kernel adds the same quarters in the same order).
template <bool INT8, int MT, bool GROUPED, bool OUTIN, int KS = 1>
__global__ __launch_bounds__(256) void up_stream_kernel(const uint16_t* __restrict__ x, const void* __restrict__ w1,
                                                        const void* __restrict__ wv, const uint16_t* __restrict__ s1,
                                                        const uint16_t* __restrict__ sv, ScaleLayout sl,
                                                        const int32_t* __restrict__ counts,
                                                        const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ perm, int d, int f,
                                                        uint16_t* __restrict__ h) {
  static_assert(INT8 || !GROUPED, "grouped scales belong to int8 weights");
  static_assert(KS == 1 || KS == 4, "the d axis is whole or split in 4");
  typedef WRow<INT8> W;
  const int e = blockIdx.y;
  const int n_e = counts[e];
  if (n_e == 0) return;
  const int off = offsets[e];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const int n0 = KS == 1 ? (blockIdx.x * 4 + wave) * 128 : blockIdx.x * 128;
  if (n0 >= f) return;  // KS = 1: no workgroup barrier in this kernel; KS = 4: the whole workgroup
  const int klo = KS == 1 ? 0 : wave * (d / KS), khi = KS == 1 ? d : klo + d / KS;  // this wave's part of d
  __shared__ f32x4_t red[KS == 1 ? 1 : 3][2][MT][8][64];  // KS = 4: partial sums of waves 1..3
  __shared__ float redc[KS > 1 && GROUPED ? 3 : 1][2][8][64];  // ... and their units (grouped scales)
  const int col = n0 + 8 * c16;
  const size_t ebase = size_t(e) * d * f;
  // [in, out]: row 8g of each 32-deep step, column col; [out, in]: row col, k 8g of each step
  const size_t lane_base = OUTIN ? ebase + size_t(col) * d + 8 * g : ebase + size_t(8 * g) * f + col;
  const uint16_t* s1e = INT8 ? s1 + size_t(e) * sl.estride + col : nullptr;  // group 0's scales of the lane
  const uint16_t* sve = INT8 ? sv + size_t(e) * sl.estride + col : nullptr;

  for (int mb = 0; mb < n_e; mb += 16 * MT) {
    const uint16_t* arow[MT];
    bool aval[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mb + mt * 16 + c16;
      aval[mt] = m < n_e;
      arow[mt] = x + size_t(aval[mt] ? perm[off + m] : 0) * d + 8 * g;
    }
    f32x4_t acc1[MT][8], acc2[MT][8];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int c = 0; c < 8; ++c) { acc1[mt][c] = f32x4_t{0, 0, 0, 0}; acc2[mt][c] = f32x4_t{0, 0, 0, 0}; }

    auto load = [&](UpStep<INT8, MT>& st, int k0) {
      const size_t rb = lane_base + (OUTIN ? size_t(k0) : size_t(k0) * f);
      const size_t rs = OUTIN ? size_t(d) : size_t(f);  // between the 8 rows (columns for OUTIN) of the block
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        st.b1[r] = W::load(w1, rb + size_t(r) * rs);
        st.b2[r] = W::load(wv, rb + size_t(r) * rs);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)  // rows past the expert's end read its first row; they are never stored
        st.a[mt] = *reinterpret_cast<const u32x4_t*>(arow[mt] + k0);
    };
    // GROUPED: the current group's scales (zero replaced by one), the byte masks of its columns with a non-zero
    // scale, and the raw scales of the next group (loaded a group ahead)
    float cur1[8], curv[8];
    u32x2_t m1, mv;
    u32x4_t pend1, pendv;
    auto enter_group = [&](bool rescale) {
      float n1[8], nv[8];
      group_scales8(pend1, n1, m1);
      group_scales8(pendv, nv, mv);
      if (rescale) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const float r1 = cur1[c] / n1[c], rv = curv[c] / nv[c];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) { acc1[mt][c] *= r1; acc2[mt][c] *= rv; }
        }
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) { cur1[c] = n1[c]; curv[c] = nv[c]; }
    };
    auto compute = [&](const UpStep<INT8, MT>& st) {
      u32x4_t t[8];
      block_operands<INT8, GROUPED, OUTIN>(st.b1, m1, t);
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc1[mt][c] = mfma16x16x32(st.a[mt], t[c], acc1[mt][c]);
      block_operands<INT8, GROUPED, OUTIN>(st.b2, mv, t);
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc2[mt][c] = mfma16x16x32(st.a[mt], t[c], acc2[mt][c]);
    };

    // d is a multiple of 64: two 32-deep steps per iteration, the next step's loads in flight during compute.
    UpStep<INT8, MT> sa, sb;
    auto steps = [&](int k_lo, int k_hi) {
      for (int k0 = k_lo; k0 < k_hi; k0 += 64) {
        load(sb, k0 + 32);
        // int8 with 32-row tiles: keep each step's loads (activation rows included) ahead of the other step's
        // MFMAs; left to itself the scheduler sinks the activation loads to their first use and then waits for
        // every load in flight (measured: T = 64 up-projection 0.473 -> 0.469 ms; the same barrier in the bf16
        // and 16-row forms was slower)
        if constexpr (INT8 && MT == 2) __builtin_amdgcn_sched_barrier(0);
        compute(sa);
        // past the end the last step is loaded again and not used: no branch around the loads, whose join
        // would make the compiler wait for every load in flight
        load(sa, min(k0 + 64, khi - 32));
        if constexpr (INT8 && MT == 2) __builtin_amdgcn_sched_barrier(0);
        compute(sb);
      }
    };
    load(sa, klo);
    if constexpr (GROUPED && KS == 1) {
      // group boundaries are multiples of 64 rows: each group is a whole number of iterations
      const int ng = d / sl.gsize;
      pend1 = load_raw8(s1e);
      pendv = load_raw8(sve);
      for (int gi = 0; gi < ng; ++gi) {
        enter_group(gi > 0);
        if (gi + 1 < ng) {
          pend1 = load_raw8(s1e + size_t(gi + 1) * f);
          pendv = load_raw8(sve + size_t(gi + 1) * f);
        }
        steps(gi * sl.gsize, (gi + 1) * sl.gsize);
      }
    } else if constexpr (GROUPED) {  // the groups that meet this wave's quarter [klo, khi)
      const int g0 = klo / sl.gsize, g1 = (khi - 1) / sl.gsize;
      pend1 = load_raw8(s1e + size_t(g0) * f);
      pendv = load_raw8(sve + size_t(g0) * f);
      for (int gi = g0; gi <= g1; ++gi) {
        enter_group(gi > g0);
        if (gi < g1) {
          pend1 = load_raw8(s1e + size_t(gi + 1) * f);
          pendv = load_raw8(sve + size_t(gi + 1) * f);
        }
        steps(max(klo, gi * sl.gsize), min(khi, (gi + 1) * sl.gsize));
      }
    } else {
      steps(klo, khi);
    }
    if constexpr (KS > 1) {  // quarters 1..3 to LDS; wave 0 adds them in order and writes h
      if (wave > 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            red[wave - 1][0][mt][c][lane] = acc1[mt][c];
            red[wave - 1][1][mt][c][lane] = acc2[mt][c];
          }
        if constexpr (GROUPED) {
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            redc[wave - 1][0][c][lane] = cur1[c];
            redc[wave - 1][1][c][lane] = curv[c];
          }
        }
      }
      __syncthreads();
      if (wave == 0) {
        if constexpr (GROUPED) {
          // each quarter's sum is in units of its last group's scale: bring quarters 0..2 to the unit u of
          // quarter 3, t = fma(q2, c2 / u, fma(q1, c1 / u, q0 * (c0 / u))) + q3, in that unit from here on
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const float u1 = redc[2][0][c][lane], uv = redc[2][1][c][lane];
            const float r1[3] = {cur1[c] / u1, redc[0][0][c][lane] / u1, redc[1][0][c][lane] / u1};
            const float rv[3] = {curv[c] / uv, redc[0][1][c][lane] / uv, redc[1][1][c][lane] / uv};
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                float t1 = acc1[mt][c][v] * r1[0], tv = acc2[mt][c][v] * rv[0];
                t1 = __builtin_fmaf(red[0][0][mt][c][lane][v], r1[1], t1);
                tv = __builtin_fmaf(red[0][1][mt][c][lane][v], rv[1], tv);
                t1 = __builtin_fmaf(red[1][0][mt][c][lane][v], r1[2], t1);
                tv = __builtin_fmaf(red[1][1][mt][c][lane][v], rv[2], tv);
                acc1[mt][c][v] = t1 + red[2][0][mt][c][lane][v];
                acc2[mt][c][v] = tv + red[2][1][mt][c][lane][v];
              }
            cur1[c] = u1;
            curv[c] = uv;
          }
        } else {
#pragma unroll
          for (int q = 0; q < KS - 1; ++q)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
              for (int c = 0; c < 8; ++c) {
                acc1[mt][c] += red[q][0][mt][c][lane];
                acc2[mt][c] += red[q][1][mt][c][lane];
              }
        }
      }
      __syncthreads();  // the next pass may overwrite red
      if (wave != 0) continue;
    }

    float sc1[8], scv[8];
    if (GROUPED) {  // the accumulators are in units of the last group's scale
#pragma unroll
      for (int c = 0; c < 8; ++c) { sc1[c] = cur1[c]; scv[c] = curv[c]; }
    } else if (INT8) {
      load_scales8(s1e, sc1);
      load_scales8(sve, scv);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = mb + mt * 16 + 4 * g + v;
        if (m < n_e) {
          float hv[8];
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            float a = acc1[mt][c][v], b = acc2[mt][c][v];
            if (INT8) { a *= sc1[c]; b *= scv[c]; }
            hv[c] = gelu_erf(a) * b;
          }
          u32x4_t o;
#pragma unroll
          for (int j = 0; j < 4; ++j) o[j] = pack_bf16(hv[2 * j], hv[2 * j + 1]);
          *reinterpret_cast<u32x4_t*>(h + size_t(off + m) * f + col) = o;
        }
      }
    }
  }
}

template <bool INT8, int MT>
struct DownStep {
  typename WRow<INT8>::T b[8];
  u32x4_t a[MT];
};

template <bool INT8, int MT, bool GROUPED, bool OUTIN>
__global__ __launch_bounds__(256) void down_stream_kernel(const uint16_t* __restrict__ h, const void* __restrict__ w2,
                                                          const uint16_t* __restrict__ s2, ScaleLayout sl,
                                                          const int32_t* __restrict__ counts,
                                                          const int32_t* __restrict__ offsets, int d, int f, int S,
                                                          int64_t split_stride, float* __restrict__ y) {
  static_assert(INT8 || !GROUPED, "grouped scales belong to int8 weights");
  typedef WRow<INT8> W;
  const int e = blockIdx.z;
  const int n_e = counts[e];
  if (n_e == 0) return;
  const int off = offsets[e];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const int n0 = (blockIdx.x * 4 + wave) * 128;
  if (n0 >= d) return;
  const int col = n0 + 8 * c16;
  const int kbeg = down_chunk_begin(blockIdx.y, f, S), kend = down_chunk_begin(blockIdx.y + 1, f, S);
  // [in, out]: row 8g of each 32-deep step, column col; [out, in]: row col, k 8g of each step
  const size_t ebase = size_t(e) * f * d;
  const size_t lane_base = OUTIN ? ebase + size_t(col) * f + 8 * g : ebase + size_t(8 * g) * d + col;
  const uint16_t* s2e = INT8 ? s2 + size_t(e) * sl.estride + col : nullptr;  // group 0's scales of the lane

  for (int mb = 0; mb < n_e; mb += 16 * MT) {
    const uint16_t* arow[MT];
    bool aval[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mb + mt * 16 + c16;
      aval[mt] = m < n_e;
      arow[mt] = h + size_t(off + (aval[mt] ? m : 0)) * f + 8 * g;
    }
    f32x4_t acc[MT][8];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[mt][c] = f32x4_t{0, 0, 0, 0};

    auto load = [&](DownStep<INT8, MT>& st, int k0) {
      const size_t rb = lane_base + (OUTIN ? size_t(k0) : size_t(k0) * d);
      const size_t rs = OUTIN ? size_t(f) : size_t(d);
#pragma unroll
      for (int r = 0; r < 8; ++r) st.b[r] = W::load(w2, rb + size_t(r) * rs);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)  // rows past the expert's end read its first row; they are never stored
        st.a[mt] = *reinterpret_cast<const u32x4_t*>(arow[mt] + k0);
    };
    // GROUPED: the current group's scales (zero replaced by one), the byte mask of its columns with a non-zero
    // scale, and the raw scales of the next group (loaded a group ahead)
    float cur[8];
    u32x2_t msk;
    u32x4_t pend;
    auto enter_group = [&](bool rescale) {
      float ns[8];
      group_scales8(pend, ns, msk);
      if (rescale) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const float r = cur[c] / ns[c];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[mt][c] *= r;
        }
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) cur[c] = ns[c];
    };
    auto compute = [&](const DownStep<INT8, MT>& st) {
      u32x4_t t[8];
      block_operands<INT8, GROUPED, OUTIN>(st.b, msk, t);
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt][c] = mfma16x16x32(st.a[mt], t[c], acc[mt][c]);
    };

    DownStep<INT8, MT> sa, sb;
    auto steps = [&](int klo, int khi) {
      for (int k0 = klo; k0 < khi; k0 += 64) {
        load(sb, k0 + 32);
        compute(sa);
        load(sa, min(k0 + 64, kend - 32));  // unused past the end: no branch, as in up_stream_kernel
        compute(sb);
      }
    };
    load(sa, kbeg);
    if constexpr (GROUPED) {
      // the chunk [kbeg, kend) meets groups g0 .. g1 (boundaries are multiples of 64 rows)
      const int g0 = kbeg / sl.gsize, g1 = (kend - 1) / sl.gsize;
      pend = load_raw8(s2e + size_t(g0) * d);
      for (int gi = g0; gi <= g1; ++gi) {
        enter_group(gi > g0);
        if (gi < g1) pend = load_raw8(s2e + size_t(gi + 1) * d);
        steps(max(kbeg, gi * sl.gsize), min(kend, (gi + 1) * sl.gsize));
      }
    } else {
      steps(kbeg, kend);
    }

    float sc[8];
    if (GROUPED) {  // the accumulators are in units of the chunk's last group's scale
#pragma unroll
      for (int c = 0; c < 8; ++c) sc[c] = cur[c];
    } else if (INT8) {
      load_scales8(s2e, sc);
    }
    float* ys = y + int64_t(blockIdx.y) * split_stride;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = mb + mt * 16 + 4 * g + v;
        if (m < n_e) {
          f32x4_t o0, o1;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            o0[c] = INT8 ? acc[mt][c][v] * sc[c] : acc[mt][c][v];
            o1[c] = INT8 ? acc[mt][c + 4][v] * sc[c + 4] : acc[mt][c + 4][v];
          }
          float* dst = ys + size_t(off + m) * d + col;
          *reinterpret_cast<f32x4_t*>(dst) = o0;
          *reinterpret_cast<f32x4_t*>(dst + 4) = o1;
        }
      }
    }
  }
}

// bf16 [in, out] up-projection for 16-row token tiles with 64 columns per wave: lane l covers columns
// n0 + 4 (l & 15) .. +3 and k rows 8 (l >> 4) .. +7 of each 32-deep step as 8-byte row pieces (a wave reads
// 128-byte strips of each weight row), transposed in registers into 4 MFMA operands.  Half the accumulators of
// up_stream_kernel, so two waves fit per SIMD.  With enough experts hit to fill the chip this streams the weights
// faster (measured on MI355X at T = 8, Grok-1 shape: 6.8 -> 7.2 TB/s); with a few experts the 16-byte pieces
// of up_stream_kernel keep more bytes in flight per wave and win.  Each output element is the same MFMA over the
// same k in the same order as in up_stream_kernel: the results are bit-identical.
__global__ __launch_bounds__(256, 2) void up_stream_narrow_kernel(const uint16_t* __restrict__ x,
                                                                  const uint16_t* __restrict__ w1,
                                                                  const uint16_t* __restrict__ wv,
                                                                  const int32_t* __restrict__ counts,
                                                                  const int32_t* __restrict__ offsets,
                                                                  const int32_t* __restrict__ perm, int d, int f,
                                                                  uint16_t* __restrict__ h) {
  const int e = blockIdx.y;
  const int n_e = counts[e];
  if (n_e == 0) return;
  const int off = offsets[e];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const int n0 = (blockIdx.x * 4 + wave) * 64;
  if (n0 >= f) return;  // no workgroup barrier in this kernel
  const int col = n0 + 4 * c16;
  const size_t lane_base = size_t(e) * d * f + size_t(8 * g) * f + col;
  struct Step {
    u32x2_t b1[8], b2[8];
    u32x4_t a;
  };
  // 8 rows of 4 bf16 columns -> 4 operands (column c: its 8 k values, two per dword)
  auto transpose = [](const u32x2_t r[8], u32x4_t t[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
      for (int q = 0; q < 4; ++q) t[c][q] = __builtin_amdgcn_perm(r[2 * q + 1][c >> 1], r[2 * q][c >> 1], sel);
    }
  };
  for (int mb = 0; mb < n_e; mb += 16) {
    const int m = mb + c16;
    const bool aval = m < n_e;
    const uint16_t* arow = x + size_t(aval ? perm[off + m] : 0) * d + 8 * g;
    f32x4_t acc1[4], acc2[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      acc1[c] = f32x4_t{0, 0, 0, 0};
      acc2[c] = f32x4_t{0, 0, 0, 0};
    }
    auto load = [&](Step& st, int k0) {
      const size_t rb = lane_base + size_t(k0) * f;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        st.b1[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(w1 + rb + size_t(r) * f));
        st.b2[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(wv + rb + size_t(r) * f));
      }
      st.a = *reinterpret_cast<const u32x4_t*>(arow + k0);  // past the expert's end: its first row, not stored
    };
    auto compute = [&](const Step& st) {
      u32x4_t t[4];
      transpose(st.b1, t);
#pragma unroll
      for (int c = 0; c < 4; ++c) acc1[c] = mfma16x16x32(st.a, t[c], acc1[c]);
      transpose(st.b2, t);
#pragma unroll
      for (int c = 0; c < 4; ++c) acc2[c] = mfma16x16x32(st.a, t[c], acc2[c]);
    };
    // d is a multiple of 64: two 32-deep steps per iteration, the next step's loads in flight during compute
    Step sa, sb;
    load(sa, 0);
    for (int k0 = 0; k0 < d; k0 += 64) {
      load(sb, k0 + 32);
      compute(sa);
      load(sa, min(k0 + 64, d - 32));  // unused past the end: no branch, as in up_stream_kernel
      compute(sb);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = mb + 4 * g + v;
      if (r < n_e) {
        u32x2_t o;
#pragma unroll
        for (int j = 0; j < 2; ++j)
          o[j] = pack_bf16(gelu_erf(acc1[2 * j][v]) * acc2[2 * j][v], gelu_erf(acc1[2 * j + 1][v]) * acc2[2 * j + 1][v]);
        *reinterpret_cast<u32x2_t*>(h + size_t(off + r) * f + col) = o;
      }
    }
  }
}

// The up-projection's split of the d axis over the 4 waves of a workgroup (KS = 4) when its grid of one workgroup
// per 512 columns and expert would leave CUs idle (a layer's share of d_ff on one of several GPUs; measured at
// f = 4096: 64 workgroups, 3.3 TB/s).  d / 4 a multiple of 128 (the stages of the [out, in] kernel, which splits
// the same way).  With grouped int8 scales the quarter sums are brought to one unit by exact-order fused
// multiply-adds whose ratios are 1 when every group has the same scale, so such a layer keeps the bits of the
// per-channel form.
int up_stream_ksplit(int d, int f, int E) {
  return (d % 512 == 0 && ((f + 511) / 512) * E < 256) ? 4 : 1;
}

// The 64-column bf16 kernel: [in, out] weights, 16-row token tiles, the whole d axis per wave, and enough experts
// that can be hit for min(slots, E) * f / 256 >= 1024 workgroups (at Grok-1 shape: four or more tokens; measured
// up-projection ms, up_stream_kernel -> this kernel: T = 1 0.28 -> 0.28 (not taken), T = 2 0.36 -> 0.39, T = 4
// 0.48 -> 0.45, T = 8 0.95 -> 0.90, T = 16 0.95 -> 0.90).
bool up_stream_narrow(int d, int f, int E, int slots, bool int8, bool outin, int mt) {
  return !int8 && !outin && mt == 1 && f % 256 == 0 && up_stream_ksplit(d, f, E) == 1 &&
         int64_t(slots < E ? slots : E) * (f / 256) >= 1024;
}

hipError_t launch_up_stream(const uint16_t* x, const void* w1, const void* wv, const uint16_t* s1,
                            const uint16_t* sv, ScaleLayout sl, bool outin, const int32_t* counts,
                            const int32_t* offsets, const int32_t* perm, int d, int f, int E, int slots, bool int8,
                            int mt, uint16_t* h, hipStream_t s) {
  const dim3 grid((f + 511) / 512, E), block(256);
  const bool grouped = int8 && sl.gsize < d;
  if (up_stream_narrow(d, f, E, slots, int8, outin, mt)) {
    up_stream_narrow_kernel<<<dim3(f / 256, E), block, 0, s>>>(x, static_cast<const uint16_t*>(w1),
                                                               static_cast<const uint16_t*>(wv), counts, offsets,
                                                               perm, d, f, h);
    return hipGetLastError();
  }
  if (up_stream_ksplit(d, f, E) == 4) {
    const dim3 grid4((f + 127) / 128, E);
#define GM_UP4(I8, MT, GR, OI) up_stream_kernel<I8, MT, GR, OI, 4><<<grid4, block, 0, s>>>(x, w1, wv, s1, sv, sl, \
                                                                                        counts, offsets, perm, d, f, h)
#define GM_UP4_MT(I8, GR, OI) do { if (mt == 1) GM_UP4(I8, 1, GR, OI); else GM_UP4(I8, 2, GR, OI); } while (0)
#define GM_UP4_L(I8, GR) do { if (outin) GM_UP4_MT(I8, GR, true); else GM_UP4_MT(I8, GR, false); } while (0)
    if (grouped) GM_UP4_L(true, true);
    else if (int8) GM_UP4_L(true, false);
    else GM_UP4_L(false, false);
#undef GM_UP4_L
#undef GM_UP4_MT
#undef GM_UP4
    return hipGetLastError();
  }
#define GM_UP(I8, MT, GR, OI) up_stream_kernel<I8, MT, GR, OI><<<grid, block, 0, s>>>(x, w1, wv, s1, sv, sl, counts, \
                                                                                  offsets, perm, d, f, h)
#define GM_UP_MT(I8, GR, OI) do { if (mt == 1) GM_UP(I8, 1, GR, OI); else GM_UP(I8, 2, GR, OI); } while (0)
#define GM_UP_L(I8, GR) do { if (outin) GM_UP_MT(I8, GR, true); else GM_UP_MT(I8, GR, false); } while (0)
  if (grouped) GM_UP_L(true, true);
  else if (int8) GM_UP_L(true, false);
  else GM_UP_L(false, false);
#undef GM_UP_L
#undef GM_UP_MT
#undef GM_UP
  return hipGetLastError();
}

hipError_t launch_down_stream(const uint16_t* h, const void* w2, const uint16_t* s2, ScaleLayout sl, bool outin,
                              const int32_t* counts, const int32_t* offsets, int d, int f, int E, int slots, int S,
                              bool int8, int mt, float* y, hipStream_t s) {
  const dim3 grid((d + 511) / 512, S, E), block(256);
  const int64_t stride = int64_t(slots) * d;
  const bool grouped = int8 && sl.gsize < f;
  if (int8 && !grouped && !outin)  // LDS-staged weights (expert_stream_lds.hip)
    return launch_down_stream_lds(h, w2, s2, sl.estride, counts, offsets, d, f, E, slots, S, mt, y, s);
#define GM_DOWN(I8, MT, GR, OI) down_stream_kernel<I8, MT, GR, OI><<<grid, block, 0, s>>>(h, w2, s2, sl, counts, \
                                                                                      offsets, d, f, S, stride, y)
#define GM_DOWN_MT(I8, GR, OI) do { if (mt == 1) GM_DOWN(I8, 1, GR, OI); else GM_DOWN(I8, 2, GR, OI); } while (0)
#define GM_DOWN_L(I8, GR) do { if (outin) GM_DOWN_MT(I8, GR, true); else GM_DOWN_MT(I8, GR, false); } while (0)
  if (grouped) GM_DOWN_L(true, true);
  else if (int8) GM_DOWN_L(true, false);
  else GM_DOWN_L(false, false);
#undef GM_DOWN_L
#undef GM_DOWN_MT
#undef GM_DOWN
  return hipGetLastError();
}

}  // namespace gm
