// Device-side helpers shared by the gfx950 kernels of the Grok-1 MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

namespace gm {

// bf16 bit pattern (low or high half of a dword) -> float, exact.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// float -> bf16 bit pattern, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t f2bf(float v) {
  uint32_t u = __float_as_uint(v);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// GELU in the exact (erf) form, 0.5 z (1 + erf(z / sqrt 2)), with erf evaluated by Abramowitz & Stegun,
// Handbook of Mathematical Functions, formula 7.1.26 (|error of erf| <= 1.5e-7, far below the bf16 rounding of
// h): erf(a) = 1 - P(t) exp(-a^2), P(t) = a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5, t = 1 / (1 + p a), for a >= 0,
// extended by odd symmetry.  With a = |z| / sqrt 2 that gives GELU(z) = max(z, 0) - 0.5 |z| P(t) exp(-a^2) for
// either sign of z (for z < 0 this avoids the cancellation of 1 + erf(z / sqrt 2)).  Branch-free.
__device__ __forceinline__ float gelu_erf(float z) {
  const float az = fabsf(z);
  const float a = az * 0.70710678118654752440f;
  const float t = __builtin_amdgcn_rcpf(__fmaf_rn(0.3275911f, a, 1.0f));
  float poly = __fmaf_rn(1.061405429f, t, -1.453152027f);
  poly = __fmaf_rn(poly, t, 1.421413741f);
  poly = __fmaf_rn(poly, t, -0.284496736f);
  poly = __fmaf_rn(poly, t, 0.254829592f);
  poly *= t;
  const float pe = poly * __expf(-a * a);
  return __fmaf_rn(-0.5f * az, pe, fmaxf(z, 0.0f));
}

// Two floats -> two bf16 (round to nearest, ties to even, as f2bf for finite values; one v_cvt_pk_bf16_f32), lo
// in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}

// One gfx950 bf16 MFMA, 16x16 output, K = 32 (8 bf16 per lane in each operand).
// Lane l: A row (l & 15), k = 8 (l >> 4) .. +7; B column (l & 15), same k; D column (l & 15),
// rows 4 (l >> 4) .. +3.
__device__ __forceinline__ f32x4_t mfma16x16x32(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}

// One gfx950 bf16 MFMA, 32x32 output, K = 16.
// Lane l: A row (l & 31), k = 8 (l >> 5) .. +7; B column (l & 31), same k;
// D column (l & 31), element v at row (v & 3) + 8 (v >> 2) + 4 (l >> 5).
__device__ __forceinline__ f32x16_t mfma32x32x16(const u32x4_t& a, const u32x4_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}

// Register transpose of an 8x8 block of bf16.  r[i] holds row i (8 consecutive columns, two per dword).
// Returns in t[c] column c: its 8 row values, rows 2q and 2q+1 in dword q (low, high).
__device__ __forceinline__ void transpose8x8_bf16(const u32x4_t r[8], u32x4_t t[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int q = 0; q < 4; ++q) t[c][q] = __builtin_amdgcn_perm(r[2 * q + 1][c >> 1], r[2 * q][c >> 1], sel);
  }
}

// Same for int8 rows: r[i] holds row i as 8 int8 (one per byte, column c in byte c).  Converts every value to
// bf16 exactly (|q| <= 128 has at most 8 significant bits) and returns column-major bf16 pairs as above.
__device__ __forceinline__ void transpose8x8_i8_to_bf16(const u32x2_t r[8], u32x4_t t[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t w0 = r[2 * q][c >> 2], w1 = r[2 * q + 1][c >> 2];
      const float v0 = float(int32_t(w0 << (24 - 8 * (c & 3))) >> 24);
      const float v1 = float(int32_t(w1 << (24 - 8 * (c & 3))) >> 24);
      t[c][q] = __builtin_amdgcn_perm(__float_as_uint(v1), __float_as_uint(v0), 0x07060302u);
    }
  }
}

// 8 int8 values (byte i of the pair = element i) -> 8 bf16, exactly, two per dword (element 2q in the low half
// of dword q).
__device__ __forceinline__ u32x4_t i8x8_to_bf16(const u32x2_t& v) {
  u32x4_t t;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t w = v[q >> 1];
    const int b0 = 2 * (q & 1);
    const float f0 = float(int32_t(w << (24 - 8 * b0)) >> 24);
    const float f1 = float(int32_t(w << (16 - 8 * b0)) >> 24);
    t[q] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
  }
  return t;
}

}  // namespace gm
