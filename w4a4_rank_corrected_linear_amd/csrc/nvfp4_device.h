// NVFP4 device helpers shared by the activation quantizer and the weight preparation:
// E4M3 scale codes, E2M1 codes and the quantizer of two 16-value blocks.
#pragma once
#include "common.h"

namespace svdq {

// E4M3 (FN) code of a non-negative float32, round to nearest even, saturating at 448
// (code 0x7E).  Normal range: round the fp32 significand to 3 bits; below 2^-6 the
// grid step is 2^-9, so the code is rne(v * 2^9) (8 lands on the smallest normal,
// code 0x08).  Branch-free: both roundings are computed and one is selected.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t sub = (uint32_t)__builtin_rintf(fminf(v, 0x1p-6f) * 512.0f);
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFFu + ((u >> 20) & 1u);
  const int e = (int)(u >> 23) - 127 + 7;
  const uint32_t nrm = (uint32_t)min(max((e << 3) | (int)((u >> 20) & 7u), 0), 0x7E);
  return !(v < 448.0f) ? 0x7Eu : (v < 0x1p-6f ? sub : nrm);
}

// Value of an E4M3 code (0..0x7E, non-negative).
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = c >> 3, m = c & 7u;
  const float sub = (float)m * 0x1p-9f;
  const float nrm = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return e == 0 ? sub : nrm;
}

// Twice the E2M1 magnitude of code mag (0, 1, 2, 3, 4, 6, 8, 12), from a nibble table.
__device__ __forceinline__ uint32_t e2m1_twice(uint32_t mag) {
  return __builtin_amdgcn_ubfe(0xC8643210u, 4 * mag, 4);
}

// Codes, dequantized values and the two block scales of the lane's 32 values.
//
// The quotient xhat / d of a block shares one divisor d = fl32(s g) > 0.  With
// r = RN(1/d) (one correctly rounded division per block), y = RN(xhat r) is within an
// ulp of xhat / d, the remainder e = xhat - y d is exact (fma), and RN(y + e r) is the
// correctly rounded quotient (Markstein's theorem for division by fma), ties included.
// The sign is xhat's own (d > 0; -0 stays -0).  The theorem needs d and the quotients
// inside the normal range: a block with d < 2^-100 or amax r > 2^100 (never produced by
// sane scales) makes the wave take the IEEE division instead, tested once per wave.
// The dequantized value e2m1 * s is (2 e2m1) * (s / 2), exact in fp32 and in bf16.
// Block scale codes sc, scales s, divisors d = fl32(s g) and reciprocals r of the lane's
// two blocks; true when a block leaves the range of the fma division (see above).
__device__ __forceinline__ bool nvfp4_block_scales(const float (&xh)[32], float g, float (&s)[2],
                                                   float (&d)[2], float (&r)[2], uint32_t (&sc)[2]) {
  const float denom = 6.0f * g;  // fl32(6 g)
  bool odd = false;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(xh[16 * b + i]));
    const uint32_t scode = e4m3_code(amax / denom);
    sc[b] = scode;
    s[b] = e4m3_value(scode);
    d[b] = s[b] * g;  // fl32(s g)
    r[b] = s[b] > 0.f ? 1.0f / d[b] : 0.f;
    odd |= s[b] > 0.f && !(d[b] >= 0x1p-100f && amax * r[b] <= 0x1p100f);
  }
  return odd;
}

// The lane's codes packed as the operand dwords: dw[2 b + h] holds the eight codes of
// block b, k = 16 b + 8 h + [0, 8), element e in bits 4e..4e+3 (the quantizer's GEMM
// operand and interchange layouts both store these dwords as they are).  The quotients
// are those of nvfp4_quant32, refined as y - e' r with e' = y d - xhat, which keeps the
// sign of a zero quotient (-0 stays -0: the sign is the quotient's, i.e. xhat's), so
// the converter's own signed codes are the codes; it writes two of them into byte i of
// the dword (its destination-byte operand).  A block with s = 0 has zero codes.
__device__ __forceinline__ void nvfp4_quant32_packed(const float (&xh)[32], float g,
                                                     uint32_t (&dw)[4], uint32_t (&sc)[2]) {
  float s[2], d[2], r[2];
  const bool odd = nvfp4_block_scales(xh, g, s, d, r, sc);
  float quot[32];
  if (__any(odd)) {
#pragma unroll
    for (int i = 0; i < 32; ++i)
      quot[i] = __builtin_amdgcn_fmed3f(s[i >> 4] > 0.f ? xh[i] / d[i >> 4] : 0.f, -8.0f, 8.0f);
  } else {
    // |quotient| <= 6 / (1 - 2^-4): the converter saturates it at 6 without a clamp
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float y = xh[i] * r[i >> 4];
      const float en = __builtin_fmaf(y, d[i >> 4], -xh[i]);  // exact: y d - xhat
      quot[i] = __builtin_fmaf(-en, r[i >> 4], y);
    }
  }
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e0 = 16 * b + 8 * h;
      uint32_t w = 0;
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, quot[e0 + 0], quot[e0 + 1], 1.0f, 0);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, quot[e0 + 2], quot[e0 + 3], 1.0f, 1);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, quot[e0 + 4], quot[e0 + 5], 1.0f, 2);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, quot[e0 + 6], quot[e0 + 7], 1.0f, 3);
      dw[2 * b + h] = s[b] > 0.f ? w : 0u;
    }
}

__device__ __forceinline__ void nvfp4_quant32(const float (&xh)[32], float g, uint32_t (&codes)[32],
                                              float (&deq)[32], uint32_t (&sc)[2]) {
  float s[2], d[2], r[2];
  const bool odd = nvfp4_block_scales(xh, g, s, d, r, sc);
  float quot[32];
  if (__any(odd)) {
#pragma unroll
    for (int i = 0; i < 32; ++i) quot[i] = s[i >> 4] > 0.f ? xh[i] / d[i >> 4] : 0.f;
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float y = xh[i] * r[i >> 4];
      const float e = __builtin_fmaf(-y, d[i >> 4], xh[i]);
      quot[i] = __builtin_fmaf(e, r[i >> 4], y);
    }
  }
  // E2M1 magnitudes from the hardware converter (scale 1: nearest, ties to the even
  // code, saturating at 6; checked against e2m1_mag on every midpoint and its ulp
  // neighbours); quotients are clamped to 8 first so an overflowed quotient of the
  // division path saturates too.  The sign is xhat's.
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const float half_s = 0.5f * s[b];
    const uint32_t live = s[b] > 0.f ? 0xFu : 0u;
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const float q0 = __builtin_amdgcn_fmed3f(quot[16 * b + i], -8.0f, 8.0f);
      const float q1 = __builtin_amdgcn_fmed3f(quot[16 * b + i + 1], -8.0f, 8.0f);
      const uint32_t pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, q0, q1, 1.0f, 0);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t xb = __float_as_uint(xh[16 * b + i + h]);
        const uint32_t c = (((pk >> (4 * h)) & 7u) | ((xb >> 28) & 8u)) & live;
        codes[16 * b + i + h] = c;
        const float v = (float)e2m1_twice(c & 7u) * half_s;  // exact
        deq[16 * b + i + h] = __uint_as_float(__float_as_uint(v) | ((c & 8u) << 28));
      }
    }
  }
}

}  // namespace svdq
