// Device-side helpers and data layouts shared by the gfx950 kernels.
//
// Kernel ("compact") layout of 4-bit int4 operands
// ------------------------------------------------
// The int4 GEMM runs on the scaled FP6 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4 with
// E2M3 operands).  An int4 code v in [-7, 7] is the E2M3 subnormal with sign bit 5
// and the magnitude |v| in bits 2:0, whose value is v/8; two E8M0 block scales of
// 2^3 make the MFMA return the exact integer dot product of a 64-group in fp32.
// The MFMA reads 32 six-bit fields per lane (6 dwords, field f in bits 6f..6f+5).
//
// In memory a 16-value run is stored in 8 bytes (x0, x1), which is what 16 codes
// take as nibbles.  Fields carry information only in bits {0,1,2,5}; in the 96-bit
// triple (out0, out1, out2) of a 16-field run the always-zero positions of out0
// (Z0) and of out2 (Z2) are disjoint and together are exactly the informative
// positions of out1, so
//     x0 = out0 | (out1 & Z0),   x1 = out2 | (out1 & Z2)
// and the decode back to MFMA fields is four bit operations:
//     out0 = x0 & ~Z0,  out2 = x1 & ~Z2,  out1 = (x0 & Z0) | (x1 & Z2).
//
// Ordering: rows are grouped in blocks of 32; one 64-group of one row-block is a
// 1 KiB chunk [half h (k 32h..32h+31)][row % 32][16 B = pair0 (x0,x1), pair1].
// Pair p of half h holds k = 64 g + 32 h + 16 p + j, j = 0..15, field j.
//     byte offset(row, g) = ((row / 32) * G + g) * 1024 + h * 512 + (row % 32) * 16
// Per-group scales sit group-major: scales[g * R_pad + row] (bf16).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svdq {

constexpr uint32_t kZ0 = 0x18618618u;
constexpr uint32_t kZ2 = 0x61861861u;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v8s __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Triple (out0, out1, out2) of 16 E2M3 fields -> compact (x0, x1).
__device__ __forceinline__ void fp6_compact(uint32_t o0, uint32_t o1, uint32_t o2,
                                            uint32_t& x0, uint32_t& x1) {
  x0 = o0 | (o1 & kZ0);
  x1 = o2 | (o1 & kZ2);
}

// Compact (x0, x1) -> the three MFMA dwords of 16 E2M3 fields.
__device__ __forceinline__ void fp6_expand(uint32_t x0, uint32_t x1, uint32_t& o0,
                                           uint32_t& o1, uint32_t& o2) {
  o0 = x0 & ~kZ0;
  o2 = x1 & ~kZ2;
  o1 = (x0 & kZ0) | (x1 & kZ2);
}

// E2M3 field of an int4 code in [-7, 7]: sign in bit 5, magnitude in bits 2:0.
__device__ __forceinline__ uint32_t e2m3_field(int q) {
  return (q < 0 ? 0x20u : 0u) | (uint32_t)(q < 0 ? -q : q);
}

__device__ __forceinline__ int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

}  // namespace svdq
