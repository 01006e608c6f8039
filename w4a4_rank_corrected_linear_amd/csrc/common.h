// Device-side helpers and data layouts shared by the gfx950 kernels.
//
// Lane-slot layout of int4 GEMM operands
// --------------------------------------
// The int4 GEMM runs on the scaled FP6 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4 with
// E2M3 operands).  An int4 code v in [-7, 7] is the E2M3 subnormal with sign bit 5
// and the magnitude |v| in bits 2:0, whose value is v/8; E8M0 block scales make the
// MFMA return an exact multiple of the integer dot product of a 64-group in fp32.
//
// Both operands (activations written by the quantizer, weights written by the pack)
// are stored as the MFMA reads them: rows are grouped in blocks of 32, and one
// 64-group of one row-block is a 1536-byte chunk
//     chunk(row, g) = ((row / 32) * G + g) * 1536
// in which lane slot l = 32 h + row % 32 (h = 0, 1) holds the 32 fields of
// k = 64 g + 32 h + f, f = 0..31, field f in bits 6f..6f+5 of six dwords; dwords
// 0-3 sit at chunk + 16 l and dwords 4-5 at chunk + 1024 + 8 l, so a 64-lane
// 16-byte and a 64-lane 8-byte access read one whole operand.
//
// Scale records (operands of the rescale MFMA, one 64-bit load each)
// -------------------------------------------------------------------
// Activation scales sit group-major as 8-byte records, record g * M_pad + row: the
// bf16 scale in bits 15:0 for an even group g and in bits 31:16 for an odd one, zeros
// elsewhere, i.e. the bf16x4 operand {s, 0, 0, 0} or {0, s, 0, 0}.  Weight scales sit
// as one 8-byte record per pair of groups, record (g / 2) * N + n = {sw[n, g & ~1],
// sw[n, g | 1], 0, 0}.  The product of the two operands over the four bf16 positions
// picks sw[n, g] sx[m, g] for either parity, so one weight record serves both groups
// of a pair.
//
// Fragment layout of the low-rank activations U (fp32, the quantizer's partial sums
// per k-split): [split][M_pad / 32][rank / 16][2][64][4] floats.  For rows of one
// 32-row block and ranks 16 c .. 16 c + 15, lane l = row % 32 + 32 * ((rank % 16) / 8)
// holds ranks 16 c + 8 (l / 32) + [0, 8): elements 0-3 in the first 1 KiB, 4-7 in the
// second, so the GEMM reads each half as one contiguous 64-lane 16-byte load in the
// B-operand order of v_mfma_f32_32x32x16_bf16.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svdq {

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

// E2M3 field of an int4 code in [-7, 7]: sign in bit 5, magnitude in bits 2:0.
__device__ __forceinline__ uint32_t e2m3_field(int q) {
  return (q < 0 ? 0x20u : 0u) | (uint32_t)(q < 0 ? -q : q);
}

__device__ __forceinline__ int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

// Index (in floats) of U[split][row][j] in the fragment layout above.
__host__ __device__ __forceinline__ size_t u_frag_index(int split, int row, int j, int M_pad,
                                                        int rank) {
  const int lane = (row & 31) + 32 * ((j & 15) >> 3);
  const int e = j & 7;
  return ((((size_t)split * (M_pad >> 5) + (row >> 5)) * (rank >> 4) + (j >> 4)) * 2 + (e >> 2)) *
             256 + lane * 4 + (e & 3);
}

}  // namespace svdq
