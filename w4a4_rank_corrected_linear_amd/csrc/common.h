// Device-side helpers and data layouts shared by the gfx950 kernels.
//
// Lane-slot layout of int4 GEMM operands
// --------------------------------------
// The int4 GEMM runs on the scaled FP6 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4 with
// E2M3 operands).  An int4 code v in [-8, 7] is the E2M3 number v/8 with sign bit 5
// and the magnitude |v| in bits 3:0 (|v| <= 7: a subnormal; |v| = 8: the normal 1.0,
// exponent field 1 and mantissa 0); E8M0 block scales make the
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
// FP4 lane-slot layout of NVFP4 GEMM operands
// ---------------------------------------------
// The NVFP4 GEMM runs on v_mfma_f32_32x32x16_f16, one 16-value NVFP4 block of k per
// MFMA, in which lane l takes row l % 32 and k = 8 (l / 32) + [0, 8) of the block.  Both
// operands (activations written by the quantizer, weights written by the pack) keep
// their E2M1 codes in that order: chunk (row / 32, q) of 1 KiB holds the 64-group
// k = 64 q .. 64 q + 63 of a 32-row block, lane slot l = 32 h + row % 32 (16 bytes) holds
// in dword j the eight codes of block 4 q + j, k = 64 q + 16 j + 8 h + [0, 8) (element 2i
// in the low nibble of byte i).  The quantizer writes the activation chunks slot-major
// (lane slot l's four dwords at bytes 16 l .. 16 l + 15, one 16-byte read per lane);
// the pack writes the weight chunks dword-major (dword j of lane slot l at byte
// 256 j + 4 l), so that the 64 dwords of one block, which the GEMM's weight expansion
// reads together, are one run of 256 bytes with no LDS bank conflicts.  Block scales
// are the exact fp16 values of the E4M3 scales, [K/64][rows][4]: the four blocks of a
// row's 64-group are 8 adjacent bytes.
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

// Stores of the quantizers' GEMM operands, written through the L2 at device scope
// (global_store ... sc1): the data is read once, by the next kernel, on every XCD, so
// it need not sit dirty in the writing XCD's L2 until the release at the kernel's end
// writes it back.  Same box, whole call: 53.4 -> 52.6 us at M = 4096, K = N = 3072
// int4 (quantizer 9.8 -> 9.0 us), 87.0 -> 86.1 us for NVFP4, unchanged at the QKV and
// MLP-down shapes.  Non-temporal stores (nt) made the quantizer as fast but the GEMM
// after it slower (QKV +12 us, MLP-down +9 us): the operands then come from HBM
// instead of the Infinity Cache.  The stores are ordinary vector stores; the wait
// counters still cover them, so the waits the compiler places only grow stricter.
typedef uint32_t wt_u4 __attribute__((ext_vector_type(4)));
typedef uint32_t wt_u2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_wt(void* p, uint4 v) {
  const wt_u4 w{v.x, v.y, v.z, v.w};
  asm volatile("global_store_dwordx4 %0, %1, off sc1" :: "v"(p), "v"(w) : "memory");
}
__device__ __forceinline__ void store_wt(void* p, uint2 v) {
  const wt_u2 w{v.x, v.y};
  asm volatile("global_store_dwordx2 %0, %1, off sc1" :: "v"(p), "v"(w) : "memory");
}
__device__ __forceinline__ void store_wt(void* p, uint32_t v) {
  asm volatile("global_store_dword %0, %1, off sc1" :: "v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void store_wt(float* p, v4f v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" :: "v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void store_wt(float* p, float v) {
  asm volatile("global_store_dword %0, %1, off sc1" :: "v"(p), "v"(v) : "memory");
}

// LDS DMA copy: lane i's 16 bytes at g go to LDS at lds + 16 i (lds wave-uniform).
// Written as asm so that the compiler does not see it: for the builtin it waits for
// every copy in flight before any LDS access of the wave (it cannot tell the copy's
// destination from the accessed tile), which serializes a ring of tiles.  Every read
// of a copied tile must therefore follow an explicit s_waitcnt vmcnt that covers the
// copy; the instruction has no register result.
__device__ __forceinline__ void lds_dma16(const void* g, const void* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds;
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(m0) : "memory");
}

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// E2M3 field of an int4 code in [-8, 7]: sign in bit 5, magnitude |q| in bits 3:0
// (the value q/8: subnormal for |q| <= 7, the normal 1.0 for |q| = 8).
__device__ __forceinline__ uint32_t e2m3_field(int q) {
  return (q < 0 ? 0x20u : 0u) | (uint32_t)(q < 0 ? -q : q);
}

__device__ __forceinline__ int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

// exp(y) for y <= 0 with a two-part reduction: y = n ln2 + r, |r| <= ln2/2, ln2 split
// into a 12-bit head (n ln2_hi exact) and a tail; exp(r) = 2^(r log2 e) on the hardware
// exponential (its argument stays within 1/2, so the product's rounding is negligible),
// then the exponent n by ldexp, which also yields fp32 subnormals below FLT_MIN.
__device__ __forceinline__ float exp_nonpos(float y) {
  const float n = __builtin_rintf(y * 1.4426950408889634f);
  float r = __builtin_fmaf(-n, 0.693145751953125f, y);
  r = __builtin_fmaf(-n, 1.4286068203094173e-6f, r);
  return __builtin_ldexpf(__builtin_amdgcn_exp2f(r * 1.4426950408889634f), (int)n);
}

// erfc(z) for z >= 0 after Numerical Recipes' erfcc (Press et al., "Incomplete Gamma
// Function, Error Function ...", Chebyshev-fitted: erfc(z) = t exp(-z^2 + P(t)),
// t = 1 / (1 + z/2), fractional error below 1.2e-7 everywhere).
__device__ __forceinline__ float erfc_nonneg(float z) {
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.5f, z, 1.0f));
  float p = 0.17087277f;
  p = __builtin_fmaf(p, t, -0.82215223f);
  p = __builtin_fmaf(p, t, 1.48851587f);
  p = __builtin_fmaf(p, t, -1.13520398f);
  p = __builtin_fmaf(p, t, 0.27886807f);
  p = __builtin_fmaf(p, t, -0.18628806f);
  p = __builtin_fmaf(p, t, 0.09678418f);
  p = __builtin_fmaf(p, t, 0.37409196f);
  p = __builtin_fmaf(p, t, 1.00002368f);
  p = __builtin_fmaf(p, t, -1.26551223f);
  return t * exp_nonpos(fmaxf(__builtin_fmaf(-z, z, p), -200.0f));
}

// Exact (erf) GELU in fp32: v Phi(v) = v/2 * erfc(-v/sqrt 2); erfc of the negative
// argument is 2 - erfc(|.|), so the v < 0 side keeps its relative accuracy.
__device__ __forceinline__ float gelu_f32(float v) {
  const float e = erfc_nonneg(fabsf(v) * 0.70710678118654752f);
  return 0.5f * v * (v < 0.f ? e : 2.0f - e);
}

// Index (in floats) of U[split][row][j] in the fragment layout above.
__host__ __device__ __forceinline__ size_t u_frag_index(int split, int row, int j, int M_pad,
                                                        int rank) {
  const int lane = (row & 31) + 32 * ((j & 15) >> 3);
  const int e = j & 7;
  return ((((size_t)split * (M_pad >> 5) + (row >> 5)) * (rank >> 4) + (j >> 4)) * 2 + (e >> 2)) *
             256 + lane * 4 + (e & 3);
}

// u = h + m + l + e with h, m, l bf16 and |e| <= 2^-27 |u| (each step's remainder is
// exact in fp32 and keeps 8 more bits): the low-rank term's fp32 U fed to bf16 MFMAs
// as three products whose sum is U L2 to fp32 accuracy (two terms leave 2^-18 |u|,
// which is visible next to large |U|).
struct Bf16x3 {
  __bf16 h, m, l;
};
__device__ __forceinline__ Bf16x3 split3_bf16(float u) {
  Bf16x3 r;
  r.h = (__bf16)u;
  const float r1 = u - (float)r.h;
  r.m = (__bf16)r1;
  r.l = (__bf16)(r1 - (float)r.m);
  return r;
}

}  // namespace svdq
