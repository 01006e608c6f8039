// Weight packing: interchange layout -> kernel layout (an offline step).
//
// int4: codes [N][K/2] two's complement nibbles -> E2M3 lane slots of common.h
//       (row-blocks of 32 output columns), scales [N][K/64] bf16 -> [K/64][N]
//       8-byte records {s, 0, 0, 0} (common.h).
//       Every code of the int4 range [-8, 7] is an exact E2M3 value q/8: |q| <= 7
//       are subnormals (magnitude in bits 2:0) and -8 is the normal -1.0 (exponent
//       field 1, mantissa 0), i.e. the same sign-magnitude field with magnitude 8.
// lora_down: [r][K] bf16 -> fragment order of the quantizer's low-rank MFMAs: for
//       k-block kb (128 values), rank slice sl (16 ranks) and call c (0..3), lane
//       l = 16 q + i holds lora_down[16 sl + i][128 kb + 32 q + 8 c .. + 8] (16 B), and
//       the 64 lanes of one (kb, sl, c) are 1 KiB contiguous.
// nvfp4: codes [N][K/2] E2M1 nibbles and scales [N][K/16] E4M3 bytes -> the FP4
//       lane-slot chunks of common.h (4 bits per weight, per 32 output columns and
//       64-group) and the scales as exact fp16 values [K/64][N][4].  An E4M3 NaN scale
//       raises the range flag.
#include "common.h"
#include "kernels.h"

namespace svdq {

// One thread per (row-block, group, lane slot h*32 + row % 32): reads the 16
// interchange bytes of 32 codes and writes their six dwords of E2M3 fields.
__global__ void __launch_bounds__(256)
k_pack_int4_codes(const uint8_t* __restrict__ codes, uint8_t* __restrict__ out, int N, int K) {
  const int G = K >> 6;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)N * G * 2;
  if (t >= total) return;
  const int slot = (int)(t & 63);
  const int r = slot & 31, h = slot >> 5;
  const int64_t rest = t >> 6;         // (row-block, group)
  const int g = (int)(rest % G);
  const int64_t rb = rest / G;
  const int64_t n = rb * 32 + r;
  const uint4 v = *reinterpret_cast<const uint4*>(codes + n * (K >> 1) + 32 * g + 16 * h);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[6] = {0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
  for (int f = 0; f < 32; ++f) {
    const uint32_t nib = (w[f >> 3] >> (4 * (f & 7))) & 0xFu;
    const int q = (nib & 8u) ? (int)nib - 16 : (int)nib;
    const uint32_t fld = e2m3_field(q);
    const int pos = 6 * f, word = pos >> 5, bit = pos & 31;
    o[word] |= fld << bit;
    if (bit > 26) o[word + 1] |= fld >> (32 - bit);
  }
  uint8_t* chunk = out + (size_t)rest * 1536;
  *reinterpret_cast<uint4*>(chunk + slot * 16) = make_uint4(o[0], o[1], o[2], o[3]);
  *reinterpret_cast<uint2*>(chunk + 1024 + slot * 8) = make_uint2(o[4], o[5]);
}

// Weight scale records, one per pair of groups: {sw[n, 2p], sw[n, 2p + 1], 0, 0}.
__global__ void __launch_bounds__(256)
k_pair_scales(const uint16_t* __restrict__ in, uint2* __restrict__ out, int N, int G) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= (int64_t)N * (G / 2)) return;
  const int64_t p = t / N, n = t % N;
  out[t] = make_uint2((uint32_t)in[n * G + 2 * p] | ((uint32_t)in[n * G + 2 * p + 1] << 16), 0u);
}

// NVFP4 codes: one thread per (column block, 64-group, lane slot 32 h + n % 32): the
// four dwords of blocks 4 q + j, each the eight codes k = 64 q + 16 j + 8 h + [0, 8) of
// column n, are 4 interchange bytes apiece (element 2i in the low nibble of byte i).
__global__ void __launch_bounds__(256)
k_pack_nvfp4_codes(const uint8_t* __restrict__ codes, uint32_t* __restrict__ out, int N, int K) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int Q = K >> 6;
  if (t >= (int64_t)N * Q * 2) return;
  const int slot = (int)(t & 63), h = slot >> 5;
  const int64_t rest = t >> 6;  // (column block, group)
  const int q = (int)(rest % Q);
  const int64_t n = (rest / Q) * 32 + (slot & 31);
  const uint8_t* src = codes + n * (K / 2) + 32 * q + 4 * h;
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = *reinterpret_cast<const uint32_t*>(src + 8 * j);
  // dword-major chunk (weights): dword j of lane slot s at dword 64 j + s of the chunk
#pragma unroll
  for (int j = 0; j < 4; ++j) out[(rest * 4 + j) * 64 + slot] = w[j];
}

// NVFP4 scales: one thread per (64-group q, column n): the four E4M3 scales of the
// group as their exact fp16 values, at [q][n][0..3]; a NaN code raises the flag.
__global__ void __launch_bounds__(256)
k_pack_nvfp4_scales(const uint8_t* __restrict__ scales, uint2* __restrict__ out, int N, int K,
                    int* __restrict__ flag) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int Q = K >> 6;
  if (t >= (int64_t)N * Q) return;
  const int64_t q = t / N, n = t % N;
  const uint32_t sc4 = *reinterpret_cast<const uint32_t*>(scales + n * (K / 16) + 4 * q);
  uint32_t h[4];
  bool nan = false;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t sc = (sc4 >> (8 * j)) & 0xFFu;
    nan |= (sc & 0x7Fu) == 0x7Fu;
    const uint32_t e = (sc >> 3) & 15u, m = sc & 7u;
    float s = e == 0 ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
    if (sc & 0x80u) s = -s;
    h[j] = __builtin_bit_cast(uint16_t, (_Float16)s);  // exact: E4M3 values are fp16 numbers
  }
  out[t] = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
  if (nan) atomicOr(flag, 1);
}

// One thread per 16-byte unit of the packed lora_down.
__global__ void __launch_bounds__(256)
k_pack_lora_down(const uint16_t* __restrict__ in, uint4* __restrict__ out, int rank, int K) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int nsl = rank / 16;
  const int64_t total = (int64_t)(K / 128) * nsl * 4 * 64;
  if (t >= total) return;
  const int lane = (int)(t & 63), c = (int)((t >> 6) & 3);
  const int64_t rest = t >> 8;
  const int sl = (int)(rest % nsl);
  const int64_t kb = rest / nsl;
  const int i = lane & 15, q = lane >> 4;
  out[t] = *reinterpret_cast<const uint4*>(in + (int64_t)(16 * sl + i) * K + 128 * kb + 32 * q + 8 * c);
}

__global__ void k_zero_flag(int* flag) { *flag = 0; }

hipError_t launch_pack_int4(const uint8_t* codes, const uint16_t* scales, uint8_t* out_codes,
                            void* out_scales, int* flag, int N, int K, hipStream_t st) {
  const int G = K >> 6;
  hipLaunchKernelGGL(k_zero_flag, dim3(1), dim3(1), 0, st, flag);
  const int64_t total = (int64_t)N * G * 2;
  hipLaunchKernelGGL(k_pack_int4_codes, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st,
                     codes, out_codes, N, K);
  const int64_t ts = (int64_t)N * (G / 2);
  hipLaunchKernelGGL(k_pair_scales, dim3((unsigned)((ts + 255) / 256)), dim3(256), 0, st,
                     scales, reinterpret_cast<uint2*>(out_scales), N, G);
  return hipGetLastError();
}



hipError_t launch_pack_lora_down(const uint16_t* in, uint16_t* out, int rank, int K, hipStream_t st) {
  const int64_t total = (int64_t)(K / 128) * (rank / 16) * 4 * 64;
  hipLaunchKernelGGL(k_pack_lora_down, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, in,
                     reinterpret_cast<uint4*>(out), rank, K);
  return hipGetLastError();
}

hipError_t launch_pack_nvfp4(const uint8_t* codes, const uint8_t* scales, uint8_t* out_codes,
                             uint16_t* out_scales, int* flag, int N, int K, hipStream_t st) {
  hipLaunchKernelGGL(k_zero_flag, dim3(1), dim3(1), 0, st, flag);
  const int64_t tc = (int64_t)N * (K / 64) * 2;
  hipLaunchKernelGGL(k_pack_nvfp4_codes, dim3((unsigned)((tc + 255) / 256)), dim3(256), 0, st, codes,
                     reinterpret_cast<uint32_t*>(out_codes), N, K);
  const int64_t ts = (int64_t)N * (K / 64);
  hipLaunchKernelGGL(k_pack_nvfp4_scales, dim3((unsigned)((ts + 255) / 256)), dim3(256), 0, st,
                     scales, reinterpret_cast<uint2*>(out_scales), N, K, flag);
  return hipGetLastError();
}

}  // namespace svdq
