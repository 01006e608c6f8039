// Weight packing: interchange layout -> kernel layout (an offline step).
//
// int4: codes [N][K/2] two's complement nibbles -> E2M3 lane slots of common.h
//       (row-blocks of 32 output columns), scales [N][K/64] bf16 -> [K/64][N]
//       8-byte records {s, 0, 0, 0} (common.h).
//       A -8 code cannot be held by the sign-magnitude E2M3 field: it raises the
//       range flag, which the host turns into SVDQ_ERR_RANGE.
// lora_down: [r][K] bf16 -> fragment order of the quantizer's low-rank MFMAs: for
//       k-block kb (128 values), rank slice sl (16 ranks) and call c (0..3), lane
//       l = 16 q + i holds lora_down[16 sl + i][128 kb + 32 q + 8 c .. + 8] (16 B), and
//       the 64 lanes of one (kb, sl, c) are 1 KiB contiguous.
// nvfp4: codes [N][K/2] E2M1 nibbles and scales [N][K/16] E4M3 bytes -> the exact
//       dequantized weights e2m1 * s as bf16 [N][K] (2 and 4 significant bits: the
//       product is a bf16 number).  An E4M3 NaN scale raises the range flag.
#include "common.h"
#include "kernels.h"

namespace svdq {

// One thread per (row-block, group, lane slot h*32 + row % 32): reads the 16
// interchange bytes of 32 codes and writes their six dwords of E2M3 fields.
__global__ void __launch_bounds__(256)
k_pack_int4_codes(const uint8_t* __restrict__ codes, uint8_t* __restrict__ out, int N, int K,
                  int* __restrict__ flag) {
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
  bool bad = false;
#pragma unroll
  for (int f = 0; f < 32; ++f) {
    const uint32_t nib = (w[f >> 3] >> (4 * (f & 7))) & 0xFu;
    const int q = (nib & 8u) ? (int)nib - 16 : (int)nib;
    bad |= (q == -8);
    const uint32_t fld = e2m3_field(q < -7 ? -7 : q);
    const int pos = 6 * f, word = pos >> 5, bit = pos & 31;
    o[word] |= fld << bit;
    if (bit > 26) o[word + 1] |= fld >> (32 - bit);
  }
  uint8_t* chunk = out + (size_t)rest * 1536;
  *reinterpret_cast<uint4*>(chunk + slot * 16) = make_uint4(o[0], o[1], o[2], o[3]);
  *reinterpret_cast<uint2*>(chunk + 1024 + slot * 8) = make_uint2(o[4], o[5]);
  if (bad) atomicOr(flag, 1);
}

// Weight scale records, one per pair of groups: {sw[n, 2p], sw[n, 2p + 1], 0, 0}.
__global__ void __launch_bounds__(256)
k_pair_scales(const uint16_t* __restrict__ in, uint2* __restrict__ out, int N, int G) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= (int64_t)N * (G / 2)) return;
  const int64_t p = t / N, n = t % N;
  out[t] = make_uint2((uint32_t)in[n * G + 2 * p] | ((uint32_t)in[n * G + 2 * p + 1] << 16), 0u);
}

// One thread per 8 weights (4 code bytes, one E4M3 scale).
__global__ void __launch_bounds__(256)
k_pack_nvfp4(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
             uint4* __restrict__ out, int N, int K, int* __restrict__ flag) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)N * K / 8;
  if (t >= total) return;
  const int64_t n = t / (K / 8), k8 = t % (K / 8);
  const uint32_t w = *reinterpret_cast<const uint32_t*>(codes + n * (K / 2) + 4 * k8);
  const uint32_t sc = scales[n * (K / 16) + k8 / 2];
  if ((sc & 0x7Fu) == 0x7Fu) atomicOr(flag, 1);
  const uint32_t e = (sc >> 3) & 15u, m = sc & 7u;
  float s = e == 0 ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  if (sc & 0x80u) s = -s;
  uint32_t o[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    uint32_t half[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t c = (w >> (4 * (2 * p + h))) & 15u;
      const uint32_t mag = c & 7u;
      const float a = mag < 4 ? 0.5f * (float)mag
                              : (float)(2u << ((mag - 4u) >> 1)) * (1.0f + 0.5f * (float)(mag & 1u));
      const float v = (c & 8u) ? -(a * s) : a * s;
      half[h] = __float_as_uint(v) >> 16;
    }
    o[p] = half[0] | (half[1] << 16);
  }
  out[t] = make_uint4(o[0], o[1], o[2], o[3]);
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
                     codes, out_codes, N, K, flag);
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

hipError_t launch_pack_nvfp4(const uint8_t* codes, const uint8_t* scales, uint16_t* out, int* flag,
                             int N, int K, hipStream_t st) {
  hipLaunchKernelGGL(k_zero_flag, dim3(1), dim3(1), 0, st, flag);
  const int64_t total = (int64_t)N * K / 8;
  hipLaunchKernelGGL(k_pack_nvfp4, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, codes,
                     scales, reinterpret_cast<uint4*>(out), N, K, flag);
  return hipGetLastError();
}

}  // namespace svdq
