// K1, nvfp4: smoothing + per-16-block amax + E4M3 block scale + E2M1 codes + rank-r
// low-rank down projection, one pass over X.
//
// Layer definition: Diffusers docs "Nunchaku Lite", "Supported quantization types"
// (svdq_w4a4, nvfp4, group 16, SVDQ low-rank correction).  Readings, as stated in
// svdq.h: xhat = bf16(x m); per block of 16, s = E4M3(fl32(amax / fl32(6 g))) (round
// to nearest even, saturating at 448); code = E2M1(fl32(xhat / fl32(s g))) (nearest,
// ties to the even code, saturating at 6), sign from the quotient's sign bit; s = 0
// gives zero codes; U = xhat @ lora_down^T in fp32.
//
// As in the int4 quantizer, lane l holds row l%16 and the 32 consecutive values
// k0 .. k0 + 31 of a 128-wide k-block (k0 = 128 kb + 32 q, q = l/16), i.e. two whole
// NVFP4 blocks, so every amax is an in-lane max.
//
// Two kernels share the quantizer below: k1_nvfp4_fused (the layer's own path, batch
// skeleton of k1_batch.h) writes the exact dequantized GEMM operand
// A' = e2m1(code) * s as bf16 [M_pad][K] (|e2m1| has 2 and s 4 significant bits, so the
// product is exact in bf16) and partial U per k-split; the per-tensor scale g stays
// out of A' and is applied to the GEMM's fp32 result.  k1_nvfp4_interchange
// (svdq_quantize_act) writes codes [M][K/2] (element 2j in bits 3:0), E4M3 scale
// bytes [M][K/16] and U [M][r].
#include "common.h"
#include "k1_batch.h"
#include "kernels.h"

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
__device__ __forceinline__ void nvfp4_quant32(const float (&xh)[32], float g, uint32_t (&codes)[32],
                                              float (&deq)[32], uint32_t (&sc)[2]) {
  const float denom = 6.0f * g;  // fl32(6 g)
  float s[2], d[2], r[2];
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

struct QuantNvfp4Fused {
  __device__ static void block(const K1Args& a, const float (&xh)[32], int row, int k0, int q) {
    (void)q;
    uint32_t codes[32], sc[2];
    float deq[32];
    nvfp4_quant32(xh, a.g, codes, deq, sc);
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      w[i] = (__float_as_uint(deq[2 * i]) >> 16) | (__float_as_uint(deq[2 * i + 1]) & 0xFFFF0000u);
    uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.out) + (size_t)row * a.K + k0);
#pragma unroll
    for (int c = 0; c < 4; ++c) dst[c] = make_uint4(w[4 * c], w[4 * c + 1], w[4 * c + 2], w[4 * c + 3]);
  }
};

__global__ void __launch_bounds__(256, 2) k1_nvfp4_fused(K1Args a) { k1_batch<QuantNvfp4Fused>(a); }

struct K1Load {
  uint4 x[4];
  uint4 m[4];
  uint4 l[2][4];
};

// Interchange kernel: a 512-thread workgroup owns 16 rows; wave w takes the 128-wide
// k-blocks kb = w, w+8, ... and prefetches the next block's X, smoothing and
// lora_down operands into registers.  U is summed over the 8 waves in LDS.
__global__ void __launch_bounds__(512)
k1_nvfp4_interchange(const uint16_t* __restrict__ x, int M, int K,
                     const uint16_t* __restrict__ smooth, const uint16_t* __restrict__ ldown,
                     int rank, float g, uint8_t* __restrict__ out, uint8_t* __restrict__ scales,
                     float* __restrict__ uact) {
  __shared__ float ured[8][16][33];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;
  const int q = lane >> 4;
  const int row0 = blockIdx.x * 16;
  const int row = row0 + r;
  const bool valid = row < M;
  const int nkb = K >> 7;

  v4f u0 = {0.f, 0.f, 0.f, 0.f};
  v4f u1 = {0.f, 0.f, 0.f, 0.f};

  auto load = [&](int kb, K1Load& L) {
    const int k0 = 128 * kb + 32 * q;
    const uint4* xp = reinterpret_cast<const uint4*>(x + (size_t)row * K + k0);
    const uint4* mp = reinterpret_cast<const uint4*>(smooth + k0);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      L.x[c] = valid ? xp[c] : make_uint4(0, 0, 0, 0);
      L.m[c] = mp[c];
    }
    if (rank > 0) {
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        if (sl * 16 < rank) {
          const uint4* lp = reinterpret_cast<const uint4*>(ldown + (size_t)(16 * sl + r) * K + k0);
#pragma unroll
          for (int c = 0; c < 4; ++c) L.l[sl][c] = lp[c];
        }
      }
    }
  };

  K1Load cur, nxt;
  int kb = wave;
  if (kb < nkb) load(kb, cur);
  for (; kb < nkb; kb += 8) {
    if (kb + 8 < nkb) load(kb + 8, nxt);
    const int k0 = 128 * kb + 32 * q;

    float xh[32];
    uint32_t xb[16];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t* xw = reinterpret_cast<const uint32_t*>(&cur.x[c]);
      const uint32_t* mw = reinterpret_cast<const uint32_t*>(&cur.m[c]);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float p0 = __uint_as_float(xw[p] << 16) * __uint_as_float(mw[p] << 16);
        const float p1 = __uint_as_float(xw[p] & 0xFFFF0000u) * __uint_as_float(mw[p] & 0xFFFF0000u);
        const v2bf pk = {(__bf16)p0, (__bf16)p1};
        const uint32_t w = __builtin_bit_cast(uint32_t, pk);
        xb[4 * c + p] = w;
        xh[8 * c + 2 * p] = __uint_as_float(w << 16);
        xh[8 * c + 2 * p + 1] = __uint_as_float(w & 0xFFFF0000u);
      }
    }

    uint32_t codes[32], sc[2];
    float deq[32];
    nvfp4_quant32(xh, g, codes, deq, sc);

    {
      if (valid) {
        uint32_t w[4];
#pragma unroll
        for (int d4 = 0; d4 < 4; ++d4) {
          uint32_t acc = 0;
#pragma unroll
          for (int i = 7; i >= 0; --i) acc = (acc << 4) | codes[8 * d4 + i];
          w[d4] = acc;
        }
        *reinterpret_cast<uint4*>(out + ((size_t)row * K + k0) / 2) = make_uint4(w[0], w[1], w[2], w[3]);
        *reinterpret_cast<uint16_t*>(scales + (size_t)row * (K / 16) + k0 / 16) =
            (uint16_t)(sc[0] | (sc[1] << 8));
      }
    }

    if (rank > 0) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const v4i a4 = {(int)xb[4 * c], (int)xb[4 * c + 1], (int)xb[4 * c + 2], (int)xb[4 * c + 3]};
        const v8bf a = __builtin_bit_cast(v8bf, a4);
        u0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(v8bf, cur.l[0][c]), u0, 0,
                                                     0, 0);
        if (rank > 16)
          u1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(v8bf, cur.l[1][c]), u1,
                                                       0, 0, 0);
      }
    }
    cur = nxt;
  }

  if (rank > 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ured[wave][4 * q + i][r] = u0[i];
      ured[wave][4 * q + i][16 + r] = u1[i];
    }
    __syncthreads();
    for (int t = threadIdx.x; t < 16 * rank; t += 512) {
      const int rr = t / rank, cc = t % rank;
      float v = ured[0][rr][cc];
#pragma unroll
      for (int w = 1; w < 8; ++w) v += ured[w][rr][cc];
      if (row0 + rr < M) uact[(size_t)(row0 + rr) * rank + cc] = v;
    }
  }
}

// fused = false: codes [M][K/2], scales [M][K/16] (E4M3 bytes), U [M][r] fp32.
// fused = true : A' bf16 [M_pad][K] (rows >= M are zero), partial U per k-split in the
//                fragment layout of common.h.
hipError_t launch_k1_nvfp4(bool fused, const uint16_t* x, int M, int K, const uint16_t* smooth,
                           const uint16_t* ldown, int rank, float g, uint8_t* out, uint8_t* scales,
                           float* uact, int M_pad, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  if (fused) {
    K1Args a{x, M, K, smooth, ldown, rank, out, scales, uact, M_pad, g};
    dim3 grid(M_pad / 16, k1_splits(K));
    hipExtLaunchKernelGGL(k1_nvfp4_fused, grid, dim3(256), 0, st, ev0, ev1, 0, a);
  } else {
    dim3 grid((M + 15) / 16);
    hipExtLaunchKernelGGL(k1_nvfp4_interchange, grid, dim3(512), 0, st, ev0, ev1, 0, x, M, K,
                          smooth, ldown, rank, g, out, scales, uact);
  }
  return hipGetLastError();
}

}  // namespace svdq
