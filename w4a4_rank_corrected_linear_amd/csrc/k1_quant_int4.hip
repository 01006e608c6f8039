// K1, int4: smoothing + per-64-group amax + symmetric int4 quantization + packing
// + rank-r low-rank down projection, one pass over X.
//
// Layer definition: Diffusers docs "Nunchaku Lite", "Supported quantization types"
// (svdq_w4a4, int4, group 64, SVDQ low-rank correction); the readings of the open
// steps (smoothing multiplier, amax/7 bf16 scale, round-half-even, symmetric clamp,
// U from the smoothed activations) are those of the layer definition in svdq.h.
//
// Work split: a 256-thread workgroup owns 16 rows; wave w takes the 64-groups
// g = w, w+4, ...  Lane l holds row l%16 and, per group, the two 8-value chunks at
// k = 64g + 32j + 8(l/16), j = 0, 1.  That is exactly the A-operand layout of
// v_mfma_f32_16x16x32_bf16 for the 32-wide k-step j, so the smoothed values feed
// the low-rank MFMA straight from registers.  The group amax is an in-lane max over
// 16 values and two cross-lane steps (lanes l^16, l^32).  Per-wave partial U tiles
// are summed in LDS in a fixed order (deterministic).
#include "common.h"
#include "kernels.h"

namespace svdq {

// round-half-even(xh / s), decided exactly, clamped to [-7, 7].
// y1 = xh * (1/s) is within a few ulp of the quotient; one remainder step
// e = xh - y1 s (exact by fma) and y2 = y1 + e/s lands on the correctly rounded
// quotient, in particular exactly on k + 1/2 at a tie, while a non-tie quotient of
// a bf16 numerator by a bf16 divisor is at least 2^-9 away from any half-integer.
// Scales below 2^-125 (1/s could overflow) take an exact division instead.
__device__ __forceinline__ int quant_int4(float xh, float s, float rcp, bool tiny) {
  float y;
  if (tiny) {
    y = __fdiv_rn(xh, s);
  } else {
    float y1 = xh * rcp;
    float e = __builtin_fmaf(-y1, s, xh);
    y = __builtin_fmaf(e, rcp, y1);
  }
  float q = __builtin_rintf(y);
  q = fminf(fmaxf(q, -7.0f), 7.0f);
  return (int)q;
}

template <bool COMPACT>
__global__ void __launch_bounds__(256)
k1_quant_int4(const uint16_t* __restrict__ x, int M, int K,
              const uint16_t* __restrict__ smooth, const uint16_t* __restrict__ ldown, int rank,
              uint8_t* __restrict__ codes, uint16_t* __restrict__ scales,
              uint16_t* __restrict__ uact, int M_out, int M_pad) {
  __shared__ float ured[4][16][33];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;
  const int q = lane >> 4;
  const int row0 = blockIdx.x * 16;
  const int row = row0 + r;
  const bool valid = row < M;
  const int G = K >> 6;

  v4f u0 = {0.f, 0.f, 0.f, 0.f};
  v4f u1 = {0.f, 0.f, 0.f, 0.f};

  for (int g = wave; g < G; g += 4) {
    uint4 xr[2], mr[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int k = 64 * g + 32 * j + 8 * q;
      xr[j] = valid ? *reinterpret_cast<const uint4*>(x + (size_t)row * K + k) : make_uint4(0, 0, 0, 0);
      mr[j] = *reinterpret_cast<const uint4*>(smooth + k);
    }
    float xh[16];
    uint32_t xb[8];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t* xw = reinterpret_cast<const uint32_t*>(&xr[j]);
      const uint32_t* mw = reinterpret_cast<const uint32_t*>(&mr[j]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t xv = (i & 1) ? (xw[i >> 1] >> 16) : (xw[i >> 1] & 0xFFFFu);
        const uint32_t mv = (i & 1) ? (mw[i >> 1] >> 16) : (mw[i >> 1] & 0xFFFFu);
        const float p = bf16_to_f32(xv) * bf16_to_f32(mv);  // exact product
        const uint32_t hb = f32_to_bf16_rne(p);
        xh[8 * j + i] = bf16_to_f32(hb);
        if (i & 1) xb[4 * j + (i >> 1)] |= hb << 16;
        else xb[4 * j + (i >> 1)] = hb;
      }
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(xh[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    const uint32_t s_bits = f32_to_bf16_rne(amax / 7.0f);
    const float s = bf16_to_f32(s_bits);
    const bool tiny = (s > 0.f) && (s < 0x1p-125f);
    const float rcp = (s > 0.f && !tiny) ? __frcp_rn(s) : 0.f;

    int qv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) qv[i] = quant_int4(xh[i], s, rcp, tiny);

    if (valid || COMPACT) {
      if constexpr (!COMPACT) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          uint32_t w = 0;
#pragma unroll
          for (int i = 0; i < 8; ++i) w |= (uint32_t)(qv[8 * j + i] & 0xF) << (4 * i);
          const size_t off = ((size_t)row * K + 64 * g + 32 * j + 8 * q) >> 1;
          *reinterpret_cast<uint32_t*>(codes + off) = w;
        }
        if (q == 0) scales[(size_t)row * G + g] = (uint16_t)s_bits;
      }
    }
    if constexpr (COMPACT) {
      // rows >= M were loaded as zeros: they produce zero codes and scales, which
      // keeps the padded workspace fully defined.
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        uint64_t acc = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc |= (uint64_t)e2m3_field(qv[8 * j + i]) << (6 * i);
        uint32_t t0, t1, t2;
        if ((q & 1) == 0) {
          t0 = (uint32_t)acc;
          t1 = (uint32_t)(acc >> 32);
          t2 = 0;
        } else {
          t0 = 0;
          t1 = (uint32_t)acc << 16;
          t2 = (uint32_t)(acc >> 16);
        }
        t0 |= __shfl_xor(t0, 16);
        t1 |= __shfl_xor(t1, 16);
        t2 |= __shfl_xor(t2, 16);
        uint32_t x0, x1;
        fp6_compact(t0, t1, t2, x0, x1);
        if ((q & 1) == 0) {
          const size_t off = ((size_t)(row >> 5) * G + g) * 1024 + j * 512 + (row & 31) * 16 + (q >> 1) * 8;
          *reinterpret_cast<uint2*>(codes + off) = make_uint2(x0, x1);
        }
      }
      if (q == 0) scales[(size_t)g * M_pad + row] = (uint16_t)s_bits;
    }

    if (rank > 0) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int k = 64 * g + 32 * j + 8 * q;
        v8s a;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a[2 * i] = (short)(xb[4 * j + i] & 0xFFFFu);
          a[2 * i + 1] = (short)(xb[4 * j + i] >> 16);
        }
        const uint4 b0 = *reinterpret_cast<const uint4*>(ldown + (size_t)r * K + k);
        u0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a),
                                                     __builtin_bit_cast(v8bf, b0), u0, 0, 0, 0);
        if (rank > 16) {
          const uint4 b1 = *reinterpret_cast<const uint4*>(ldown + (size_t)(16 + r) * K + k);
          u1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a),
                                                       __builtin_bit_cast(v8bf, b1), u1, 0, 0, 0);
        }
      }
    }
  }

  if (rank > 0) {
    // C layout of the 16x16 MFMA: lane l holds column l%16, rows 4(l/16) + i.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ured[wave][4 * q + i][r] = u0[i];
      ured[wave][4 * q + i][16 + r] = u1[i];
    }
    __syncthreads();
    for (int t = threadIdx.x; t < 16 * rank; t += 256) {
      const int rr = t / rank, cc = t % rank;
      const float v = ((ured[0][rr][cc] + ured[1][rr][cc]) + ured[2][rr][cc]) + ured[3][rr][cc];
      if (row0 + rr < M_out) uact[(size_t)(row0 + rr) * rank + cc] = (uint16_t)f32_to_bf16_rne(v);
    }
  }
}

// compact = false: interchange layout (codes [M][K/2], scales [M][K/64], U [M][r]).
// compact = true : kernel layout for K2, M_pad rows (codes per common.h, scales
//                  [K/64][M_pad], U [M_pad][r]); rows >= M are written as zeros.
hipError_t launch_k1_int4(bool compact, const uint16_t* x, int M, int K, const uint16_t* smooth,
                          const uint16_t* ldown, int rank, uint8_t* codes, uint16_t* scales,
                          uint16_t* uact, int M_pad, hipStream_t st) {
  const int M_out = compact ? M_pad : M;
  dim3 grid((M_out + 15) / 16);
  if (compact)
    hipLaunchKernelGGL(k1_quant_int4<true>, grid, dim3(256), 0, st, x, M, K, smooth, ldown, rank,
                       codes, scales, uact, M_out, M_pad);
  else
    hipLaunchKernelGGL(k1_quant_int4<false>, grid, dim3(256), 0, st, x, M, K, smooth, ldown, rank,
                       codes, scales, uact, M_out, M_pad);
  return hipGetLastError();
}

}  // namespace svdq
