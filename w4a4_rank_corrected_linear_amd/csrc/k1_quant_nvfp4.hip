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
// Two kernels share the quantizer below: k1_nvfp4_fused32 and k1_nvfp4_stream (the
// layer's own path, the row-pair and row-stream skeletons of k1_rows32.h and
// k1_stream.h)
// write the GEMM operand 4-bit: the E2M1 codes in the FP4 lane-slot layout of common.h
// and each block's E4M3 scale as its exact fp16 value, plus partial U per k-split; the
// per-tensor scale g stays out of the operand and is applied to the GEMM's fp32
// result.  k1_nvfp4_interchange (svdq_quantize_act) writes codes [M][K/2] (element 2j
// in bits 3:0), E4M3 scale bytes [M][K/16] and U [M][r].
#include "common.h"
#include "k1_common.h"
#include "k1_rows32.h"
#include "k1_stream.h"
#include "nvfp4_device.h"
#include "kernels.h"

namespace svdq {

struct QuantNvfp4Fused {
  static constexpr int kStores = 3;  // vector memory stores per call (wait counts)
  __device__ static void block(const K1Args& a, const float (&xh)[32], int row, int k0, int q) {
    (void)q;
    uint32_t dw[4], sc[2];
    nvfp4_quant32_packed(xh, a.g, dw, sc);
    // the lane's 32 values are blocks j0 and j0 + 1 of the 64-group k0 / 64; in each,
    // half h (eight codes, one dword dw[2 b + h]) goes to lane slot 32 h + row % 32
    const int g64 = k0 >> 6, j0 = (k0 >> 4) & 3;
    uint8_t* chunk = a.out + ((size_t)(row >> 5) * (a.K >> 6) + g64) * 1024;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      store_wt(chunk + (h * 32 + (row & 31)) * 16 + j0 * 4, make_uint2(dw[h], dw[2 + h]));
    // the two block scales as fp16 (exact: E4M3 values are fp16 numbers)
    const uint32_t h0 = __builtin_bit_cast(uint16_t, (_Float16)e4m3_value(sc[0]));
    const uint32_t h1 = __builtin_bit_cast(uint16_t, (_Float16)e4m3_value(sc[1]));
    store_wt(static_cast<uint16_t*>(a.scales) + ((size_t)g64 * a.M_pad + row) * 4 + j0, h0 | (h1 << 16));
  }
};

// The two skeletons of the int4 quantizer, chosen the same way (k1_quant_int4.hip).
template <bool GELU_IN>
__global__ void __launch_bounds__(768, 1) k1_nvfp4_fused32(K1Args a) {
  k1_rows32<QuantNvfp4Fused, GELU_IN>(a);
}
template <bool GELU_IN>
__global__ void __launch_bounds__(768, 1) k1_nvfp4_stream(K1Args a) {
  k1_stream<QuantNvfp4Fused, GELU_IN>(a);
}

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

    uint32_t w[4], sc[2];
    nvfp4_quant32_packed(xh, g, w, sc);

    {
      if (valid) {
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
// fused = true : E2M1 codes in the FP4 lane-slot layout and fp16 block scales
//                [K/64][M_pad][4] (common.h; rows >= M are zero), partial U per k-split
//                in the fragment layout of common.h.
hipError_t launch_k1_nvfp4(bool fused, bool gelu_in, const uint16_t* x, int M, int K, const uint16_t* smooth,
                           const uint16_t* ldown, int rank, float g, uint8_t* out, uint8_t* scales,
                           float* uact, int M_pad, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  if (fused) {
    K1Args a{x, M, K, smooth, ldown, rank, out, scales, uact, M_pad, g};
    const int splits = k1_splits(K);
    if ((int64_t)(M_pad / 32) * splits <= device_cu_count()) {
      hipExtLaunchKernelGGL(gelu_in ? k1_nvfp4_fused32<true> : k1_nvfp4_fused32<false>,
                            dim3(M_pad / 32, splits), dim3(64 * kK1RowsWaves), 0, st, ev0, ev1, 0, a);
    } else {
      const int P = k1_stream_workgroups(M_pad, splits);
      hipExtLaunchKernelGGL(gelu_in ? k1_nvfp4_stream<true> : k1_nvfp4_stream<false>, dim3(P, splits),
                            dim3(64 * kK1StreamWaves), 0, st, ev0, ev1, 0, a);
    }
  } else {
    if (gelu_in) return hipErrorInvalidValue;  // the GELU input is a fused-layout option only
    dim3 grid((M + 15) / 16);
    hipExtLaunchKernelGGL(k1_nvfp4_interchange, grid, dim3(512), 0, st, ev0, ev1, 0, x, M, K,
                          smooth, ldown, rank, g, out, scales, uact);
  }
  return hipGetLastError();
}

}  // namespace svdq
