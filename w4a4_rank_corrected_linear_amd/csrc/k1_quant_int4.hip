// K1, int4: smoothing + per-64-group amax + symmetric int4 quantization + packing
// + rank-r low-rank down projection, one pass over X.
//
// Layer definition: Diffusers docs "Nunchaku Lite", "Supported quantization types"
// (svdq_w4a4, int4, group 64, SVDQ low-rank correction), with the readings stated
// in svdq.h: xhat = bf16(x m), s = bf16(amax / 7), q = round-half-even(xhat / s)
// clamped to the int4 range [-8, 7], U = xhat @ lora_down^T (fp32 accumulation, not
// rounded).
//
// Two kernels share the quantizer below:
//  * k1_int4_fused / k1_int4_stream (the layer's own path) use the row-pair skeleton
//    of k1_rows32.h or the row-stream skeleton of k1_stream.h and write the GEMM
//    operand layout, scales [K/64][M_pad] (8-byte records by
//    group parity, see common.h) and partial U per k-split in the fragment layout;
//  * k1_int4_interchange (svdq_quantize_act) streams whole rows with register
//    prefetch and writes codes [M][K/2], scales [M][K/64] and U [M][r].
// In both, lane l holds half h = q % 2 of the 64-group g = k0 / 64 (q = l / 16): the
// amax is an in-lane max over 32 values and one cross-lane step (lane l ^ 16).  The
// same 32 values are one MFMA lane slot of the GEMM's A operand, so the fused layout
// is produced in registers by v_cvt_scalef32_2xpk16_fp6_f32.
#include "common.h"
#include "k1_common.h"
#include "k1_rows32.h"
#include "k1_stream.h"
#include "kernels.h"

namespace svdq {

typedef int v6i __attribute__((ext_vector_type(6)));

// Scale and clamped quotients of the lane's 32 values (all lanes must call it).
__device__ __forceinline__ uint32_t int4_quant32(const float (&xh)[32], float (&cq)[32]) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(xh[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 16));
  const uint32_t s_bits = f32_to_bf16_rne(amax / 7.0f);
  const float s = bf16_to_f32(s_bits);
  const bool tiny = (s > 0.f) && (s < 0x1p-125f);
  // q = round-half-even(xhat / s), decided exactly without a division.  r = v_rcp_f32(s)
  // is within one ulp of 1/s, so xhat r is within 7.02 * 2^-23 < 2^-20 of the quotient
  // Q.  y = fl(xhat r + 192) - 192 puts it on the grid of 2^-16 (the fma rounds once,
  // in the binade [128, 256); the subtraction is exact): at a tie Q = k + 1/2, itself
  // on the grid, y is exactly k + 1/2 (the error is below half a step), and a non-tie
  // quotient of two bf16 numbers with |Q| >= 1/4 lies more than 2^-12 from every
  // half-integer (Q = a / (b 2^d) with integers |a|, b < 256 and d <= 2), far beyond
  // the 2^-17 + 2^-20 that y can move, so y rounds to the integer Q rounds to.
  // With s = 0 every value is 0 and r = 0 gives y = 0.  A normal bf16 scale is within
  // 2^-9 relative of amax / 7, so |y| <= 7.014 and rounding to the nearest integer
  // already lands in [-7, 7]: the common path needs no clamp.  Scales below 2^-125
  // (subnormal bf16 scales lose precision, and 1/s may overflow) take the exact
  // division and the clamp to [-8, 7] (a subnormal scale can round far below amax / 7,
  // so quotients reach beyond 8 in magnitude); that case is tested once per wave so
  // the common path stays straight-line.
  const float rcp = s > 0.f ? __builtin_amdgcn_rcpf(s) : 0.f;
  if (!__any(tiny)) {
#pragma unroll
    for (int i = 0; i < 32; ++i) cq[i] = __builtin_fmaf(xh[i], rcp, 192.0f) - 192.0f;
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float y = tiny ? __fdiv_rn(xh[i], s) : __builtin_fmaf(xh[i], rcp, 192.0f) - 192.0f;
      cq[i] = __builtin_amdgcn_fmed3f(y, -8.0f, 7.0f);
    }
  }
  return s_bits;
}

struct QuantInt4Fused {
  static constexpr int kStores = 3;  // vector memory stores per call (wait counts)
  __device__ static void block(const K1Args& a, const float (&xh)[32], int row, int k0, int q) {
    float cq[32];
    const uint32_t s_bits = int4_quant32(xh, cq);
    const int g = k0 >> 6, h = q & 1;
    // E2M3 fields of value q/8: the converter divides by the scale 8 and rounds to
    // nearest even on the E2M3 grid, whose step is 1/8 up to 1.0, i.e. to q/8 (q = -8
    // is the normal -1.0; a clamped -7.5 sits midway between -0.875 and -1.0 and goes
    // to the even -1.0, as round-half-even takes -7.5 to -8).  Output field 2j
    // comes from src0[j] and field 2j+1 from src1[j]: even k go to src0 and odd k
    // to src1, so field f holds k = f.
    v16f ev, od;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      ev[j] = cq[2 * j];
      od[j] = cq[2 * j + 1];
    }
    // The converter reads its 32 sources over several passes while writing its six
    // results, so the results must not share registers with the sources: the builtin
    // lets the register allocator place them overlapping (seen at an offset of two
    // registers, which corrupts codes), the early-clobber output of the asm does not.
    v6i f6;
    asm volatile("v_cvt_scalef32_2xpk16_fp6_f32 %0, %1, %2, %3"
                 : "=&v"(f6) : "v"(ev), "v"(od), "s"(8.0f));
    // GEMM A-operand layout: chunk (row-block, group) of 1536 B; lane slot
    // h*32 + row%32 holds dwords 0-3 at slot*16 and dwords 4-5 at 1024 + slot*8.
    uint8_t* chunk = a.out + ((size_t)(row >> 5) * (a.K >> 6) + g) * 1536;
    const int slot = h * 32 + (row & 31);
    store_wt(chunk + slot * 16, make_uint4(f6[0], f6[1], f6[2], f6[3]));
    store_wt(chunk + 1024 + slot * 8, make_uint2(f6[4], f6[5]));
    if (h == 0)
      store_wt(static_cast<uint2*>(a.scales) + (size_t)g * a.M_pad + row, make_uint2(s_bits << (16 * (g & 1)), 0u));
  }
};

// Two skeletons of the same computation (identical codes, scales and U): 32 rows per
// workgroup when all workgroups fit in one round on the CUs; else resident workgroups,
// one per CU, that stream 16-row units and keep their k-split's operands loaded.
template <bool GELU_IN>
__global__ void __launch_bounds__(768, 1) k1_int4_fused(K1Args a) {
  k1_rows32<QuantInt4Fused, GELU_IN>(a);
}
template <bool GELU_IN>
__global__ void __launch_bounds__(768, 1) k1_int4_stream(K1Args a) {
  k1_stream<QuantInt4Fused, GELU_IN>(a);
}

// Interchange kernel: a 512-thread workgroup owns 16 rows; wave w takes the 128-wide
// k-blocks kb = w, w+8, ... and prefetches the next block's X, smoothing and
// lora_down operands into registers.  U is summed over the 8 waves in LDS.
struct K1Load {
  uint4 x[4];
  uint4 m[4];
  uint4 l[2][4];  // lora_down B operands for the rank slices (0..15, 16..31)
};

__global__ void __launch_bounds__(512)
k1_int4_interchange(const uint16_t* __restrict__ x, int M, int K,
                    const uint16_t* __restrict__ smooth, const uint16_t* __restrict__ ldown,
                    int rank, uint8_t* __restrict__ codes, uint16_t* __restrict__ scales,
                    float* __restrict__ uact) {
  __shared__ float ured[8][16][33];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;
  const int q = lane >> 4;
  const int row0 = blockIdx.x * 16;
  const int row = row0 + r;
  const bool valid = row < M;
  const int G = K >> 6;
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
    const int g = 2 * kb + (q >> 1);
    const int h = q & 1;

    // smoothing: xhat = bf16(x * m), one rounding of an exact product
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
        const v2bf pk = {(__bf16)p0, (__bf16)p1};  // v_cvt_pk_bf16_f32: round to nearest even
        const uint32_t w = __builtin_bit_cast(uint32_t, pk);
        xb[4 * c + p] = w;
        xh[8 * c + 2 * p] = __uint_as_float(w << 16);
        xh[8 * c + 2 * p + 1] = __uint_as_float(w & 0xFFFF0000u);
      }
    }
    float cq[32];
    const uint32_t s_bits = int4_quant32(xh, cq);

    {
      // Round to integer by adding 1.5 * 2^23: the low bits of the sum are the two's
      // complement code (-8 <= q <= 7); the add itself rounds half to even.
      uint32_t w[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        uint32_t acc = 0;
#pragma unroll
        for (int i = 7; i >= 0; --i) {
          const uint32_t b = __float_as_uint(cq[8 * d + i] + 12582912.0f);
          acc = (acc << 4) | (b & 0xFu);
        }
        w[d] = acc;
      }
      if (valid) {
        *reinterpret_cast<uint4*>(codes + ((size_t)row * K + k0) / 2) = make_uint4(w[0], w[1], w[2], w[3]);
        if (h == 0) scales[(size_t)row * G + g] = (uint16_t)s_bits;
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
    // C layout of the 16x16 MFMA: lane l holds column l%16, rows 4(l/16) + i.
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

// fused = false: interchange layout (codes [M][K/2], scales [M][K/64], U [M][r] fp32).
// fused = true : GEMM layout, M_pad rows (operand chunks of 1536 B per 32-row block
//                and group, scale records [K/64][M_pad], partial U per k-split in
//                the fragment layout of common.h, fp32);
//                rows >= M are zero.
hipError_t launch_k1_int4(bool fused, bool gelu_in, const uint16_t* x, int M, int K, const uint16_t* smooth,
                          const uint16_t* ldown, int rank, uint8_t* codes, void* scales,
                          float* uact, int M_pad, hipStream_t st, hipEvent_t ev0,
                          hipEvent_t ev1) {
  if (fused) {
    K1Args a{x, M, K, smooth, ldown, rank, codes, scales, uact, M_pad, 1.0f};
    const int splits = k1_splits(K);
    if ((int64_t)(M_pad / 32) * splits <= device_cu_count()) {
      hipExtLaunchKernelGGL(gelu_in ? k1_int4_fused<true> : k1_int4_fused<false>,
                            dim3(M_pad / 32, splits), dim3(64 * kK1RowsWaves), 0, st, ev0, ev1, 0, a);
    } else {
      const int P = k1_stream_workgroups(M_pad, splits);
      hipExtLaunchKernelGGL(gelu_in ? k1_int4_stream<true> : k1_int4_stream<false>, dim3(P, splits),
                            dim3(64 * kK1StreamWaves), 0, st, ev0, ev1, 0, a);
    }
  } else {
    if (gelu_in) return hipErrorInvalidValue;  // the GELU input is a fused-layout option only
    dim3 grid((M + 15) / 16);
    hipExtLaunchKernelGGL(k1_int4_interchange, grid, dim3(512), 0, st, ev0, ev1, 0, x, M, K,
                          smooth, ldown, rank, codes, static_cast<uint16_t*>(scales), uact);
  }
  return hipGetLastError();
}

}  // namespace svdq
