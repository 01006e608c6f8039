// K2, nvfp4: the 4-bit x 4-bit GEMM of the NVFP4 layer on exactly dequantized bf16
// operands, fused with the per-tensor scale, the rank-r up projection, the bias and
// the bf16 store.
//
//   Y[m,n] = bf16( g * sum_k A'[m,k] B'[n,k] + sum_j U[m,j] L2t[n,j] + b[n] ),
//   A' = e2m1(x code) * s_x,  B' = e2m1(w code) * s_w   (exact in bf16), g = g_x g_w
//
// (Diffusers docs "Nunchaku Lite", "Supported quantization types": svdq_w4a4 nvfp4,
// group 16 with E4M3 block scales, SVDQ low-rank correction.)  CDNA4's scaled MFMAs
// take power-of-two scales per 32 values, not E4M3 scales per 16, so the block
// scales are folded into the operands instead: every product A' B' is exact and the
// sum over k accumulates in the fp32 MFMA accumulator, with no per-block rescale.
//
// Tiling: 256 threads (2 x 2 waves), tile 128 x 128, wave tile 64 x 64 (2 x 2 blocks
// of v_mfma_f32_32x32x16_bf16), two workgroups per CU.  A stage is 64 values of k:
// both 128 x 64 operand tiles (16 KiB each) are copied into LDS by global_load_lds
// (16 B per lane) into one of two buffers while the other is consumed.  LDS holds a
// tile as 16-byte units u = row * 8 + (c ^ (row & 7)), c = k / 8 within the stage: the
// XOR swizzle puts the eight rows that one MFMA operand read touches at once in
// distinct bank groups; it is applied by choosing each lane's source address.
//
// The accumulator blocks are held transposed (the weight fragment is the MFMA's first
// operand): lane l % 32 is the output row, its 16 elements are columns
// 8 q + 4 (l / 32) + p of the block (element 4 q + p).  Epilogues: + bias and the bf16
// store; the same with the exact GELU before the rounding; or the fused QKV epilogue
// (per-head RMSNorm over the 128 columns of a tile, the channel weights and the rotary
// turn of adjacent column pairs, on the Q and K tiles), as in the int4 GEMM.
#include "common.h"
#include "kernels.h"

namespace svdq {

template <int EPI>
__global__ void __launch_bounds__(256, 2)
k2_gemm_bf16(const uint16_t* __restrict__ A, const float* __restrict__ U, int nsplit,
             const uint16_t* __restrict__ B, const uint16_t* __restrict__ L2t,
             const uint16_t* __restrict__ bias, float g, uint16_t* __restrict__ Y, int M, int N,
             int K, int M_pad, int rank, QkEpi qk) {
  constexpr int BM = 128, BN = 128;
  constexpr int TILE = 128 * 64;  // bf16 elements of one operand tile per stage
  __shared__ __attribute__((aligned(16))) uint16_t A0[TILE], A1[TILE], B0[TILE], B1[TILE];
  __shared__ float red[EPI == kEpiQkNormRope ? 256 : 1];  // per-row sums of squares, by wave

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_n = N / BN;
  const int tn = blockIdx.x % tiles_n, tm = blockIdx.x / tiles_n;
  const int row0 = tm * BM, col0 = tn * BN;
  const int S = K >> 6;

  // Each wave copies 4 KiB of each operand tile per stage: 4 DMA instructions, lane i
  // of instruction t filling unit u = 64 (4 wave + t) + i.
  auto dma = [&](int s, uint16_t* Ab, uint16_t* Bb) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int u = 64 * (4 * wave + t) + lane;
      const int r = u >> 3, c = (u & 7) ^ (r & 7);
      const size_t off = (size_t)r * K + 64 * s + 8 * c;
      __builtin_amdgcn_global_load_lds(A + (size_t)row0 * K + off, Ab + 8 * 64 * (4 * wave + t), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(B + (size_t)col0 * K + off, Bb + 8 * 64 * (4 * wave + t), 16, 0, 0);
    }
  };

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // Operand fragment of MFMA k-step kk: lane l reads row (l % 32) of the 32-row
  // block, values k = 16 kk + 8 (l / 32) + [0, 8).
  auto frag = [&](const uint16_t* T, int row, int kk) {
    const int c = 2 * kk + (lane >> 5);
    const int u = row * 8 + (c ^ (row & 7));
    return *reinterpret_cast<const v8bf*>(T + 8 * u);
  };

  auto compute = [&](const uint16_t* Ab, const uint16_t* Bb) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      v8bf a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = frag(Ab, wm * 64 + 32 * i + (lane & 31), kk);
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = frag(Bb, wn * 64 + 32 * j + (lane & 31), kk);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
    }
  };

  auto sync_all = [&]() {
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
  };

  dma(0, A0, B0);
  for (int s = 0; s < S; s += 2) {
    sync_all();
    if (s + 1 < S) dma(s + 1, A1, B1);
    compute(A0, B0);
    if (s + 1 < S) {
      sync_all();
      if (s + 2 < S) dma(s + 2, A0, B0);
      compute(A1, B1);
    }
  }
  sync_all();

  // Epilogue: acc * g, + U @ L2t^T (U split into three bf16 terms), + bias, then (QKV
  // mode) the per-head norm and rotation, and bf16 stores through a per-wave LDS tile
  // (rows of 80 B).
  const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rowb = row0 + wm * 64 + 32 * i;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int colb = col0 + wn * 64 + 32 * j;
      v16f c = acc[i][j];
#pragma unroll
      for (int e = 0; e < 16; ++e) c[e] *= g;
      for (int kk = 0; kk < rank; kk += 16) {
        // U = sum of the quantizer's k-split partials, added in order
        float uf[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int sp = 0; sp < nsplit; ++sp) {
          // fragment layout: ranks 0-3 of the lane's eight, then 4-7 one KiB further
          const float* up = U + u_frag_index(sp, rowb + lr, kk + 8 * lh, M_pad, rank);
          const float4 u0 = *reinterpret_cast<const float4*>(up);
          const float4 u1 = *reinterpret_cast<const float4*>(up + 256);
          uf[0] += u0.x; uf[1] += u0.y; uf[2] += u0.z; uf[3] += u0.w;
          uf[4] += u1.x; uf[5] += u1.y; uf[6] += u1.z; uf[7] += u1.w;
        }
        v8bf hi, mid, lo;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const Bf16x3 s3 = split3_bf16(uf[t]);
          hi[t] = s3.h;
          mid[t] = s3.m;
          lo[t] = s3.l;
        }
        const uint4 lb = *reinterpret_cast<const uint4*>(L2t + (size_t)(colb + lr) * rank + kk + 8 * lh);
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, lb), hi, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, lb), mid, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, lb), lo, c, 0, 0, 0);
      }
      if (bias) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint2 b2 = *reinterpret_cast<const uint2*>(bias + colb + 8 * q + 4 * lh);
          c[4 * q + 0] += __uint_as_float(b2.x << 16);
          c[4 * q + 1] += __uint_as_float(b2.x & 0xFFFF0000u);
          c[4 * q + 2] += __uint_as_float(b2.y << 16);
          c[4 * q + 3] += __uint_as_float(b2.y & 0xFFFF0000u);
        }
      }
      acc[i][j] = c;
    }
  }
  if constexpr (EPI == kEpiQkNormRope) {
    // Q and K tiles (the first two thirds of the columns) are one head each: the lane
    // pair (l, l + 32) holds one row's 32 + 32 columns of the wave, the partner wave
    // (wave ^ 1, same rows) the other 64.  Tile-uniform branch around the barrier.
    const int third = N / 3;
    if (col0 < 2 * third) {
      const uint16_t* nw = col0 < third ? qk.norm_q : qk.norm_k;
      float ss[2] = {0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) ss[i] = fmaf(acc[i][j][e], acc[i][j][e], ss[i]);
#pragma unroll
      for (int i = 0; i < 2; ++i) ss[i] += __shfl_xor(ss[i], 32);
      sync_all();  // every wave is past its LDS operand reads before red is written
      if (lh == 0) {
        red[wave * 64 + lr] = ss[0];
        red[wave * 64 + 32 + lr] = ss[1];
      }
      sync_all();
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float inv = 1.0f / sqrtf((ss[i] + red[(wave ^ 1) * 64 + 32 * i + lr]) * (1.0f / 128.0f) +
                                       qk.eps);
        const int row = min(row0 + wm * 64 + 32 * i + lr, M - 1);  // pad rows are not stored
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int c = wn * 64 + 32 * j + 8 * q + 4 * lh;  // channel of element 4q
            const uint2 w2 = *reinterpret_cast<const uint2*>(nw + c);
            const float w[4] = {__uint_as_float(w2.x << 16), __uint_as_float(w2.x & 0xFFFF0000u),
                                __uint_as_float(w2.y << 16), __uint_as_float(w2.y & 0xFFFF0000u)};
            const float4 cs = *reinterpret_cast<const float4*>(qk.rope + (size_t)row * 128 + c);
            float n[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) n[p] = acc[i][j][4 * q + p] * inv * w[p];
            acc[i][j][4 * q + 0] = n[0] * cs.x - n[1] * cs.y;
            acc[i][j][4 * q + 1] = n[1] * cs.x + n[0] * cs.y;
            acc[i][j][4 * q + 2] = n[2] * cs.z - n[3] * cs.w;
            acc[i][j][4 * q + 3] = n[3] * cs.z + n[2] * cs.w;
          }
      }
    }
  }
  uint16_t* tile = A0 + wave * (32 * 40);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rowb = row0 + wm * 64 + 32 * i;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int colb = col0 + wn * 64 + 32 * j;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t h[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float v = acc[i][j][4 * q + p];
          h[p] = f32_to_bf16_rne(EPI == kEpiGelu ? gelu_f32(v) : v);
        }
        *reinterpret_cast<uint2*>(tile + lr * 40 + 8 * q + 4 * lh) =
            make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int qd = lane + 64 * t;
        const int rin = qd >> 2, ch = qd & 3;
        const uint4 v = *reinterpret_cast<const uint4*>(tile + rin * 40 + ch * 8);
        const int row = rowb + rin;
        if (row < M) *reinterpret_cast<uint4*>(Y + (size_t)row * N + colb + ch * 8) = v;
      }
    }
  }
}

hipError_t launch_k2_bf16(const uint16_t* A, const float* U, int nsplit, const uint16_t* B,
                          const uint16_t* L2t, const uint16_t* bias, float g, uint16_t* Y, int M,
                          int N, int K, int M_pad, int rank, int epi, const QkEpi& qk,
                          hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  if (M_pad % 128 != 0 || N % 128 != 0 || K % 64 != 0) return hipErrorInvalidValue;
  if (epi == kEpiQkNormRope && (N % 384 != 0 || !qk.norm_q || !qk.norm_k || !qk.rope))
    return hipErrorInvalidValue;
  dim3 grid((N / 128) * (M_pad / 128));
  auto k = epi == kEpiQkNormRope ? k2_gemm_bf16<kEpiQkNormRope>
           : epi == kEpiGelu     ? k2_gemm_bf16<kEpiGelu>
                                 : k2_gemm_bf16<kEpiPlain>;
  hipExtLaunchKernelGGL(k, grid, dim3(256), 0, st, ev0, ev1, 0, A, U, nsplit, B, L2t, bias, g, Y,
                        M, N, K, M_pad, rank, qk);
  return hipGetLastError();
}

}  // namespace svdq
