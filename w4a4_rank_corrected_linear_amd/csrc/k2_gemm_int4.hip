// K2, int4: the 4-bit x 4-bit residual GEMM with per-group rescale, fused with the
// rank-r up projection, the bias and the bf16 store.
//
//   Y[m,n] = bf16( sum_g sx[m,g] sw[n,g] P_g[m,n] + sum_j U[m,j] L2t[n,j] + b[n] ),
//   P_g    = sum_{k in g} qx[m,k] qw[n,k]   (exact integers)
//
// (Diffusers docs "Nunchaku Lite", "Supported quantization types": svdq_w4a4 int4
// group 64 with the SVDQ low-rank correction.)
//
// Per 32x32 output block and 64-group the wave issues
//   D = v_mfma_scale_f32_32x32x64_f8f6f4(A_g, B_g)  E2M3 codes, block scales 2^3:
//                                                  D = P_g exactly, in fp32
//   S = v_mfma_f32_32x32x16_bf16(sx, sw)            only k = 0 non-zero: the exact
//                                                  outer product sx[m] sw[n]
//   acc = fma(S, D, acc)                             the only VALU op per element
// so the matrix cores do both the integer dot products and the scale products and
// the vector ALU does one fused multiply-add per output element and group.
//
// Tiling: 256 threads (2 x 2 waves), workgroup tile 128 x BN, wave tile 64 x BN/2
// (2 x BN/64 blocks of 32 x 32).  Two 64-groups per stage, double-buffered in LDS:
// operands arrive from HBM/L2 in the compact 4-bit layout (common.h), are expanded
// to MFMA E2M3 dwords once per workgroup and stored as 24-byte lane slots, so each
// wave reads a fragment as 64 consecutive slots.
#include "common.h"
#include "kernels.h"

namespace svdq {

template <int BN>
__global__ void __launch_bounds__(256, 2)
k2_gemm_int4(const uint4* __restrict__ A, const uint16_t* __restrict__ sA,
             const uint16_t* __restrict__ U, const uint4* __restrict__ B,
             const uint16_t* __restrict__ sB, const uint16_t* __restrict__ L2t,
             const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y,
             int M, int N, int K, int M_pad, int rank) {
  constexpr int BM = 128;
  constexpr int WN = BN / 64;         // 32-col blocks per wave
  constexpr int RB = BM / 32;         // row-blocks per tile
  constexpr int CB = BN / 32;         // col-blocks per tile
  constexpr int A_LD = RB * 2 * 64 / 256;
  constexpr int B_LD = CB * 2 * 64 / 256;
  constexpr int SB_PER_G = BN / 8;    // uint4 of B scales per group
  __shared__ uint32_t ldsA[2][RB * 2 * 64 * 6];
  __shared__ uint32_t ldsB[2][CB * 2 * 64 * 6];
  __shared__ __attribute__((aligned(16))) uint16_t ldsSA[2][2][BM];
  __shared__ __attribute__((aligned(16))) uint16_t ldsSB[2][2][BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int col0 = blockIdx.x * BN;
  const int row0 = blockIdx.y * BM;
  const int rb0 = row0 >> 5, cb0 = col0 >> 5;
  const int G = K >> 6;
  const int S = G >> 1;

  uint4 ra[A_LD], rbv[B_LD], rs;

  auto gload = [&](int s) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int idx = tid + 256 * i;
      const int c = idx >> 6, within = idx & 63;
      ra[i] = A[((size_t)(rb0 + (c >> 1)) * G + 2 * s + (c & 1)) * 64 + within];
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int idx = tid + 256 * i;
      const int c = idx >> 6, within = idx & 63;
      rbv[i] = B[((size_t)(cb0 + (c >> 1)) * G + 2 * s + (c & 1)) * 64 + within];
    }
    if (tid < 32) {
      const int gl = tid >> 4, w = tid & 15;
      rs = *reinterpret_cast<const uint4*>(sA + (size_t)(2 * s + gl) * M_pad + row0 + 8 * w);
    } else if (tid >= 64 && tid < 64 + 2 * SB_PER_G) {
      const int t = tid - 64;
      const int gl = t / SB_PER_G, w = t % SB_PER_G;
      rs = *reinterpret_cast<const uint4*>(sB + (size_t)(2 * s + gl) * N + col0 + 8 * w);
    }
  };

  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int idx = tid + 256 * i;
      const int c = idx >> 6, within = idx & 63;
      const int slot = ((c & 1) * RB + (c >> 1)) * 64 + within;
      uint32_t o[6];
      fp6_expand(ra[i].x, ra[i].y, o[0], o[1], o[2]);
      fp6_expand(ra[i].z, ra[i].w, o[3], o[4], o[5]);
      uint2* dst = reinterpret_cast<uint2*>(&ldsA[buf][slot * 6]);
      dst[0] = make_uint2(o[0], o[1]);
      dst[1] = make_uint2(o[2], o[3]);
      dst[2] = make_uint2(o[4], o[5]);
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int idx = tid + 256 * i;
      const int c = idx >> 6, within = idx & 63;
      const int slot = ((c & 1) * CB + (c >> 1)) * 64 + within;
      uint32_t o[6];
      fp6_expand(rbv[i].x, rbv[i].y, o[0], o[1], o[2]);
      fp6_expand(rbv[i].z, rbv[i].w, o[3], o[4], o[5]);
      uint2* dst = reinterpret_cast<uint2*>(&ldsB[buf][slot * 6]);
      dst[0] = make_uint2(o[0], o[1]);
      dst[1] = make_uint2(o[2], o[3]);
      dst[2] = make_uint2(o[4], o[5]);
    }
    if (tid < 32) {
      const int gl = tid >> 4, w = tid & 15;
      *reinterpret_cast<uint4*>(&ldsSA[buf][gl][8 * w]) = rs;
    } else if (tid >= 64 && tid < 64 + 2 * SB_PER_G) {
      const int t = tid - 64;
      const int gl = t / SB_PER_G, w = t % SB_PER_G;
      *reinterpret_cast<uint4*>(&ldsSB[buf][gl][8 * w]) = rs;
    }
  };

  v16f acc[2][WN];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const v16f zero = {};
  gload(0);
  lstore(0);
  __syncthreads();

  for (int s = 0; s < S; ++s) {
    const int buf = s & 1;
    if (s + 1 < S) gload(s + 1);
    {
      // Fragments of both groups of the stage, straight from LDS.
      v8i af[2][2], bfr[2][WN];
      uint32_t sxv[2][2], swv[2][WN];
#pragma unroll
      for (int gl = 0; gl < 2; ++gl) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const uint2* src = reinterpret_cast<const uint2*>(
              &ldsA[buf][((gl * RB + wm * 2 + i) * 64 + lane) * 6]);
          const uint2 p0 = src[0], p1 = src[1], p2 = src[2];
          af[gl][i] = v8i{(int)p0.x, (int)p0.y, (int)p1.x, (int)p1.y, (int)p2.x, (int)p2.y, 0, 0};
          const uint32_t sl = ldsSA[buf][gl][wm * 64 + 32 * i + (lane & 31)];
          sxv[gl][i] = lane < 32 ? sl : 0u;
        }
#pragma unroll
        for (int j = 0; j < WN; ++j) {
          const uint2* src = reinterpret_cast<const uint2*>(
              &ldsB[buf][((gl * CB + wn * WN + j) * 64 + lane) * 6]);
          const uint2 p0 = src[0], p1 = src[1], p2 = src[2];
          bfr[gl][j] = v8i{(int)p0.x, (int)p0.y, (int)p1.x, (int)p1.y, (int)p2.x, (int)p2.y, 0, 0};
          const uint32_t sl = ldsSB[buf][gl][(wn * WN + j) * 32 + (lane & 31)];
          swv[gl][j] = lane < 32 ? sl : 0u;
        }
      }
      // Two-deep software pipeline over the 2 * 2 * WN (group, block) steps: the
      // MFMAs of step b+1 are issued before the rescale FMAs of step b.  The empty
      // volatile asm statements are ordering points (volatile asm keeps program
      // order): step b+1's operands pass one after step b-1's accumulator is final,
      // so at most two steps' MFMA results are live.
      constexpr int NB = 2 * 2 * WN;
      v16f dq[2], sq[2];
      auto issue = [&](int b, int slot) {
        const int gl = b / (2 * WN), i = (b / WN) % 2, j = b % WN;
        uint32_t sx = sxv[gl][i], sw = swv[gl][j];
        int a0 = af[gl][i][0];
        asm volatile("" : "+v"(sx), "+v"(sw), "+v"(a0));
        v8i a = af[gl][i];
        a[0] = a0;
        dq[slot] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bfr[gl][j], zero, 2, 2, 0, 130,
                                                                   0, 130);
        const v8s so = v8s{(short)sx, 0, 0, 0, 0, 0, 0, 0};
        const v8s wo = v8s{(short)sw, 0, 0, 0, 0, 0, 0, 0};
        sq[slot] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, so),
                                                           __builtin_bit_cast(v8bf, wo), zero, 0, 0, 0);
      };
      issue(0, 0);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if (b + 1 < NB) issue(b + 1, (b + 1) & 1);
        const int i = (b / WN) % 2, j = b % WN;
        v16f& a = acc[i][j];
#pragma unroll
        for (int e = 0; e < 16; ++e) a[e] = __builtin_fmaf(sq[b & 1][e], dq[b & 1][e], a[e]);
        asm volatile("" : "+v"(a));
      }
    }
    if (s + 1 < S) lstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: acc += U @ L2t^T on the bf16 MFMA, + bias, round to bf16, store.
  const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rowb = row0 + wm * 64 + 32 * i;
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int colb = col0 + (wn * WN + j) * 32;
      v16f c = acc[i][j];
      for (int kk = 0; kk < rank; kk += 16) {
        const uint4 ua = *reinterpret_cast<const uint4*>(U + (size_t)(rowb + lr) * rank + kk + 8 * lh);
        const uint4 lb = *reinterpret_cast<const uint4*>(L2t + (size_t)(colb + lr) * rank + kk + 8 * lh);
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, ua),
                                                    __builtin_bit_cast(v8bf, lb), c, 0, 0, 0);
      }
      const float bv = bias ? bf16_to_f32(bias[colb + lr]) : 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = rowb + 8 * (e >> 2) + 4 * lh + (e & 3);
        if (row < M) Y[(size_t)row * N + colb + lr] = (uint16_t)f32_to_bf16_rne(c[e] + bv);
      }
    }
  }
}

hipError_t launch_k2_int4(const uint8_t* A, const uint16_t* sA, const uint16_t* U,
                          const uint8_t* B, const uint16_t* sB, const uint16_t* L2t,
                          const uint16_t* bias, uint16_t* Y, int M, int N, int K, int M_pad,
                          int rank, hipStream_t st) {
  const int BM = 128;
  dim3 grid(N / 128, M_pad / BM);
  hipLaunchKernelGGL(k2_gemm_int4<128>, grid, dim3(256), 0, st, reinterpret_cast<const uint4*>(A),
                     sA, U, reinterpret_cast<const uint4*>(B), sB, L2t, bias, Y, M, N, K, M_pad, rank);
  return hipGetLastError();
}

}  // namespace svdq
