// K2, int4: the 4-bit x 4-bit residual GEMM with per-group rescale, fused with the
// rank-r up projection, the bias and the bf16 store.
//
//   Y[m,n] = bf16( sum_g sx[m,g] sw[n,g] P_g[m,n] + sum_j U[m,j] L2t[n,j] + b[n] ),
//   P_g    = sum_{k in g} qx[m,k] qw[n,k]   (exact integers)
//
// (Diffusers docs "Nunchaku Lite", "Supported quantization types": svdq_w4a4 int4
// group 64 with the SVDQ low-rank correction.)
//
// Per 32x32 output block and 64-group a wave issues
//   D = v_mfma_scale_f32_32x32x64_f8f6f4(A_g, B_g)  E2M3 codes, block scales 2^3:
//                                                  D = P_g exactly, in fp32
//   S = v_mfma_f32_32x32x8_bf16(sx, sw)             only k = 0 non-zero: the exact
//                                                  outer product sx[m] sw[n]
//   acc = fma(S, D, acc)                             one VALU op per element and group
// and the schedule alternates one MFMA with eight FMAs, so the matrix core runs the
// next block's MFMAs under the current block's rescale.
//
// Tiling: 256 threads (2 x 2 waves), workgroup tile 128 x BN, wave tile 64 x BN/2
// (2 x BN/64 blocks of 32 x 32), two workgroups per CU.  A stage is two 64-groups.
// Operands are prefetched two stages ahead:
//   A  arrives from K1 already as MFMA E2M3 lane slots (1536 B per 32-row block and
//      group: 64 x 16 B of dwords 0-3, then 64 x 8 B of dwords 4-5); the two groups
//      of one row-block are 3 KiB contiguous, copied by LDS DMA (global_load_lds,
//      16 B per lane) into one of three LDS buffers;
//   B  (weights, compact 4-bit layout of common.h) and the per-group scales go
//      through registers (two register sets) and are expanded into lane slots and
//      written to one of two LDS buffers one stage before use.
#include "common.h"
#include "kernels.h"

namespace svdq {

typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));

template <int BN>
__global__ void __launch_bounds__(256, 2)
k2_gemm_int4(const uint8_t* __restrict__ A, const uint16_t* __restrict__ sA,
             const float* __restrict__ U, int nsplit, const uint8_t* __restrict__ B,
             const uint16_t* __restrict__ sB, const uint16_t* __restrict__ L2t,
             const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y,
             int M, int N, int K, int M_pad, int rank) {
  constexpr int BM = 128;
  constexpr int WN = BN / 64;          // 32-col blocks per wave
  constexpr int RB = BM / 32;          // row-blocks per tile
  constexpr int CB = BN / 32;          // col-blocks per tile
  constexpr int B_DEC = CB * 2 * 64 / 256;  // 16-byte compact chunks decoded per thread
  static_assert(CB * 2 * 64 % 256 == 0, "tile/thread mismatch");
  static_assert(RB == 4, "one row-block per wave for the A copy");

  // Double-buffered stage data, one LDS object per buffer: every access below names
  // its buffer statically, which lets loads from one buffer proceed while the DMA
  // into the other is still in flight.
  //   A   [row-block][group][1536 B] E2M3 lane slots (DMA)
  //   Br  [col-block][group][1024 B] compact weights (DMA)
  //   S*  [group][rows or cols] bf16 scales (DMA)
  //   Bd  [group][col-block][1536 B] expanded weights (written by the decode step)
  __shared__ __attribute__((aligned(16))) uint32_t A0[RB * 2 * 384], A1[RB * 2 * 384];
  __shared__ __attribute__((aligned(16))) uint32_t Br0[CB * 2 * 256], Br1[CB * 2 * 256];
  __shared__ __attribute__((aligned(16))) uint16_t SA0[2 * BM], SA1[2 * BM];
  __shared__ __attribute__((aligned(16))) uint16_t SB0[2 * BN], SB1[2 * BN];
  __shared__ __attribute__((aligned(16))) uint32_t Bd[CB * 2 * 384];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int col0 = blockIdx.x * BN;
  const int row0 = blockIdx.y * BM;
  const int rb0 = row0 >> 5, cb0 = col0 >> 5;
  const int G = K >> 6;
  const int S = G >> 1;

  // Copies of stage s into one buffer set.  global_load_lds writes 16 B per active
  // lane at dst + 16 * lane.
  auto dma = [&](int s, uint32_t* Ab, uint32_t* Brb, uint16_t* SAb, uint16_t* SBb) {
    {  // A: wave w copies row-block w, groups 2s and 2s+1 (3 KiB contiguous)
      const uint8_t* src = A + ((size_t)(rb0 + wave) * G + 2 * s) * 1536 + lane * 16;
      uint32_t* dst = Ab + wave * 2 * 384;
#pragma unroll
      for (int t = 0; t < 3; ++t)
        __builtin_amdgcn_global_load_lds(src + t * 1024, dst + t * 256, 16, 0, 0);
    }
    // compact B: col-block cb, groups 2s and 2s+1 are 2 KiB contiguous
#pragma unroll
    for (int d = wave; d < CB * 2; d += 4) {
      const int cb = d >> 1, part = d & 1;
      const uint8_t* src = B + ((size_t)(cb0 + cb) * G + 2 * s + part) * 1024 + lane * 16;
      __builtin_amdgcn_global_load_lds(src, Brb + d * 256, 16, 0, 0);
    }
    if (wave == 0 && lane < 32) {          // row scales of groups 2s, 2s+1
      const int gl = lane >> 4, w = lane & 15;
      __builtin_amdgcn_global_load_lds(sA + (size_t)(2 * s + gl) * M_pad + row0 + 8 * w, SAb, 16,
                                       0, 0);
    }
    if (wave == 1 && lane < BN / 4) {      // column scales of groups 2s, 2s+1
      const int gl = lane / (BN / 8), w = lane % (BN / 8);
      __builtin_amdgcn_global_load_lds(sB + (size_t)(2 * s + gl) * N + col0 + 8 * w, SBb, 16, 0,
                                       0);
    }
  };

  // Expand the compact weights of one stage into MFMA lane slots.
  auto decode = [&](const uint32_t* Brb) {
#pragma unroll
    for (int i = 0; i < B_DEC; ++i) {
      const int idx = tid + 256 * i;
      const int c = idx >> 6, within = idx & 63;   // c = 2 * col-block + group
      const uint4 v = *reinterpret_cast<const uint4*>(Brb + c * 256 + within * 4);
      uint32_t o[6];
      fp6_expand(v.x, v.y, o[0], o[1], o[2]);
      fp6_expand(v.z, v.w, o[3], o[4], o[5]);
      uint32_t* base = Bd + ((c & 1) * CB + (c >> 1)) * 384;
      *reinterpret_cast<uint4*>(base + within * 4) = make_uint4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<uint2*>(base + 256 + within * 2) = make_uint2(o[4], o[5]);
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
  const int e8 = 130;  // E8M0 2^3 per operand: E2M3 code q/8 -> q
  const bool lo_half = lane < 32;

  auto compute = [&](const uint32_t* Ab, const uint16_t* SAb, const uint16_t* SBb) {
#pragma unroll
    for (int gl = 0; gl < 2; ++gl) {
      v8i af[2], bfr[WN];
      v2i sa[2], sb[WN];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t* base = Ab + ((wm * 2 + i) * 2 + gl) * 384;
        const v4i lo = *reinterpret_cast<const v4i*>(base + lane * 4);
        const v2i hi = *reinterpret_cast<const v2i*>(base + 256 + lane * 2);
        af[i] = __builtin_shufflevector(lo, __builtin_shufflevector(hi, hi, 0, 1, -1, -1), 0, 1, 2, 3,
                                        4, 5, -1, -1);
        const int sv = SAb[gl * BM + wm * 64 + 32 * i + (lane & 31)];
        sa[i] = v2i{lo_half ? sv : 0, 0};
      }
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const uint32_t* base = Bd + (gl * CB + wn * WN + j) * 384;
        const v4i lo = *reinterpret_cast<const v4i*>(base + lane * 4);
        const v2i hi = *reinterpret_cast<const v2i*>(base + 256 + lane * 2);
        bfr[j] = __builtin_shufflevector(lo, __builtin_shufflevector(hi, hi, 0, 1, -1, -1), 0, 1, 2,
                                         3, 4, 5, -1, -1);
        const int sv = SBb[gl * BN + (wn * WN + j) * 32 + (lane & 31)];
        sb[j] = v2i{lo_half ? sv : 0, 0};
      }
      // Block steps b = (i, j).  Empty volatile asm statements are ordering points
      // (volatile asm keeps program order) on registers that are used anyway: the
      // operands of step b's MFMAs pass one just before them, and each half of step
      // b's accumulator passes one after its FMAs, so no MFMA is hoisted far ahead
      // of its step and at most two steps' MFMA results are live.
      int e8r = e8;
#pragma unroll
      for (int b = 0; b < 2 * WN; ++b) {
        const int i = b / WN, j = b % WN;
        asm volatile("" : "+v"(e8r), "+v"(sa[i]), "+v"(sb[j]));
        const v16f d = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bfr[j], zero, 2, 2, 0,
                                                                        e8r, 0, e8r);
        const v16f sc = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(
            __builtin_bit_cast(v4bf, sa[i]), __builtin_bit_cast(v4bf, sb[j]), zero, 0, 0, 0);
        v16f& a = acc[i][j];
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = __builtin_fmaf(sc[e], d[e], a[e]);
        asm volatile("" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]),
                     "+v"(a[6]), "+v"(a[7]));
#pragma unroll
        for (int e = 8; e < 16; ++e) a[e] = __builtin_fmaf(sc[e], d[e], a[e]);
        asm volatile("" : "+v"(a[8]), "+v"(a[9]), "+v"(a[10]), "+v"(a[11]), "+v"(a[12]),
                     "+v"(a[13]), "+v"(a[14]), "+v"(a[15]));
      }
    }
  };

  // Workgroup barrier after this wave's memory operations are done.  The compiler
  // completes every outstanding vector-memory operation before an s_barrier, so each
  // stage issues its successor's DMA after its last barrier: the copy then runs
  // under the whole compute phase and is awaited at the next stage's first barrier.
  auto sync_all = [&]() {
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
  };

  // Stage s uses buffer set s % 2: wait for its DMA and for the end of the previous
  // compute, expand its weights, synchronize, start the DMA of stage s+1 into the
  // other set, compute.
  dma(0, A0, Br0, SA0, SB0);
  for (int s = 0; s < S; s += 2) {
    sync_all();
    decode(Br0);
    sync_all();
    if (s + 1 < S) dma(s + 1, A1, Br1, SA1, SB1);
    compute(A0, SA0, SB0);
    if (s + 1 < S) {
      sync_all();
      decode(Br1);
      sync_all();
      if (s + 2 < S) dma(s + 2, A0, Br0, SA0, SB0);
      compute(A1, SA1, SB1);
    }
  }
  sync_all();

  // Epilogue: acc += U @ L2t^T on the bf16 MFMA, + bias, round to bf16; each 32x32
  // block goes through a per-wave LDS tile (rows of 80 B) so Y is written with
  // 16-byte stores.
  const int lr = lane & 31, lh = lane >> 5;
  uint16_t* tile = reinterpret_cast<uint16_t*>(A0) + wave * (32 * 40);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rowb = row0 + wm * 64 + 32 * i;
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int colb = col0 + (wn * WN + j) * 32;
      v16f c = acc[i][j];
      for (int kk = 0; kk < rank; kk += 16) {
        // U is fp32: split into bf16 hi + lo (u - hi is exact in fp32), two MFMAs;
        // what is dropped is below 2^-17 |u|.
        // U = sum of the quantizer's k-split partials, added in order
        float uf[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int sp = 0; sp < nsplit; ++sp) {
          const float* up = U + ((size_t)sp * M_pad + rowb + lr) * rank + kk + 8 * lh;
          const float4 u0 = *reinterpret_cast<const float4*>(up);
          const float4 u1 = *reinterpret_cast<const float4*>(up + 4);
          uf[0] += u0.x; uf[1] += u0.y; uf[2] += u0.z; uf[3] += u0.w;
          uf[4] += u1.x; uf[5] += u1.y; uf[6] += u1.z; uf[7] += u1.w;
        }
        v8bf hi, lo;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          hi[t] = (__bf16)uf[t];
          lo[t] = (__bf16)(uf[t] - (float)hi[t]);
        }
        const uint4 lb = *reinterpret_cast<const uint4*>(L2t + (size_t)(colb + lr) * rank + kk + 8 * lh);
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hi, __builtin_bit_cast(v8bf, lb), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lo, __builtin_bit_cast(v8bf, lb), c, 0, 0, 0);
      }
      const float bv = bias ? bf16_to_f32(bias[colb + lr]) : 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int rin = 8 * (e >> 2) + 4 * lh + (e & 3);
        tile[rin * 40 + lr] = (uint16_t)f32_to_bf16_rne(c[e] + bv);
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

hipError_t launch_k2_int4(const uint8_t* A, const uint16_t* sA, const float* U, int nsplit,
                          const uint8_t* B, const uint16_t* sB, const uint16_t* L2t,
                          const uint16_t* bias, uint16_t* Y, int M, int N, int K, int M_pad,
                          int rank, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  const int BM = 128;
  if (N % 192 == 0) {
    dim3 grid(N / 192, M_pad / BM);
    hipExtLaunchKernelGGL(k2_gemm_int4<192>, grid, dim3(256), 0, st, ev0, ev1, 0, A, sA, U, nsplit, B, sB,
                          L2t, bias, Y, M, N, K, M_pad, rank);
  } else {
    dim3 grid(N / 128, M_pad / BM);
    hipExtLaunchKernelGGL(k2_gemm_int4<128>, grid, dim3(256), 0, st, ev0, ev1, 0, A, sA, U, nsplit, B, sB,
                          L2t, bias, Y, M, N, K, M_pad, rank);
  }
  return hipGetLastError();
}

}  // namespace svdq
