// K2, nvfp4: the 4-bit x 4-bit GEMM of the NVFP4 layer, fused with the per-tensor
// scale, the rank-r up projection, the bias and the bf16 store.
//
//   Y[m,n] = bf16( g * sum_k A'[m,k] B'[n,k] + sum_j U[m,j] L2t[n,j] + b[n] ),
//   A' = e2m1(x code) * s_x,  B' = e2m1(w code) * s_w,  g = g_x g_w
//
// (Diffusers docs "Nunchaku Lite", "Supported quantization types": svdq_w4a4 nvfp4,
// group 16 with E4M3 block scales, SVDQ low-rank correction.)
//
// Both operands stay 4-bit in memory: E2M1 codes in the FP4 lane-slot layout of
// common.h and the block scales as fp16 values.  CDNA4's scaled MFMAs take
// power-of-two scales per 32 values, and its scaled FP4 converters use only the
// exponent of their scale, so an E4M3 scale (with mantissa bits) is applied in
// registers instead: each lane converts its eight codes of a 16-block to fp16 (scale
// 1) and multiplies them by the block scale with packed fp16 multiplies.  Every
// product e2m1 * s has at most six significant bits and lies in [2^-10, 2688], so the
// operand is exact in fp16 and v_mfma_f32_32x32x16_f16 (k = 16: one NVFP4 block per
// MFMA) accumulates the exact products in fp32; no per-block rescale is needed.
//
// Tiling: one 512-thread workgroup (8 waves, two per SIMD) per CU, tile 256 x BN with
// BN = 64 WN (192 or 128), wave tile 64 x BN/2 (2 x WN blocks of 32 x 32), the
// accumulators held transposed (the weight fragment is the MFMA's first operand): lane
// l % 32 is the output row, its 16 elements are columns 8 q + 4 (l / 32) + p of the
// block (element 4 q + p).  A stage is one 64-group of k (four NVFP4 blocks).  A 3-slot
// LDS ring holds per stage the eight activation code chunks (8 KiB), the weight code
// chunks (BN/32 KiB) and both tiles' scales (8 bytes per row or column), copied by LDS
// DMA two stages ahead.  Activation operands are expanded per wave, in registers
// (each is used by the two waves of a row range); weight operands (used by four waves)
// are expanded once per workgroup, a stage ahead and split evenly over the waves, into
// one of two fp16 LDS tiles in the MFMA's operand order, from which every wave reads
// its stage's fragments.  One barrier per stage.  The tile order is XCD-aware
// (tile_coords in k2_common.h).
//
// Epilogues: + bias and the bf16 store; the same with the exact GELU before the
// rounding; or the fused QKV epilogue (128-wide tiles, one head each: per-row RMSNorm
// over the head, the channel weights and the rotary turn of adjacent column pairs on
// the Q and K tiles), as in the int4 GEMM.
#include "common.h"
#include "k2_common.h"
#include "kernels.h"

namespace svdq {

typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// The fp16 MFMA operand of one lane and NVFP4 block: the eight E2M1 codes of dword d
// (element 2i in the low nibble of byte i) times the block scale s, exact.
__device__ __forceinline__ v8h fp4_expand(uint32_t d, uint32_t s16) {
  const _Float16 s = __builtin_bit_cast(_Float16, (uint16_t)s16);
  const v2h ss = {s, s};
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 0) * ss;
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 1) * ss;
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 2) * ss;
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 3) * ss;
  return (v8h){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

template <int WN, int EPI>
__global__ void __launch_bounds__(512, 1)
k2_gemm_fp4(const uint8_t* __restrict__ A, const uint16_t* __restrict__ sA,
            const float* __restrict__ U, int nsplit, const uint8_t* __restrict__ B,
            const uint16_t* __restrict__ sB, const uint16_t* __restrict__ L2t,
            const uint16_t* __restrict__ bias, float g, uint16_t* __restrict__ Y, int M, int N,
            int K, int M_pad, int rank, QkEpi qk, int y_wt) {
  constexpr int BM = 256, BN = 64 * WN, CB = BN / 32;
  constexpr int AC = 8 * 1024, BC = CB * 1024;  // code bytes per stage
  constexpr int AS = BM * 8, BS = BN * 8;       // scale bytes per stage
  constexpr int SLOT = AC + BC + AS + BS;
  constexpr int NF = 2 + WN;                    // fragments per wave and stage
  static_assert(WN == 2 || WN == 3, "tile width 128 or 192");
  static_assert(EPI != kEpiQkNormRope || WN == 2, "the QKV epilogue needs one head per tile");
  __shared__ __attribute__((aligned(16))) uint8_t ring[3 * SLOT];
  __shared__ float red[EPI == kEpiQkNormRope ? 512 : 1];  // per-row sums of squares, by wave

  const int tid = threadIdx.x;
  const int lane = tid & 63, lr = lane & 31, lh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_n = N / BN, tiles_m = M_pad / BM;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int row0 = tm * BM, col0 = tn * BN;
  const int rb0 = row0 >> 5, cb0 = col0 >> 5;
  const int Q = K >> 6;  // stages (64-groups); K is a multiple of 128, so Q is even

  // Copies of a stage: wave w copies activation chunk rb0 + w; waves below CB weight
  // chunk cb0 + w; the others the stage's scale rows (activations: 2 KiB, weights: BS
  // bytes) as up to two 1 KiB jobs each.  Every source pointer is formed once and
  // advances by a fixed stride per stage; the destinations are fixed offsets into the
  // slot (LDS base in M0).
  const uint32_t voff = lane * 16;
  constexpr int JOBS = 2 + (BS + 1023) / 1024;  // scale jobs: A KiB 0, 1; B KiB 0 (, 1)
  const uint8_t* srcA = A + (size_t)(rb0 + wave) * Q * 1024;
  const uint8_t* srcB = B + (size_t)(cb0 + (wave < CB ? wave : 0)) * Q * 1024;
  const uint8_t* srcS[2] = {nullptr, nullptr};
  uint32_t dstS[2] = {0, 0};
  size_t strideS[2] = {0, 0};
  bool partS[2] = {false, false};
  int njobs = 0;
  for (int j = wave - CB, n = 0; wave >= CB && j < JOBS && n < 2; j += 8 - CB, ++n) {
    if (j < 2) {
      srcS[n] = reinterpret_cast<const uint8_t*>(sA + (size_t)row0 * 4) + j * 1024;
      dstS[n] = AC + BC + j * 1024;
      strideS[n] = (size_t)M_pad * 8;
    } else {
      srcS[n] = reinterpret_cast<const uint8_t*>(sB + (size_t)col0 * 4) + (j - 2) * 1024;
      dstS[n] = AC + BC + AS + (j - 2) * 1024;
      strideS[n] = (size_t)N * 8;
      partS[n] = (j - 2) * 1024 + 1024 > BS;  // the last weight-scale KiB is partial
    }
    njobs = n + 1;
  }
  const bool lane_in_part = (int)voff < BS % 1024;
  auto dma = [&](int s, int sl) {
    const uint32_t base = lds_addr(ring) + sl * SLOT;
    dma16(voff, srcA + (size_t)s * 1024, base + wave * 1024);
    if (wave < CB) dma16(voff, srcB + (size_t)s * 1024, base + AC + wave * 1024);
#pragma unroll
    for (int n = 0; n < 2; ++n)
      if (n < njobs && (!partS[n] || lane_in_part))
        dma16(voff, srcS[n] + (size_t)s * strideS[n], base + dstS[n]);
  };

  // fp16 weight operand tiles, two buffers: fragment (column block cb, block j) is
  // 1 KiB, lane l's 16 bytes at (cb 4 + j) KiB + 16 l (the MFMA's operand order)
  constexpr int W16 = CB * 4 * 1024;
  __shared__ __attribute__((aligned(16))) uint8_t w16[2 * W16];

  struct Frag {
    v4i c[2];  // activation codes of the wave's two row blocks: dword j = block j
    v2i s[2];  // their fp16 block scales, blocks 0..3
  };
  typedef __attribute__((address_space(3))) const v4i lds_u4;
  typedef __attribute__((address_space(3))) const v2i lds_u2;
  typedef __attribute__((address_space(3))) const uint32_t lds_u1;
  typedef __attribute__((address_space(3))) const uint16_t lds_h1;
  typedef __attribute__((address_space(3))) const v8h lds_h8;
  typedef __attribute__((address_space(3))) v8h lds_h8w;
  const uint32_t ring0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)ring;
  const uint32_t w160 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)w16;
  auto read = [&](int sl, Frag& f) {
    const uint32_t base = ring0 + sl * SLOT;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      f.c[i] = *(lds_u4*)(uintptr_t)(base + (wm * 2 + i) * 1024 + lane * 16);
      f.s[i] = *(lds_u2*)(uintptr_t)(base + AC + BC + ((wm * 2 + i) * 32 + lr) * 8);
    }
  };
  auto word = [](const v4i& v, int j) { return (uint32_t)v[j]; };
  auto half = [](const v2i& v, int j) { return (uint32_t)v[j >> 1] >> (16 * (j & 1)); };
  // The weight operand of the stage in ring slot sl, expanded once per workgroup into
  // buffer wb.  A column half (wn) has 4 WN fragments (column block, NVFP4 block) per
  // stage, used by its four waves (wm = 0..3); each of those waves expands WN of them
  // (fragment q = WN wm + n: column block wn WN + q / 4, block q % 4): lane l reads
  // dword j of lane slot l of the code chunk (the weight chunks are dword-major, so a
  // wave's 64 reads are one 256-byte run) and the column's scale of block j, and writes
  // the fp16 fragment.  Expanding each fragment once instead of in all four
  // waves cuts the VALU work that would otherwise bound this kernel, and the even
  // split keeps the two waves of every SIMD equally loaded.
  auto expandB = [&](int sl, int wb) {
    const uint32_t base = ring0 + sl * SLOT;
#pragma unroll
    for (int n = 0; n < WN; ++n) {
      const int q = WN * wm + n, cb = wn * WN + (q >> 2), j = q & 3;
      const uint32_t c = *(lds_u1*)(uintptr_t)(base + AC + cb * 1024 + j * 256 + lane * 4);
      const uint32_t sc = *(lds_h1*)(uintptr_t)(base + AC + BC + AS + (cb * 32 + lr) * 8 + j * 2);
      *(lds_h8w*)(uintptr_t)(w160 + wb * W16 + (cb * 4 + j) * 1024 + lane * 16) = fp4_expand(c, sc);
    }
  };

  v16f acc[2][WN];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int c = 0; c < WN; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][c][e] = 0.f;

  // Stage with activation fragments f and weight buffer wb: the stage's fp16 weight
  // fragments are read at its start; block j's activation operands are expanded in
  // registers (one set each for even and odd blocks) while block j - 1's MFMAs run;
  // after block 0, `next` issues the next stage's activation reads and expands its
  // weight operand into the other buffer.
  auto compute = [&](const Frag& f, int wb, auto&& next) {
    v8h bw[4][WN];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int c = 0; c < WN; ++c)
        bw[j][c] = *(lds_h8*)(uintptr_t)(w160 + wb * W16 + ((wn * WN + c) * 4 + j) * 1024 + lane * 16);
    v8h a[2][2];
    auto expand = [&](int j) {
#pragma unroll
      for (int i = 0; i < 2; ++i) a[j & 1][i] = fp4_expand(word(f.c[i], j), half(f.s[i], j));
    };
    expand(0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j < 3) expand(j + 1);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int c = 0; c < WN; ++c)
          acc[i][c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bw[j][c], a[j & 1][i], acc[i][c], 0, 0, 0);
      // (no scheduling barrier around it: letting the compiler interleave the next
      // stage's reads and weight expansion with this block's MFMAs saves 1.2 us at
      // 4096 x 3072 x 3072)
      if (j == 0) next();
    }
  };

  dma(0, 0);
  dma(1, 1);
  wait_vm0();
  barrier_lds();
  Frag F0, F1;
  read(0, F0);
  expandB(0, 0);
  // Two stages per iteration (Q is even), so each fragment set keeps its registers.
  // Slots rotate 0, 1, 2: stage t in slot t % 3, tracked without a division; stage t's
  // fp16 weights are in buffer t % 2.
  int sl0 = 0;  // slot of stage t
  for (int t = 0; t < Q; t += 2) {
    const int sl1 = sl0 == 2 ? 0 : sl0 + 1, sl2 = sl1 == 2 ? 0 : sl1 + 1;
    wait_vm0();
    barrier_lds();  // slot of t + 1 landed, weight buffer 0 (stage t) written
    if (t + 2 < Q) dma(t + 2, sl2);
    compute(F0, 0, [&] {
      read(sl1, F1);
      expandB(sl1, 1);
    });
    wait_vm0();
    barrier_lds();
    if (t + 3 < Q) dma(t + 3, sl0);
    compute(F1, 1, [&] {
      if (t + 2 < Q) {
        read(sl2, F0);
        expandB(sl2, 0);
      }
    });
    sl0 = sl2;
  }
  wait_vm0();
  barrier_lds();  // every wave is past its operand reads: the ring is free for staging

  // Epilogue: acc * g, + U @ L2t^T (U split into three bf16 terms), + bias, then (QKV
  // mode) the per-head norm and rotation, and bf16 stores through a per-wave LDS tile.
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rowb = row0 + wm * 64 + 32 * i;
#pragma unroll
    for (int c = 0; c < WN; ++c) {
      const int colb = col0 + (wn * WN + c) * 32;
      v16f v = acc[i][c];
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] *= g;
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
        for (int q = 0; q < 8; ++q) {
          const Bf16x3 s3 = split3_bf16(uf[q]);
          hi[q] = s3.h;
          mid[q] = s3.m;
          lo[q] = s3.l;
        }
        const uint4 lb = *reinterpret_cast<const uint4*>(L2t + (size_t)(colb + lr) * rank + kk + 8 * lh);
        v = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, lb), hi, v, 0, 0, 0);
        v = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, lb), mid, v, 0, 0, 0);
        v = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, lb), lo, v, 0, 0, 0);
      }
      if (bias) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint2 b2 = *reinterpret_cast<const uint2*>(bias + colb + 8 * q + 4 * lh);
          v[4 * q + 0] += __uint_as_float(b2.x << 16);
          v[4 * q + 1] += __uint_as_float(b2.x & 0xFFFF0000u);
          v[4 * q + 2] += __uint_as_float(b2.y << 16);
          v[4 * q + 3] += __uint_as_float(b2.y & 0xFFFF0000u);
        }
      }
      acc[i][c] = v;
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
        for (int c = 0; c < WN; ++c)
#pragma unroll
          for (int e = 0; e < 16; ++e) ss[i] = fmaf(acc[i][c][e], acc[i][c][e], ss[i]);
#pragma unroll
      for (int i = 0; i < 2; ++i) ss[i] += __shfl_xor(ss[i], 32);
      if (lh == 0) {
        red[wave * 64 + lr] = ss[0];
        red[wave * 64 + 32 + lr] = ss[1];
      }
      barrier_lds();
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float inv = 1.0f / sqrtf((ss[i] + red[(wave ^ 1) * 64 + 32 * i + lr]) * (1.0f / 128.0f) +
                                       qk.eps);
        const int row = min(row0 + wm * 64 + 32 * i + lr, M - 1);  // pad rows are not stored
#pragma unroll
        for (int c = 0; c < WN; ++c)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int ch = wn * 64 + 32 * c + 8 * q + 4 * lh;  // channel of element 4q
            const uint2 w2 = *reinterpret_cast<const uint2*>(nw + ch);
            const float w[4] = {__uint_as_float(w2.x << 16), __uint_as_float(w2.x & 0xFFFF0000u),
                                __uint_as_float(w2.y << 16), __uint_as_float(w2.y & 0xFFFF0000u)};
            const float4 cs = *reinterpret_cast<const float4*>(qk.rope + (size_t)row * 128 + ch);
            float n[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) n[p] = acc[i][c][4 * q + p] * inv * w[p];
            acc[i][c][4 * q + 0] = n[0] * cs.x - n[1] * cs.y;
            acc[i][c][4 * q + 1] = n[1] * cs.x + n[0] * cs.y;
            acc[i][c][4 * q + 2] = n[2] * cs.z - n[3] * cs.w;
            acc[i][c][4 * q + 3] = n[3] * cs.z + n[2] * cs.w;
          }
      }
    }
  }
  // bf16 stores: each 32 x 32 block through the wave's LDS tile (rows of 80 B), then 16
  // bytes per lane, four lanes per row
  uint16_t* tile = reinterpret_cast<uint16_t*>(ring) + wave * (32 * 40);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rowb = row0 + wm * 64 + 32 * i;
#pragma unroll
    for (int c = 0; c < WN; ++c) {
      const int colb = col0 + (wn * WN + c) * 32;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t h[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float v = acc[i][c][4 * q + p];
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
        if (row < M) {
          uint16_t* yp = Y + (size_t)row * N + colb + ch * 8;
          if (y_wt) store_wt(yp, v);
          else *reinterpret_cast<uint4*>(yp) = v;
        }
      }
    }
  }
}

hipError_t launch_k2_fp4(const uint8_t* A, const uint16_t* sA, const float* U, int nsplit,
                         const uint8_t* B, const uint16_t* sB, const uint16_t* L2t,
                         const uint16_t* bias, float g, uint16_t* Y, int M, int N, int K,
                         int M_pad, int rank, int epi, const QkEpi& qk, hipStream_t st,
                         hipEvent_t ev0, hipEvent_t ev1) {
  if (M_pad % 256 != 0 || N % 128 != 0 || K % 128 != 0) return hipErrorInvalidValue;
  if (epi == kEpiQkNormRope && (N % 384 != 0 || !qk.norm_q || !qk.norm_k || !qk.rope))
    return hipErrorInvalidValue;
  const bool wide = N % 192 == 0 && epi != kEpiQkNormRope;
  const int bn = wide ? 192 : 128;
  dim3 grid((N / bn) * (M_pad / 256));
  auto k = epi == kEpiQkNormRope ? k2_gemm_fp4<2, kEpiQkNormRope>
           : wide ? (epi == kEpiGelu ? k2_gemm_fp4<3, kEpiGelu> : k2_gemm_fp4<3, kEpiPlain>)
                  : (epi == kEpiGelu ? k2_gemm_fp4<2, kEpiGelu> : k2_gemm_fp4<2, kEpiPlain>);
  // Y through the L2 at device scope when the grid is one round (as in the int4 GEMM)
  const int y_wt = grid.x <= (unsigned)device_cu_count();
  hipExtLaunchKernelGGL(k, grid, dim3(512), 0, st, ev0, ev1, 0, A, sA, U, nsplit, B, sB, L2t, bias,
                        g, Y, M, N, K, M_pad, rank, qk, y_wt);
  return hipGetLastError();
}

}  // namespace svdq
