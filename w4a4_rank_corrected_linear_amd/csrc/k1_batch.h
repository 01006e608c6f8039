// Batch skeleton of the fused activation-side kernels (K1 feeding the GEMM):
// smoothing, the rank-r low-rank down projection, and a per-k-block quantizer.
//
// Work split: grid (row-blocks of 16 rows) x (k-splits of at most 1536 values).  A
// 256-thread workgroup owns 16 rows and one k-split; wave w takes the 128-wide
// k-blocks w, w+4, w+8 of the split (at most three).  Lane l holds row l%16 and the
// 32 consecutive values k = 128 kb + 32 q + [0, 32), q = l/16.
//
// Every wave first issues all of its loads: the lora_down operands into registers,
// then its X tiles (16 rows x 128 values, 4 KiB each) and smoothing slices into LDS
// with global_load_lds.  It then waits once and computes.  Two workgroups share a
// CU, so one's copies run under the other's arithmetic, and no register is spent on
// bytes in flight.  X tiles are stored as 16-byte units u = row * 16 + (c ^ (row & 7))
// (c = k / 8 within the block), which puts the eight rows of one read in distinct
// bank groups.  Rows at or past M are read from row M - 1 and zeroed.
//
// Low-rank down projection: MFMA call c (0..3) of v_mfma_f32_16x16x32_bf16 takes the
// lane's chunk c (k = ... + 8c + [0, 8)) at MFMA k-position 8q + [0, 8); its B operand
// is lora_down at the same k, read from the packed fragment order in which each
// call's 64 operands are 1 KiB contiguous.  The four waves' partial tiles are summed
// in LDS in a fixed order and written as the split's partial U (fp32, the fragment
// layout of common.h); the GEMM adds the splits in a fixed order, so U is
// deterministic.
#pragma once
#include "common.h"
#include "kernels.h"

namespace svdq {

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

struct K1Args {
  const uint16_t* x;
  int M, K;
  const uint16_t* smooth;
  const uint16_t* ldown;
  int rank;
  uint8_t* out;
  void* scales;
  float* uact;  // partial sums per k-split, fragment layout (common.h)
  int M_pad;
  float g;
};

// QUANT::block(const K1Args&, const float (&xh)[32], int row, int k0, int q) quantizes
// the lane's 32 smoothed values (row, k0 .. k0 + 31) and writes its outputs.
template <class QUANT>
__device__ __forceinline__ void k1_batch(const K1Args& a) {
  constexpr int BPW = 3;        // k-blocks per wave at most
  constexpr int RB = 16 * 128;  // bf16 values of one X tile
  __shared__ __attribute__((aligned(16))) uint16_t XS[4][BPW][RB];
  __shared__ __attribute__((aligned(16))) uint16_t MS[4][BPW][128];
  __shared__ float ured[4][16][33];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;
  const int q = lane >> 4;
  const int row0 = blockIdx.x * 16;
  const int row = row0 + r;
  const bool valid = row < a.M;
  const bool tail = row0 + 16 > a.M;  // workgroup-uniform: this block holds padding rows
  const int K = a.K;
  const int kb0 = (blockIdx.y * kK1SplitK) >> 7;
  const int nb = (min(kK1SplitK, K - (int)blockIdx.y * kK1SplitK)) >> 7;
  const int nbw = (nb - wave + 3) >> 2;  // blocks of this wave (0..3)
  const int rank = a.rank;

  // lora_down in the packed fragment order (svdq_pack_lora_down): the operands of
  // (k-block kb, slice sl, call c) are 64 lanes x 16 B contiguous
  uint4 L[BPW][2][4];
  const int nsl = rank >> 4;
#pragma unroll
  for (int j = 0; j < BPW; ++j) {
    if (j < nbw && rank > 0) {
      const int kb = kb0 + wave + 4 * j;
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        if (sl < nsl) {
          const uint4* lp = reinterpret_cast<const uint4*>(a.ldown) + ((size_t)(kb * nsl + sl) * 4) * 64 + lane;
#pragma unroll
          for (int c = 0; c < 4; ++c) L[j][sl][c] = lp[64 * c];
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < BPW; ++j) {
    if (j < nbw) {
      const int kb = kb0 + wave + 4 * j;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int u = 64 * t + lane;
        const int rr = u >> 4, c = (u & 15) ^ (rr & 7);
        const int gr = min(row0 + rr, a.M - 1);
        __builtin_amdgcn_global_load_lds(a.x + (size_t)gr * K + 128 * kb + 8 * c,
                                         &XS[wave][j][512 * t], 16, 0, 0);
      }
      if (lane < 16)
        __builtin_amdgcn_global_load_lds(a.smooth + 128 * kb + 8 * lane, &MS[wave][j][0], 16, 0, 0);
    }
  }

  // Each wave reads only the tiles it copied itself, so its own wait suffices.  The
  // wait is explicit: the compiler does not order LDS reads after global_load_lds
  // writes to the same array by itself.
  __builtin_amdgcn_s_waitcnt(0);

  v4f u0 = {0.f, 0.f, 0.f, 0.f};
  v4f u1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < BPW; ++j) {
    if (j < nbw) {
      const int k0 = 128 * (kb0 + wave + 4 * j) + 32 * q;
      // smoothing: xhat = bf16(x * m), one rounding of an exact product
      float xh[32];
      uint32_t xb[16];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int cc = 4 * q + c;
        uint4 xv = *reinterpret_cast<const uint4*>(&XS[wave][j][8 * (r * 16 + (cc ^ (r & 7)))]);
        const uint4 mv = *reinterpret_cast<const uint4*>(&MS[wave][j][8 * cc]);
        if (tail && !valid) xv = make_uint4(0, 0, 0, 0);
        const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
        const uint32_t mw[4] = {mv.x, mv.y, mv.z, mv.w};
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

      QUANT::block(a, xh, row, k0, q);

      if (rank > 0) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const v4i a4 = {(int)xb[4 * c], (int)xb[4 * c + 1], (int)xb[4 * c + 2], (int)xb[4 * c + 3]};
          const v8bf av = __builtin_bit_cast(v8bf, a4);
          u0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(v8bf, L[j][0][c]), u0, 0, 0, 0);
          if (rank > 16)
            u1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(v8bf, L[j][1][c]), u1, 0, 0, 0);
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
      store_wt(&a.uact[u_frag_index(blockIdx.y, row0 + rr, cc, a.M_pad, rank)],
               ((ured[0][rr][cc] + ured[1][rr][cc]) + ured[2][rr][cc]) + ured[3][rr][cc]);
    }
  }
}

}  // namespace svdq
