// Row-pair skeleton of the fused int4 quantizer (K1 feeding the GEMM): smoothing, the
// rank-r low-rank down projection and the per-k-block quantizer for 32 rows and one
// k-split per workgroup.
//
// Work split: grid (row-blocks of 32 rows) x (k-splits of at most 1536 values), 768
// threads: twelve waves, three per SIMD.  Wave w owns the 128-wide k-block w of the
// split for both 16-row halves, so its lora_down operands (the B operands of the
// low-rank MFMAs, in registers) serve 32 rows, and a CU reads half of lora_down once
// per launch instead of once per 16 rows.  Lane l holds row l%16 of a half and the 32
// consecutive values k = 128 kb + 32 q + [0, 32), q = l/16.
//
// Each wave issues its smoothing slice and lora_down operands (registers), then its
// two X tiles (16 rows x 128 values, 4 KiB each) into LDS with global_load_lds, and
// quantizes the two halves in turn (the compiler holds the first half's reads until
// both copies have landed: it orders LDS reads after every copy in flight; both land
// at nearly the same time, so the asm copies of k1_stream.h gain nothing here).  X
// tiles are stored
// as 16-byte units u = row * 16 + (c ^ (row & 7)) (c = k / 8 within the block), which
// puts the eight rows of one read in distinct bank groups.  The smoothing slice is
// widened to fp32 in LDS once per wave.  In the workgroup that holds the last rows,
// rows at or past M are cleared in LDS and not copied.
//
// Low-rank down projection: per half, MFMA call c (0..3) of v_mfma_f32_16x16x32_bf16
// takes the lane's chunk c at MFMA k-position 8q + [0, 8); its B operand is lora_down
// at the same k, read from the packed fragment order in which each call's 64 operands
// are 1 KiB contiguous.  The twelve waves' partial tiles are summed in LDS in a fixed
// order and written as the split's partial U (fp32, the fragment layout of common.h);
// the GEMM adds the splits in a fixed order, so U is deterministic.
#pragma once
#include "k1_common.h"

namespace svdq {

// Waits for this wave's outstanding memory operations (the LDS copies count on the
// vector memory counter).  Written as asm with a memory clobber so that the LDS reads
// of the copied tiles stay below them.
__device__ __forceinline__ void k1r_wait_vm4() { asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void k1r_wait_vm0() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory"); }

constexpr int kK1RowsWaves = 12;  // waves per workgroup = 128-wide k-blocks per split

template <class QUANT, bool GELU_IN>
__device__ __forceinline__ void k1_rows32(const K1Args& a) {
  constexpr int NW = kK1RowsWaves;
  constexpr int RB = 16 * 128;  // bf16 values of one X tile (16 rows)
  static_assert(NW * 128 == kK1SplitK, "one k-block per wave");
  __shared__ __attribute__((aligned(16))) uint16_t XS[NW][2][RB];   // 96 KiB
  __shared__ __attribute__((aligned(16))) float MSf[NW][128];       // 6 KiB
  // partial U tiles of the waves (rows padded to 36 floats, so a row's four consecutive
  // values are one aligned float4), apart from the X tiles so that a wave writes its
  // partial as soon as it is done
  __shared__ __attribute__((aligned(16))) float ured[NW][32][36];  // 54 KiB

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15;
  const int q = lane >> 4;
  const int row0 = blockIdx.x * 32;
  const int K = a.K;
  const int kb0 = (blockIdx.y * kK1SplitK) >> 7;
  const int nb = (min(kK1SplitK, K - (int)blockIdx.y * kK1SplitK)) >> 7;
  const bool has = wave < nb;
  const int kb = kb0 + wave;
  const int rank = a.rank;
  const int nsl = rank >> 4;
  const bool tail = row0 + 32 > a.M;  // workgroup-uniform: this block holds padding rows

  if (tail && has) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        *reinterpret_cast<uint4*>(&XS[wave][h][512 * t + 8 * lane]) = make_uint4(0, 0, 0, 0);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
  // issue order: smoothing slice, lora_down operands, X half 0, X half 1 (4 copies)
  uint32_t mraw = 0;
  uint4 L[2][4];
  if (has) {
    mraw = reinterpret_cast<const uint32_t*>(a.smooth + 128 * kb)[lane];
    if (rank > 0) {
#pragma unroll
      for (int sl = 0; sl < 2; ++sl)
        if (sl < nsl) {
          const uint4* lp =
              reinterpret_cast<const uint4*>(a.ldown) + ((size_t)(kb * nsl + sl) * 4) * 64 + lane;
#pragma unroll
          for (int c = 0; c < 4; ++c) L[sl][c] = lp[64 * c];
        }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int u = 64 * t + lane;
        const int rr = u >> 4, c = (u & 15) ^ (rr & 7);
        const int grow = row0 + 16 * h + rr;
        if (!tail || grow < a.M)
          __builtin_amdgcn_global_load_lds(a.x + (size_t)grow * K + 128 * kb + 8 * c,
                                           &XS[wave][h][512 * t], 16, 0, 0);
      }
  }
  v4f u0[2], u1[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    u0[h] = v4f{0.f, 0.f, 0.f, 0.f};
    u1[h] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  if (has) {
    // everything but X half 1 has landed (in-order counter); in the tail block a whole
    // copy instruction may be skipped, so there the wait is for everything
    if (tail) k1r_wait_vm0();
    else k1r_wait_vm4();
    *reinterpret_cast<float2*>(&MSf[wave][2 * lane]) =
        make_float2(__uint_as_float(mraw << 16), __uint_as_float(mraw & 0xFFFF0000u));
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (h == 1) k1r_wait_vm0();
      const int row = row0 + 16 * h + r;
      const int k0 = 128 * kb + 32 * q;
      // smoothing: xhat = bf16(x * m), one rounding of an exact product
      float xh[32];
      uint32_t xb[16];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int cc = 4 * q + c;
        const uint4 xv = *reinterpret_cast<const uint4*>(&XS[wave][h][8 * (r * 16 + (cc ^ (r & 7)))]);
        const float4 m0 = *reinterpret_cast<const float4*>(&MSf[wave][8 * cc]);
        const float4 m1 = *reinterpret_cast<const float4*>(&MSf[wave][8 * cc + 4]);
        const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
        const float mf[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float p0 = k1_input<GELU_IN>(xw[p] << 16) * mf[2 * p];
          const float p1 = k1_input<GELU_IN>(xw[p] & 0xFFFF0000u) * mf[2 * p + 1];
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
          u0[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(v8bf, L[0][c]), u0[h], 0, 0, 0);
          if (rank > 16)
            u1[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(v8bf, L[1][c]), u1[h], 0, 0, 0);
        }
      }
    }
  }
  if (rank > 0) {
    // C layout of the 16x16 MFMA: lane l holds column l%16, rows 4(l/16) + i
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ured[wave][16 * h + 4 * q + i][r] = u0[h][i];
        ured[wave][16 * h + 4 * q + i][16 + r] = u1[h][i];
      }
    __syncthreads();
    // thread t sums four consecutive ranks 4 (t % (rank/4)) .. + 3 of row t / (rank/4):
    // the nb partials are read at once (float4 each), added in wave order, and stored as
    // one float4 (four consecutive ranks are contiguous in the fragment layout)
    const int t = threadIdx.x;
    if (t < 8 * rank) {
      const int rr = t / (rank >> 2), cc = 4 * (t % (rank >> 2));
      float4 p[NW];
#pragma unroll
      for (int w = 0; w < NW; ++w)
        p[w] = w < nb ? *reinterpret_cast<const float4*>(&ured[w][rr][cc]) : make_float4(0.f, 0.f, 0.f, 0.f);
      float4 v = p[0];
#pragma unroll
      for (int w = 1; w < NW; ++w)
        if (w < nb) {
          v.x += p[w].x;
          v.y += p[w].y;
          v.z += p[w].z;
          v.w += p[w].w;
        }
      store_wt(&a.uact[u_frag_index(blockIdx.y, row0 + rr, cc, a.M_pad, rank)], v4f{v.x, v.y, v.z, v.w});
    }
  }
}

}  // namespace svdq
