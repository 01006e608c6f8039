// Row-stream skeleton of the fused quantizers (K1 feeding the GEMM) for layers whose
// 32-row workgroups do not fit one round on the CUs: smoothing, the rank-r low-rank
// down projection and the per-k-block quantizer, as in k1_rows32.h, but with every
// workgroup resident for the whole launch.
//
// Work split: grid (P, k-splits of at most 1536 values), 768 threads: twelve waves, wave
// w owning the 128-wide k-block w of its split.  Workgroup (p, s) takes the 16-row
// units p, p + P, p + 2P, ... of the M_pad rows.  Its smoothing slice and lora_down
// operands are loaded once, into LDS and registers, and serve every unit, so lora_down
// crosses L2 once per workgroup rather than once per 16 rows.  Each wave copies its unit
// tiles (16 rows x 128 values, 4 KiB) into a two-slot LDS ring with global_load_lds two
// units ahead: the copy of unit i + 2 runs under the arithmetic of unit i + 1.  The
// twelve waves' partial U tiles of a unit are summed in LDS in a fixed order (one
// barrier per unit, two partial buffers) and written as the split's partial U in the
// fragment layout, so U is deterministic.
//
// The copies (the tiles and the smoothing slice) are lds_dma16 (common.h), which the
// compiler does not see, so each read of a copied tile follows an explicit wait.  The
// waits count this wave's vector memory operations issued after the copies awaited,
// which retire in issue order: the quantizer's stores of the previous unit
// (QUANT::kStores), its partial-U store (waves 0 .. rank/16 - 1) and the next unit's
// four copies.  Operations the count leaves out can only make a wait stricter.  So that
// every count is fixed, rows at or past M are copied from row M - 1 and zeroed in
// registers.
#pragma once
#include "k1_common.h"

namespace svdq {

template <int N>
__device__ __forceinline__ void k1s_wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void k1s_wait(int n) {
  switch (n) {  // wave-uniform
    case 0: k1s_wait_vm<0>(); break;
    case 1: k1s_wait_vm<1>(); break;
    case 2: k1s_wait_vm<2>(); break;
    case 3: k1s_wait_vm<3>(); break;
    case 4: k1s_wait_vm<4>(); break;
    case 5: k1s_wait_vm<5>(); break;
    case 6: k1s_wait_vm<6>(); break;
    case 7: k1s_wait_vm<7>(); break;
    case 8: k1s_wait_vm<8>(); break;
    default: k1s_wait_vm<0>(); break;
  }
}

constexpr int kK1StreamWaves = 12;

template <int S>
struct Slot {
  constexpr int operator()() const { return S; }
};

// Workgroups per k-split: as many as fill the CUs once (one workgroup per CU), at most
// one per 16-row unit.
inline int k1_stream_workgroups(int M_pad, int splits) {
  const int units = M_pad / 16;
  const int per = device_cu_count() / splits;
  return per < 1 ? 1 : (per < units ? per : units);
}

template <class QUANT, bool GELU_IN>
__device__ __forceinline__ void k1_stream(const K1Args& a) {
  constexpr int NW = kK1StreamWaves;
  constexpr int RB = 16 * 128;  // bf16 values of one X tile (16 rows)
  static_assert(NW * 128 == kK1SplitK, "one k-block per wave");
  static_assert(QUANT::kStores >= 0 && QUANT::kStores <= 3, "wait counts");
  __shared__ __attribute__((aligned(16))) uint16_t XS[2][NW][RB];      // 96 KiB
  __shared__ __attribute__((aligned(16))) float MSf[NW][128];          // 6 KiB
  __shared__ __attribute__((aligned(16))) uint16_t MSraw[NW][128];     // 3 KiB
  __shared__ __attribute__((aligned(16))) float ured[2][NW][16][36];   // 54 KiB

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15;
  const int q = lane >> 4;
  const int K = a.K;
  const int kb0 = (blockIdx.y * kK1SplitK) >> 7;
  const int nb = (min(kK1SplitK, K - (int)blockIdx.y * kK1SplitK)) >> 7;
  const bool has = wave < nb;
  const int kb = kb0 + wave;
  const int rank = a.rank;
  const int nsl = rank >> 4;
  const int units = a.M_pad >> 4;
  const int P = gridDim.x;
  const int u_first = blockIdx.x;
  // this wave's partial-U store per unit: threads t < 4 rank store one float4 each
  const int u_st = (rank > 0 && 64 * wave < 4 * rank) ? 1 : 0;

  auto copy_unit = [&](auto SLOT, int unit) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int u = 64 * t + lane;
      const int rr = u >> 4, c = (u & 15) ^ (rr & 7);
      const int grow = min(unit * 16 + rr, a.M - 1);
      lds_dma16(a.x + (size_t)grow * K + 128 * kb + 8 * c, &XS[SLOT()][wave][512 * t]);
    }
  };

  // issue order: smoothing slice (copied to LDS), lora_down operands, the first two
  // units' copies
  uint4 L[2][4];
  if (has) {
    if (lane < 16) lds_dma16(a.smooth + 128 * kb + 8 * lane, &MSraw[wave][0]);
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
    if (u_first < units) copy_unit(Slot<0>{}, u_first);
    if (u_first + P < units) copy_unit(Slot<1>{}, u_first + P);
  }

  // prev: the previous unit's stores may still be in flight (they are counted)
  auto step = [&](auto SLOT, int unit, bool first, bool prev, bool refill) {
    constexpr int slot = SLOT();
    const bool next = unit + P < units;  // the next unit's copies are in flight
    if (has) {
      // copies younger than this unit's: (it > 0) the previous unit's stores, then
      // the next unit's copies
      k1s_wait((prev ? QUANT::kStores + u_st : 0) + (next ? 4 : 0));
      if (first) {
        // the smoothing slice landed before this unit's copies: widen it to fp32 once
        const uint32_t mraw = reinterpret_cast<const uint32_t*>(&MSraw[wave][0])[lane];
        *reinterpret_cast<float2*>(&MSf[wave][2 * lane]) =
            make_float2(__uint_as_float(mraw << 16), __uint_as_float(mraw & 0xFFFF0000u));
      }
      const int row = unit * 16 + r;
      const bool zero = row >= a.M;
      const int k0 = 128 * kb + 32 * q;
      float xh[32];
      uint32_t xb[16];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int cc = 4 * q + c;
        uint4 xv = *reinterpret_cast<const uint4*>(&XS[slot][wave][8 * (r * 16 + (cc ^ (r & 7)))]);
        if (zero) xv = make_uint4(0, 0, 0, 0);
        const float4 m0 = *reinterpret_cast<const float4*>(&MSf[wave][8 * cc]);
        const float4 m1 = *reinterpret_cast<const float4*>(&MSf[wave][8 * cc + 4]);
        const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
        const float mf[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          // smoothing: xhat = bf16(x * m), one rounding of an exact product
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
        v4f u0 = {0.f, 0.f, 0.f, 0.f}, u1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const v4i a4 = {(int)xb[4 * c], (int)xb[4 * c + 1], (int)xb[4 * c + 2], (int)xb[4 * c + 3]};
          const v8bf av = __builtin_bit_cast(v8bf, a4);
          u0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(v8bf, L[0][c]), u0, 0, 0, 0);
          if (rank > 16)
            u1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(v8bf, L[1][c]), u1, 0, 0, 0);
        }
        // C layout of the 16x16 MFMA: lane l holds column l%16, rows 4(l/16) + i
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ured[slot][wave][4 * q + i][r] = u0[i];
          ured[slot][wave][4 * q + i][16 + r] = u1[i];
        }
      }
    }
    if (rank > 0) {
      // all partials of this unit are in ured[slot]; ured[slot] is written again two
      // units later, after the next unit's barrier, which every reader has passed
      __syncthreads();
      const int t = threadIdx.x;
      if (t < 4 * rank) {
        const int rr = t / (rank >> 2), cc = 4 * (t % (rank >> 2));
        float4 p[NW];
#pragma unroll
        for (int w = 0; w < NW; ++w)
          p[w] = w < nb ? *reinterpret_cast<const float4*>(&ured[slot][w][rr][cc]) : make_float4(0.f, 0.f, 0.f, 0.f);
        float4 v = p[0];
#pragma unroll
        for (int w = 1; w < NW; ++w)
          if (w < nb) {
            v.x += p[w].x;
            v.y += p[w].y;
            v.z += p[w].z;
            v.w += p[w].w;
          }
        store_wt(&a.uact[u_frag_index(blockIdx.y, unit * 16 + rr, cc, a.M_pad, rank)], v4f{v.x, v.y, v.z, v.w});
      }
    }
    // this wave has read slot `slot` of its own tiles: refill it two units ahead
    if (refill && has && unit + 2 * P < units) copy_unit(SLOT, unit + 2 * P);
  };
  // The first unit is peeled off and followed by a full wait that the compiler sees:
  // the lora_down loads are conditional, so without it the compiler would still treat
  // them as in flight inside the loop and wait for every copy before each unit's MFMAs.
  // The peeled unit's refill is issued after that wait, and the next unit counts no
  // stores before it.
  if (u_first < units) step(Slot<0>{}, u_first, true, false, false);
  __builtin_amdgcn_s_waitcnt(0);  // on every path
  if (has && u_first + 2 * P < units) copy_unit(Slot<0>{}, u_first + 2 * P);
  for (int unit = u_first + P; unit < units; unit += 2 * P) {
    step(Slot<1>{}, unit, false, unit > u_first + P, true);
    if (unit + P < units) step(Slot<0>{}, unit + P, false, true, true);
  }
}

}  // namespace svdq
