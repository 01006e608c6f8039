// K2, int4: the 4-bit x 4-bit residual GEMM with per-group rescale, fused with the
// rank-r up projection, the bias and the bf16 store.
//
//   Y[m,n] = bf16( sum_j U[m,j] L2t[n,j] + sum_g sx[m,g] sw[n,g] P_g[m,n] + b[n] ),
//   P_g    = sum_{k in g} qx[m,k] qw[n,k]   (exact integers)
//
// (Diffusers docs "Nunchaku Lite", "Supported quantization types": svdq_w4a4 int4
// group 64 with the SVDQ low-rank correction.)
//
// Arithmetic per 32x32 output block and 64-group (the block is held transposed: lane
// l%32 is the output row, the 16 accumulator elements are output columns):
//   D = v_mfma_scale_f32_32x32x64_f8f6f4(W_g, X_g)   E2M3 codes q/8, block scales 2^2
//                                                    and 2^3: D = P_g / 2 exactly
//   S = v_mfma_f32_32x32x8_bf16(sw, sx)              the scale records of common.h:
//                                                    sw[g] sx[g] at k = 0 or 1 (lanes
//                                                    < 32) and k = 4 or 5 (lanes >= 32),
//                                                    the exact product 2 sw[n] sx[m]
//   acc = fma(S, D, acc)                             one VALU op per element and group
// The low-rank term U L2t^T (U split into three bf16 terms, split3_bf16 in common.h)
// either seeds the accumulator before the main loop (all of its global loads issued
// before the first is used) or, when K has at most two k-splits, is added in the
// epilogue from copies of U and lora_up that the last two stages DMA into the ring
// slots they leave free.
//
// Epilogues (EPI): + bias and the bf16 store; the same with the exact GELU of each
// result before the rounding; or the fused QKV epilogue (128 x 384 tiles, three heads
// of 128 columns each): on Q and K heads the RMSNorm of every row over the head (the
// waves' per-row sums of squares of each 32-column block meet in LDS and are added in
// column order), the channel weights, and the rotary turn of adjacent column pairs
// by the row's (cos, sin), all in fp32 on the unrounded result, then one rounding.
//
// Tiling: one 512-thread workgroup (8 waves, two per SIMD) per CU, tile BM x BN with
// BM = 256 (waves 4 x 2, BN = 128 or 192) or BM = 128 (waves 2 x 4, BN = 384); the
// wave tile is 64 rows x WN 32-column blocks (WN = 2 or 3), 2 WN MFMA blocks.  A
// stage is two 64-groups.  Operands live in a 3-slot LDS ring; slot s%3 holds stage s:
//   A   [row-block][group 0..1][1536 B]       activation lane slots (written by K1)
//   B   [col-block][group 0..1][1536 B]       weight lane slots (written by the pack)
//   SA  [group][BM rows], SB [BN cols]        8-byte scale records (common.h): one
//                                             weight record serves both groups
// all copied by LDS DMA (global_load_lds_dwordx4, 16 B per lane).  At the top of
// iteration t every wave waits for its own copies of stage t+1, the barrier publishes
// them and frees slot (t+2)%3, and the copies of stage t+2 start.  The twelve (or
// eight) compute steps of the stage then form one straight-line block: step b issues
// the two MFMAs of block b+1, rescales block b with the MFMA results of step b-1, and
// loads the fragments needed two steps later (B fragments into three rotating
// register sets, A fragments per group parity); the last steps already load and issue
// stage t+1's first block.  The LDS addresses of the current and the next slot are
// formed once per stage (lane, wave and slot parts in one register per operand
// stream), so every fragment read is that register plus an immediate offset.  The
// tile's bias is copied to LDS at the top of the last stage.
//
// The tile order is XCD-aware: workgroup i runs on XCD i % 8, and the eight XCDs
// take disjoint (tiles_m/4) x (tiles_n/2) sub-grids, so each XCD's L2 holds a quarter
// of the activation rows and half of the weight columns.
#include <algorithm>

#include "common.h"
#include "k2_common.h"
#include "kernels.h"

namespace svdq {


template <int BM, int BN, int EPI>
__global__ void __launch_bounds__(512, 1)
k2_gemm_int4(const uint8_t* __restrict__ A, const uint2* __restrict__ sA,
             const float* __restrict__ U, int nsplit, const uint8_t* __restrict__ B,
             const uint2* __restrict__ sB, const uint16_t* __restrict__ L2t,
             const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y,
             int M, int N, int K, int M_pad, int rank, QkEpi qk, int full_tiles, int ks,
             float* __restrict__ part, int y_wt) {
  constexpr int WMW = BM / 64;             // waves along the rows (4 or 2)
  constexpr int WNW = 8 / WMW;             // waves along the columns (2 or 4)
  constexpr int WC = BN / WNW;             // columns per wave
  constexpr int WN = WC / 32;              // 32-column blocks per wave
  constexpr int NA = BM / 32;              // 32-row blocks per tile
  constexpr int CB = BN / 32;              // 32-column blocks per tile
  constexpr int ASZ = NA * 2 * 384;        // dwords of A per stage
  constexpr int BSZ = CB * 2 * 384;        // dwords of B per stage
  constexpr int SLOT = ASZ + BSZ + 4 * BM + 2 * BN;  // + scale records: SA 2 x BM, SB BN
  constexpr int NB = 4 * WN;               // blocks per wave and stage
  constexpr int NBS = (WN == 3) ? 3 : 4;   // B register sets (divides 2 WN fragments)
  static_assert((BM == 256 && (BN == 128 || BN == 192)) || (BM == 128 && BN == 384),
                "tiles 256 x 128, 256 x 192 or 128 x 384");
  static_assert(EPI != kEpiQkNormRope || BN == 384, "the QKV epilogue takes three whole heads");
  __shared__ __attribute__((aligned(16))) uint32_t ring[3 * SLOT];
  __shared__ __attribute__((aligned(16))) uint16_t bias_s[BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int lr = lane & 31, lh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WNW, wn = wave % WNW;
  const int tiles_n = N / BN, tiles_m = M_pad / BM;
  // Workgroups below full_tiles own tile blockIdx.x and all of K.  The tiles of the
  // last, partial round (ids full_tiles and up) are split along K into ks pieces of
  // consecutive stages, one workgroup each (piece >= 0), which store their fp32
  // partial tiles for the tail kernel below to add up and finish.
  int tile_id = blockIdx.x, piece = -1;
  if ((int)blockIdx.x >= full_tiles) {
    const int q = (int)blockIdx.x - full_tiles;
    tile_id = full_tiles + q / ks;
    piece = q % ks;
  }
  int tm, tn;
  tile_coords(tile_id, tiles_m, tiles_n, tm, tn);
  const int col0 = tn * BN, row0 = tm * BM;
  const int rb0 = row0 >> 5, cb0 = col0 >> 5;
  const int G = K >> 6;
  const int S_all = G >> 1;
  const int sbase = piece < 0 ? 0 : piece * S_all / ks;                 // first stage
  const int S = piece < 0 ? S_all : (piece + 1) * S_all / ks - sbase;   // stages here


  // Copies of a stage (a 64-lane copy moves 1 KiB).  BM = 256: wave w copies A
  // row-block w (3 KiB: both groups); waves below CB copy B col-block w; wave CB the
  // row scale records (2 x 2 KiB), wave CB+1 the column scale records of the group
  // pair (BN * 8 bytes).  BM = 128: wave w copies blocks 2w and 2w+1 of the stage's 16
  // (A row-blocks 0-3, then B col-blocks 0-11; block b at 3 KiB x b in the slot),
  // waves 0 and 1 the row scale records of group 0 and 1 (1 KiB each), waves 2-4 one
  // KiB each of the column scale records.
  // Every source pointer is formed once and advances by a fixed stride per stage; the
  // KiB within a copy is a per-lane offset (voff + 1024 j) and the LDS destination (M0)
  // a fixed offset from the slot base, so a copy costs one scalar add for M0.  (s is the
  // stage relative to the piece's first.)
  const uint32_t voff = lane * 16;
  const uint32_t voff1 = voff + 1024, voff2 = voff + 2048;
  const uint32_t ring_lds = lds_addr(ring);
  // BM = 256
  const uint8_t* pA = A + ((size_t)(rb0 + (wave < NA ? wave : 0)) * G + 2 * sbase) * 1536;
  const uint8_t* pB = B + ((size_t)(cb0 + (wave < CB ? wave : 0)) * G + 2 * sbase) * 1536;
  // scale records: wave CB reads group 2s at pS and group 2s+1 M_pad records further
  // (voffS); wave CB+1 reads the BN records of pair s at pS
  const bool sa_wave = wave == CB;
  const uint8_t* pS = sa_wave ? reinterpret_cast<const uint8_t*>(sA + (size_t)2 * sbase * M_pad + row0)
                              : reinterpret_cast<const uint8_t*>(sB + (size_t)sbase * N + col0);
  const size_t strideS = sa_wave ? (size_t)2 * M_pad * 8 : (size_t)N * 8;
  const uint32_t voffS = voff + (uint32_t)M_pad * 8;
  const bool sb_tail_lane = lane < (BN - 128) / 2;
  // BM = 128
  const int blk = 2 * wave;
  const uint8_t* pX = blk < NA ? A + ((size_t)(rb0 + blk) * G + 2 * sbase) * 1536
                               : B + ((size_t)(cb0 + min(blk - NA, CB - 2)) * G + 2 * sbase) * 1536;
  const uint8_t* pX2 = pX + (size_t)G * 1536;
  const bool s_wave = wave < 5;
  const int sw = min(wave, 4);
  const uint8_t* pS2 =
      sw < 2 ? reinterpret_cast<const uint8_t*>(sA + ((size_t)2 * sbase + sw) * M_pad + row0)
             : reinterpret_cast<const uint8_t*>(sB + (size_t)sbase * N + col0) + (sw - 2) * 1024;
  const size_t strideS2 = sw < 2 ? (size_t)2 * M_pad * 8 : (size_t)N * 8;
  const uint32_t dS2 = sw < 2 ? (ASZ + BSZ) * 4 + sw * BM * 8 : (ASZ + BSZ + 4 * BM) * 4 + (sw - 2) * 1024;
  auto dma = [&](int s, int sl) {
    const uint32_t base = ring_lds + sl * (SLOT * 4);
    if constexpr (BM == 256) {
      const uint32_t da = base + wave * 3072;
      const uint8_t* a = pA + (size_t)s * 3072;
      dma16(voff, a, da);
      dma16(voff1, a, da + 1024);
      dma16(voff2, a, da + 2048);
      if (wave < CB) {
        const uint32_t db = base + (ASZ + wave * 768) * 4;
        const uint8_t* b = pB + (size_t)s * 3072;
        dma16(voff, b, db);
        dma16(voff1, b, db + 1024);
        dma16(voff2, b, db + 2048);
      } else if (sa_wave) {
        const uint32_t ds = base + (ASZ + BSZ) * 4;
        const uint8_t* c = pS + (size_t)s * strideS;
        dma16(voff, c, ds);
        dma16(voff1, c, ds + 1024);
        dma16(voffS, c, ds + BM * 8);
        dma16(voffS + 1024, c, ds + BM * 8 + 1024);
      } else if (wave == CB + 1) {
        const uint32_t ds = base + (ASZ + BSZ + 4 * BM) * 4;
        const uint8_t* c = pS + (size_t)s * strideS;
        dma16(voff, c, ds);
        if (BN > 128 && sb_tail_lane) dma16(voff1, c, ds + 1024);
      }
    } else {
      const uint32_t d0 = base + blk * 3072;
      const uint8_t* a = pX + (size_t)s * 3072;
      const uint8_t* b = pX2 + (size_t)s * 3072;
      dma16(voff, a, d0);
      dma16(voff1, a, d0 + 1024);
      dma16(voff2, a, d0 + 2048);
      dma16(voff, b, d0 + 3072);
      dma16(voff1, b, d0 + 4096);
      dma16(voff2, b, d0 + 5120);
      if (s_wave) dma16(voff, pS2 + (size_t)s * strideS2, base + dS2);
    }
  };

  // Copies for the late low-rank term: k-split sp of the tile's U (fragment layout: the
  // NA row blocks are contiguous, rank / 8 KiB each) to the start of slot sl, and with
  // split 0 lora_up's BN rows (BN * rank * 2 bytes) after it.  1 KiB per copy
  // instruction, spread over the 8 waves.
  const int u_kib = BM == 256 ? rank : rank / 2;  // KiB of the tile's U (one k-split)
  auto seed_copy = [&](int sp, int sl) {
    const uint8_t* u = reinterpret_cast<const uint8_t*>(U + u_frag_index(sp, row0, 0, M_pad, rank));
    const uint32_t dst = lds_addr(ring + sl * SLOT);
    for (int p = wave; p < u_kib; p += 8) dma16(voff, u + p * 1024, dst + p * 1024);
    if (sp == 0) {
      const uint8_t* l = reinterpret_cast<const uint8_t*>(L2t + (size_t)col0 * rank);
      for (int p = wave; p < BN * rank / 512; p += 8)
        dma16(voff, l + p * 1024, dst + u_kib * 1024 + p * 1024);
    }
  };

  dma(0, 0);
  if (1 < S) dma(1, 1);

  v16f acc[2][WN];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // Low-rank term acc^T += L2t U^T.  U (fp32, the sum of the quantizer's k-split
  // partials in split order) is split into three bf16 terms (split3_bf16), which
  // leave less than 2^-27 |u|.  rank <= 32: at most two 16-rank slices.  With at
  // most two k-splits and three stages or more, U and lora_up are copied into the ring
  // slots that the last two stages leave free and the term is added in the epilogue;
  // otherwise it seeds the accumulator here, from global memory.
  // (A split tile takes the term in piece 0, before its loop.)
  const bool late_seed = rank > 0 && nsplit <= 2 && S >= 3 && piece < 0;
  if (rank > 0 && !late_seed && piece <= 0) {
    uint4 lbv[2][WN];
    float uf[2][2][8];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 8; ++q) uf[kk][i][q] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
      if (16 * kk < rank)
#pragma unroll
        for (int j = 0; j < WN; ++j) {
          const int coln = col0 + (wn * WN + j) * 32 + lr;
          lbv[kk][j] = *reinterpret_cast<const uint4*>(L2t + (size_t)coln * rank + 16 * kk + 8 * lh);
        }
    for (int sp = 0; sp < nsplit; sp += 2) {
      float4 tv[2][2][2][2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
        if (sp + s2 < nsplit)
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
            if (16 * kk < rank)
#pragma unroll
              for (int i = 0; i < 2; ++i) {
                const float* up =
                    U + u_frag_index(sp + s2, row0 + wm * 64 + 32 * i, 16 * kk, M_pad, rank) + lane * 4;
                tv[s2][kk][i][0] = *reinterpret_cast<const float4*>(up);
                tv[s2][kk][i][1] = *reinterpret_cast<const float4*>(up + 256);
              }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
        if (sp + s2 < nsplit)
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
            if (16 * kk < rank)
#pragma unroll
              for (int i = 0; i < 2; ++i) {
                const float4 a0 = tv[s2][kk][i][0], a1 = tv[s2][kk][i][1];
                uf[kk][i][0] += a0.x; uf[kk][i][1] += a0.y; uf[kk][i][2] += a0.z; uf[kk][i][3] += a0.w;
                uf[kk][i][4] += a1.x; uf[kk][i][5] += a1.y; uf[kk][i][6] += a1.z; uf[kk][i][7] += a1.w;
              }
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      if (16 * kk < rank) {
        v8bf uh[2], um[2], ul[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const Bf16x3 t = split3_bf16(uf[kk][i][q]);
            uh[i][q] = t.h;
            um[i][q] = t.m;
            ul[i][q] = t.l;
          }
#pragma unroll
        for (int j = 0; j < WN; ++j) {
          const v8bf lv = __builtin_bit_cast(v8bf, lbv[kk][j]);
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lv, uh[i], acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lv, um[i], acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lv, ul[i], acc[i][j], 0, 0, 0);
          }
        }
      }
    }
  }

  const v16f zero = {};
  // LDS byte addresses of a ring slot with the lane, wave and slot parts folded in,
  // formed once per stage and hidden from the optimizer (an empty asm), so that each
  // read below is one of these registers plus an immediate offset
  struct Bases { uint32_t a16, a8, a8b, b16, b8, sa, sb; };
  const uint32_t ring0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint32_t*)ring;
  auto bases = [&](int sl) {
    Bases r;
    const uint32_t so = ring0 + sl * SLOT * 4;
    r.a16 = so + (wm * 4 * 384 + lane * 4) * 4;
    r.a8 = so + (wm * 4 * 384 + 256 + lane * 2) * 4;
    r.a8b = r.a8 + 2 * 384 * 4;
    r.b16 = so + (ASZ + wn * WN * 2 * 384 + lane * 4) * 4;
    r.b8 = so + (ASZ + wn * WN * 2 * 384 + 256 + lane * 2) * 4;
    r.sa = so + (ASZ + BSZ + 2 * (wm * 64 + lr)) * 4;
    r.sb = so + (ASZ + BSZ + 4 * BM + 2 * (wn * WN * 32 + lr)) * 4;
    // a8b (the second A row-block's 8-byte halves) is a register of its own, so the two
    // halves are not merged into one ds_read2 whose result would need moves
    asm volatile("" : "+v"(r.a16), "+v"(r.a8), "+v"(r.a8b), "+v"(r.b16), "+v"(r.b8), "+v"(r.sa),
                 "+v"(r.sb));
    return r;
  };
  typedef __attribute__((address_space(3))) const v4i lds_v4i;
  typedef __attribute__((address_space(3))) const v2i lds_v2i;
  auto frag = [&](uint32_t p16, int off16, uint32_t p8, int off8) {
    const v4i lo = *(lds_v4i*)(uintptr_t)(p16 + off16 * 4);
    const v2i hi = *(lds_v2i*)(uintptr_t)(p8 + off8 * 4);
    return (v8i)__builtin_shufflevector(lo, __builtin_shufflevector(hi, hi, 0, 1, -1, -1), 0, 1, 2,
                                        3, 4, 5, -1, -1);
  };
  // register sets: A fragments and row scales by group parity; B fragment k = gl WN + j
  // (2 WN per stage) and its column scale record in set k % NBS (the record of j is
  // loaded with the even group's fragment and serves the odd group's as well)
  v8i fa[2][2], fb[NBS];
  v2i fsa[2][2], fsb[NBS];
  auto loadA = [&](int set, const Bases& q, int gl) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      fa[set][i] = frag(q.a16, (i * 2 + gl) * 384, i == 0 ? q.a8 : q.a8b, gl * 384);
      fsa[set][i] = *(lds_v2i*)(uintptr_t)(q.sa + (gl * BM + 32 * i) * 8);
    }
  };
  auto loadB = [&](int k, const Bases& q) {
    const int gl = k / WN, j = k % WN;
    fb[k % NBS] = frag(q.b16, (j * 2 + gl) * 384, q.b8, (j * 2 + gl) * 384);
    if (gl == 0) fsb[k % NBS] = *(lds_v2i*)(uintptr_t)(q.sb + j * 32 * 8);
    else if (NBS != WN) fsb[k % NBS] = fsb[(k - WN) % NBS];
  };
  v16f d[2], sc[2];
  // block b of a stage: group b / (2 WN), column block (b % (2 WN)) / 2, row block b % 2
  auto issue = [&](int b) {
    const int gl = b / (2 * WN), j = (b % (2 * WN)) / 2, i = b % 2;
    const int k = gl * WN + j;
    d[b & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[k % NBS], fa[gl][i], zero, 2, 2, 0,
                                                               129, 0, 130);
    sc[b & 1] = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(
        __builtin_bit_cast(v4bf, fsb[k % NBS]), __builtin_bit_cast(v4bf, fsa[gl][i]), zero, 0, 0, 0);
  };

  // stages 0 and 1 landed for every wave
  wait_vm0();
  barrier_lds();
  {
    const Bases q0 = bases(0);
    loadA(0, q0, 0);
    loadB(0, q0);
    loadB(1, q0);
  }
  issue(0);
  __builtin_amdgcn_sched_barrier(0);

  // Step b: MFMAs of block b+1, rescale of block b, then loads.  B fragment k is loaded
  // at step 2k - 3 (the next stage's first two at steps NB-3 and NB-1), the odd-group
  // A fragments at step 0, the next stage's even-group A fragments at step NB/2 (the
  // last use of that set is the issue of block NB/2 - 1).
  auto step = [&](int b, const Bases& cq, const Bases& nq, bool next) {
    const int j = (b % (2 * WN)) / 2, i = b % 2;
    if (b + 1 < NB) issue(b + 1);
    else if (next) issue(0);
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][j][e] = __builtin_fmaf(sc[b & 1][e], d[b & 1][e], acc[i][j][e]);
    if (b & 1) {
      const int k = (b + 3) / 2;
      if (k < 2 * WN) loadB(k, cq);
      else if (next) loadB(k - 2 * WN, nq);
    }
    if (b == 0) loadA(1, cq, 1);
    if (b == NB / 2 && next) loadA(0, nq, 0);
    // issue order within the step: D, the fragment loads, half the FMAs, S, the rest
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 24, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  // stage t sits in slot sl0 = t % 3 (tracked without a division)
  int sl0 = 0;
  for (int t = 0; t + 1 < S; ++t) {
    const int sl1 = sl0 == 2 ? 0 : sl0 + 1, sl2 = sl1 == 2 ? 0 : sl1 + 1;
    if (t > 0) {
      wait_vm0();
      barrier_lds();
    }
    if (t + 2 < S) dma(t + 2, sl2);
    else if (late_seed) seed_copy(0, sl2);
    __builtin_amdgcn_sched_barrier(0);
    const Bases cq = bases(sl0), nq = bases(sl1);
#pragma unroll
    for (int b = 0; b < NB; ++b) step(b, cq, nq, true);
    sl0 = sl1;
  }
  {
    const int t = S - 1;
    if (t > 0) {
      wait_vm0();
      barrier_lds();
    }
    // the tile's bias goes to LDS under the last stage (wave 0, 16 B per lane), and
    // the second k-split of U to the slot stage t-1 has just freed
    if (bias && wave == 0 && lane < BN / 8) dma16(voff, bias + col0, lds_addr(bias_s));
    if (late_seed && nsplit == 2) seed_copy(1, sl0 == 0 ? 2 : sl0 - 1);
    const Bases cq = bases(sl0);
#pragma unroll
    for (int b = 0; b < NB; ++b) step(b, cq, cq, false);
    // keeps the last rescale ahead of the epilogue
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j) asm volatile("" : "+v"(acc[i][j]));
  }

  if (piece >= 0) {
    // Partial tile of this piece: block (wave, i, j) is 4 KiB, float4 q of lane l at
    // 16 (64 q + l) bytes, so each store instruction of a wave writes 1 KiB in a row.
    // The bias copy of the last stage lands before the wave exits.
    wait_vm0();
    float* dst = part_tile(part, tile_id - full_tiles, piece, ks, BM * BN);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        float4* d4 = reinterpret_cast<float4*>(dst + ((wave * 2 + i) * WN + j) * 1024) + lane;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          d4[64 * q] = make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                   acc[i][j][4 * q + 3]);
      }
    return;
  }

  // Epilogue: + bias, round to bf16.  Each wave stages its 64 x WC tile in LDS (the
  // ring is free once every wave has passed the barrier) and writes Y in 16-byte
  // pieces, WC/8 consecutive lanes per row, so every row segment of the tile is one
  // contiguous run of full 64-byte sectors.
  wait_vm0();
  barrier_lds();
  // Fused QKV epilogue, Q and K tiles: the tile's rows of the rotary table (128 floats
  // each) and both channel-weight vectors are copied into the ring by LDS DMA here, so
  // that the copy overlaps the low-rank MFMAs below.  They go where those MFMAs' copies
  // are not: row pairs 0..kPairsA-1 into the slot of the last stage (free after the
  // barrier above), the rest, the weights (q, then k) and the per-row sums of squares
  // red[cb][row] of the epilogue into slot (S+1) % 3 past the 16 KiB of the second
  // U split.  Rows 2p and 2p+1 of a pair are 512 bytes apart, pairs 1040 bytes (the
  // 16-byte pad spreads the rows of one read over the banks).
  [[maybe_unused]] constexpr int kPairsA = 48;
  [[maybe_unused]] const bool qk_tile = EPI == kEpiQkNormRope && col0 < 2 * (N / 3);
  [[maybe_unused]] const uint32_t rope_a = ((S + 2) % 3) * SLOT * 4;  // slot of stage S-1
  [[maybe_unused]] const uint32_t rope_b = ((S + 1) % 3) * SLOT * 4 + 16384;
  [[maybe_unused]] const uint32_t nw_off = rope_b + (BM / 2 - kPairsA) * 1040;
  [[maybe_unused]] const uint32_t red_off = nw_off + 512;
  if constexpr (EPI == kEpiQkNormRope) {
    static_assert(kPairsA * 1040 <= SLOT * 4 && 16384 + (BM / 2 - kPairsA) * 1040 + 512 + CB * BM * 4 <= SLOT * 4,
                  "the tables fit the free ring");
    if (qk_tile) {
      // rows at or past M (not stored) read row M-1; offsets from row rb = min(row0, M-1)
      const int rb = min(row0, M - 1);
      const uint8_t* rope_t = reinterpret_cast<const uint8_t*>(qk.rope + (size_t)rb * 128);
      const uint32_t base = lds_addr(ring);
#pragma unroll
      for (int t = 0; t < BM / 16; ++t) {  // row pairs p = wave + 8 t
        const int pr = wave + 8 * t;
        const int r = min(row0 + 2 * pr + lh, M - 1) - rb;  // 0 <= r < BM
        const uint32_t dst = pr < kPairsA ? rope_a + pr * 1040 : rope_b + (pr - kPairsA) * 1040;
        dma16((uint32_t)r * 512u + (uint32_t)lr * 16u, rope_t, base + dst);
      }
      if (wave == 0 && lane < 16) {
        dma16(voff, qk.norm_q, base + nw_off);
        dma16(voff, qk.norm_k, base + nw_off + 256);
      }
    }
  }
  if (late_seed) {
    // split 0 and lora_up were copied at the top of stage S-2 into slot S % 3, split 1
    // at the top of stage S-1 into slot (S+1) % 3
    typedef __attribute__((address_space(3))) const v4f lds_f4;
    const uint32_t s0 = lds_addr(ring + (S % 3) * SLOT), s1 = lds_addr(ring + ((S + 1) % 3) * SLOT);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      if (16 * kk < rank) {
        v8bf uh[2], um[2], ul[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const uint32_t o = ((wm * 2 + i) * (rank >> 4) + kk) * 2048 + lane * 16;
          v4f a0 = *(lds_f4*)(uintptr_t)(s0 + o), a1 = *(lds_f4*)(uintptr_t)(s0 + o + 1024);
          if (nsplit == 2) {
            a0 += *(lds_f4*)(uintptr_t)(s1 + o);
            a1 += *(lds_f4*)(uintptr_t)(s1 + o + 1024);
          }
          const float uf[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const Bf16x3 t = split3_bf16(uf[q]);
            uh[i][q] = t.h;
            um[i][q] = t.m;
            ul[i][q] = t.l;
          }
        }
        v8bf lv[WN];
#pragma unroll
        for (int j = 0; j < WN; ++j) {
          const uint32_t lo = s0 + u_kib * 1024 + ((wn * WN + j) * 32 + lr) * rank * 2 + kk * 32 + lh * 16;
          lv[j] = __builtin_bit_cast(v8bf, *(lds_v4i*)(uintptr_t)lo);
        }
        // the hi products of all blocks, then the mid and lo ones: an accumulator's
        // MFMAs are 2 WN apart instead of back to back
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < WN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lv[j], uh[i], acc[i][j], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < WN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lv[j], um[i], acc[i][j], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < WN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lv[j], ul[i], acc[i][j], 0, 0, 0);
      }
    }
    barrier_lds();  // the staging tiles below overwrite the seed copies
  }
  // bias of the lane's 16 columns of block j (column 32 j' + 8 q + 4 lh + p of the
  // tile, j' = wn WN + j)
  auto bias16 = [&](int j, float (&bv)[16]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint2 b2 = bias ? *reinterpret_cast<const uint2*>(bias_s + (wn * WN + j) * 32 + 8 * q + 4 * lh)
                            : make_uint2(0, 0);
      bv[4 * q + 0] = __uint_as_float(b2.x << 16);
      bv[4 * q + 1] = __uint_as_float(b2.x & 0xFFFF0000u);
      bv[4 * q + 2] = __uint_as_float(b2.y << 16);
      bv[4 * q + 3] = __uint_as_float(b2.y & 0xFFFF0000u);
    }
  };
  uint16_t* tile = reinterpret_cast<uint16_t*>(ring) + wave * (64 * (WC + 8));
  // block (i, j) rounded to bf16 into the wave's staging tile
  auto stage = [&](int i, int j, const float (&v)[16]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t h[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) h[p] = f32_to_bf16_rne(v[4 * q + p]);
      *reinterpret_cast<uint2*>(tile + (32 * i + lr) * (WC + 8) + 32 * j + 8 * q + 4 * lh) =
          make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
    }
  };
  bool staged = false;
  if constexpr (EPI == kEpiQkNormRope) {
    // Q and K heads: RMSNorm over the head's 128 columns of a row, the channel weights,
    // then the rotary turn of adjacent column pairs by the row's angles; V heads take
    // the bias only.  Column block cb of the tile is part of the tile's head cb / 4, a
    // Q, K or V head by its columns (the first, second and last N/3).  qk_tile is
    // tile-uniform, so the barriers below are reached by every wave or by none.
    //
    // Pass 1 adds the bias and forms each block's per-row sums of squares; pass 2
    // normalises and turns the Q and K blocks in registers, reading the tables copied at
    // the top of the epilogue from LDS; a barrier then frees the ring for the staging
    // tiles.
    if (qk_tile) {
      const int third = N / 3;
      uint8_t* lds = reinterpret_cast<uint8_t*>(ring);
      float* red = reinterpret_cast<float*>(lds + red_off);
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        float bv[16];
        bias16(j, bv);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          float ss = 0.f;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float v = acc[i][j][e] + bv[e];
            acc[i][j][e] = v;
            ss = fmaf(v, v, ss);
          }
          // the lane pair (l, l + 32) holds one row's 16 + 16 columns of the block
          ss += __shfl_xor(ss, 32);
          if (lh == 0) red[(wn * WN + j) * BM + wm * 64 + 32 * i + lr] = ss;
        }
      }
      wait_vm0();
      barrier_lds();
      // Lane element 4q + p of block j is channel c = 32 (cb % 4) + 8 q + 4 lh + p of its
      // head, so its four channels are the pairs c/2 and c/2 + 1 (one 16-byte read of
      // cos, sin).
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const int cb = wn * WN + j, c0 = col0 + 32 * cb;
        if (c0 >= 2 * third) continue;  // a V block (wave-uniform)
        const int h0 = cb & ~3;          // the head's first column block
        const uint16_t* nw = reinterpret_cast<const uint16_t*>(lds + nw_off + (c0 < third ? 0 : 256));
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int rr = wm * 64 + 32 * i + lr;
          const float tot = ((red[h0 * BM + rr] + red[(h0 + 1) * BM + rr]) + red[(h0 + 2) * BM + rr]) +
                            red[(h0 + 3) * BM + rr];
          const float inv = 1.0f / sqrtf(tot * (1.0f / 128.0f) + qk.eps);
          const int pr = rr >> 1;
          const float* rrow = reinterpret_cast<const float*>(
              lds + (pr < kPairsA ? rope_a + pr * 1040 : rope_b + (pr - kPairsA) * 1040) + (rr & 1) * 512);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int c = 32 * (cb & 3) + 8 * q + 4 * lh;
            const uint2 w2 = *reinterpret_cast<const uint2*>(nw + c);
            const float w[4] = {__uint_as_float(w2.x << 16), __uint_as_float(w2.x & 0xFFFF0000u),
                                __uint_as_float(w2.y << 16), __uint_as_float(w2.y & 0xFFFF0000u)};
            const float4 cs = *reinterpret_cast<const float4*>(rrow + c);
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
      barrier_lds();  // the staging tiles overwrite the tables
#pragma unroll
      for (int j = 0; j < WN; ++j)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          float v[16];
#pragma unroll
          for (int e = 0; e < 16; ++e) v[e] = acc[i][j][e];
          stage(i, j, v);
        }
      staged = true;
    }
  }
  if (!staged) {
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      float bv[16];
      bias16(j, bv);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        float v[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float x = acc[i][j][e] + bv[e];
          v[e] = EPI == kEpiGelu ? gelu_f32(x) : x;
        }
        stage(i, j, v);
      }
    }
  }
  constexpr int CPR = WC / 8;  // 16-byte pieces per staged row
#pragma unroll
  for (int r = 0; r < CPR; ++r) {
    const int c = lane + 64 * r;
    const int row = c / CPR, ch = c % CPR;
    const uint4 v = *reinterpret_cast<const uint4*>(tile + row * (WC + 8) + ch * 8);
    const int grow = row0 + wm * 64 + row;
    if (grow < M) {
      uint16_t* yp = Y + (size_t)grow * N + col0 + wn * WC + ch * 8;
      if (y_wt) store_wt(yp, v);
      else *reinterpret_cast<uint4*>(yp) = v;
    }
  }
}

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Plan by a cost model in units of one 192-wide stage (about 1.3 us on MI355X): a
// tile costs S u + 4 (u = 1 for 256 x 192 and 128 x 384 tiles, whose waves do the same
// work, 0.76 for 256 x 128; 4 for the fill, drain and epilogue), a round of tiles
// costs one tile, and a split tail costs one piece plus 8 (its partial stores, the
// second kernel and its launch).  Pieces have at least 4 stages; the split is taken
// when it is 3 % cheaper than the best whole-tile plan.  The constants are fitted to
// the DiT shapes at 4096 and 4608 tokens.  The fused QKV epilogue takes the 128 x 384
// tile (three whole heads), the others 256 x 192 or 256 x 128.
K2Plan plan_k2_int4(int M_pad, int N, int K, int epi, int max_pieces) {
  const int cus = device_cu_count();
  const int S = K / 128;
  K2Plan best, best_split;
  double best_whole = 1e30;
  double split_cost = 1e30;
  struct Shape { int bm, bn; double u; };
  static constexpr Shape kPlain[] = {{256, 192, 1.0}, {256, 128, 0.76}};
  static constexpr Shape kQkv[] = {{128, 384, 1.0}};
  const bool qkv = epi == kEpiQkNormRope;
  for (int c = 0; c < (qkv ? 1 : 2); ++c) {
    const Shape sh = qkv ? kQkv[c] : kPlain[c];
    if (N % sh.bn != 0 || M_pad % sh.bm != 0) continue;
    const double tile = S * sh.u + 4.0;
    const int tiles = (N / sh.bn) * (M_pad / sh.bm);
    const double whole = (double)((tiles + cus - 1) / cus) * tile;
    if (whole < best_whole) {
      best_whole = whole;
      best.bm = sh.bm;
      best.bn = sh.bn;
      best.tiles = best.full = tiles;
      best.ks = 1;
    }
    const int rem = tiles % cus;
    if (max_pieces > 0 && rem > 0) {
      const int ks = std::min({cus / rem, S / 4, max_pieces / rem, 16});
      if (ks >= 2) {
        const double cost = (double)(tiles / cus) * tile + (double)S / ks * sh.u + 4.0 + 8.0;
        if (cost < split_cost) {
          split_cost = cost;
          best_split.bm = sh.bm;
          best_split.bn = sh.bn;
          best_split.tiles = tiles;
          best_split.full = tiles - rem;
          best_split.ks = ks;
        }
      }
    }
  }
  return split_cost < 0.97 * best_whole ? best_split : best;
}

// Finishes the split tiles: workgroup (tail tile t, row block rb = 32 rows, column
// part cp of CW columns: the whole tile, or one head of the 128 x 384 QKV tile) adds
// the ks partial tiles in piece order, then runs the epilogue (bias, GELU or the Q/K
// norm and rotation) and stores the 32 rows of the part.  Phase 1 reads the partials in
// their stored order (a wave's float4 loads are 1 KiB in a row) and puts the sums into
// an LDS tile of 32 rows x CW; phase 2 gives each row to 8 consecutive threads.
template <int BM, int BN, int EPI>
__global__ void __launch_bounds__(256)
k2_tail_int4(const float* __restrict__ part, int ks, int full_tiles, int tiles_m, int tiles_n,
             const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y, int M, int N,
             QkEpi qk) {
  constexpr int WMW = BM / 64, WNW = 8 / WMW, WN = BN / WNW / 32;  // the GEMM's wave grid
  constexpr int CW = BN == 384 ? 128 : BN, NP = BN / CW;  // columns per workgroup, parts
  constexpr int NRB = BM / 32, C4 = CW / 4, LD = CW + 4;
  __shared__ __attribute__((aligned(16))) float T[32 * LD];
  const int t = blockIdx.x / (NRB * NP), rb = (blockIdx.x / NP) % NRB, cp = blockIdx.x % NP;
  const int wm = rb >> 1, i = rb & 1;  // rb = 2 wm + i of the GEMM
  const int tid = threadIdx.x;
  int tm, tn;
  tile_coords(full_tiles + t, tiles_m, tiles_n, tm, tn);
  const int row0 = tm * BM + 32 * rb, col0 = tn * BN + cp * CW;  // col0: the part's first column
  {
    // thread (q, lane) of every block cb = wn WN + j of this part: row lane % 32,
    // columns 32 cb + 8 q + 4 (lane / 32) + [0, 4) of the tile
    const int q = tid >> 6, lane = tid & 63;
#pragma unroll
    for (int c = 0; c < CW / 32; ++c) {
      const int cb = cp * (CW / 32) + c, wn = cb / WN, j = cb % WN;
      const size_t off = (size_t)(((wm * WNW + wn) * 2 + i) * WN + j) * 1024 + (64 * q + lane) * 4;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
      for (int p = 0; p < ks; ++p) {
        const float4 x = *reinterpret_cast<const float4*>(part + (size_t)(t * ks + p) * (BM * BN) + off);
        v.x += x.x;
        v.y += x.y;
        v.z += x.z;
        v.w += x.w;
      }
      *reinterpret_cast<float4*>(&T[(lane & 31) * LD + 32 * c + 8 * q + 4 * (lane >> 5)]) = v;
    }
  }
  __syncthreads();
  // row r = tid / 8 of the block; float4 columns sub + 8 k
  const int r = tid >> 3, sub = tid & 7;
  const int row = row0 + r;
  constexpr int NK = C4 / 8;
  float v[NK][4];
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    const int c = 4 * (sub + 8 * k);
    const float4 x = *reinterpret_cast<const float4*>(&T[r * LD + c]);
    v[k][0] = x.x;
    v[k][1] = x.y;
    v[k][2] = x.z;
    v[k][3] = x.w;
    if (bias) {
      const uint2 b2 = *reinterpret_cast<const uint2*>(bias + col0 + c);
      v[k][0] += __uint_as_float(b2.x << 16);
      v[k][1] += __uint_as_float(b2.x & 0xFFFF0000u);
      v[k][2] += __uint_as_float(b2.y << 16);
      v[k][3] += __uint_as_float(b2.y & 0xFFFF0000u);
    }
  }
  if constexpr (EPI == kEpiQkNormRope) {
    // head h of the part (128 columns) is this thread's float4 columns k = 4h .. 4h + 3,
    // channels 4 (sub + 8 (k - 4h)) of the head, so every head takes the same four
    // (cos, sin) float4s of the row; the sums of squares of a head's row meet across
    // the row's 8 threads
    constexpr int NH = CW / 128;
    const int third = N / 3;
    float4 rcs[4];
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4)
      rcs[a4] = *reinterpret_cast<const float4*>(qk.rope + (size_t)min(row, M - 1) * 128 + 4 * (sub + 8 * a4));
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const int c0 = col0 + 128 * h;
      if (c0 >= 2 * third) continue;  // a V head (workgroup-uniform)
      float ss = 0.f;
#pragma unroll
      for (int k = 4 * h; k < 4 * h + 4; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) ss = fmaf(v[k][e], v[k][e], ss);
#pragma unroll
      for (int d = 1; d < 8; d <<= 1) ss += __shfl_xor(ss, d, 8);
      const float inv = 1.0f / sqrtf(ss * (1.0f / 128.0f) + qk.eps);
      const uint16_t* nw = c0 < third ? qk.norm_q : qk.norm_k;
#pragma unroll
      for (int k = 4 * h; k < 4 * h + 4; ++k) {
        const int c = 4 * (sub + 8 * k) - 128 * h;  // channel within the head
        const uint2 w2 = *reinterpret_cast<const uint2*>(nw + c);
        const float w[4] = {__uint_as_float(w2.x << 16), __uint_as_float(w2.x & 0xFFFF0000u),
                            __uint_as_float(w2.y << 16), __uint_as_float(w2.y & 0xFFFF0000u)};
        const float4 cs = rcs[k - 4 * h];
        float n[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) n[e] = v[k][e] * inv * w[e];
        v[k][0] = n[0] * cs.x - n[1] * cs.y;
        v[k][1] = n[1] * cs.x + n[0] * cs.y;
        v[k][2] = n[2] * cs.z - n[3] * cs.w;
        v[k][3] = n[3] * cs.z + n[2] * cs.w;
      }
    }
  }
  if (row < M) {
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      uint32_t h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) h[e] = f32_to_bf16_rne(EPI == kEpiGelu ? gelu_f32(v[k][e]) : v[k][e]);
      *reinterpret_cast<uint2*>(Y + (size_t)row * N + col0 + 4 * (sub + 8 * k)) =
          make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
    }
  }
}

hipError_t launch_k2_int4(const K2Plan& plan, const uint8_t* A, const uint2* sA, const float* U,
                          int nsplit, const uint8_t* B, const uint2* sB, const uint16_t* L2t,
                          const uint16_t* bias, uint16_t* Y, int M, int N, int K, int M_pad,
                          int rank, int epi, const QkEpi& qk, float* part, hipStream_t st,
                          hipEvent_t ev0, hipEvent_t ev1, hipEvent_t ev2, hipEvent_t ev3) {
  const bool qkv = epi == kEpiQkNormRope;
  const bool shape_ok = qkv ? plan.bm == 128 && plan.bn == 384
                            : plan.bm == 256 && (plan.bn == 192 || plan.bn == 128);
  if (!shape_ok || M_pad % 256 != 0 || N % plan.bn != 0 || K % 128 != 0) return hipErrorInvalidValue;
  if (qkv && (!qk.norm_q || !qk.norm_k || !qk.rope)) return hipErrorInvalidValue;
  const bool split = plan.ks > 1;
  if (split && (!part || (int64_t)(plan.tiles - plan.full) * plan.ks > kSplitMaxPieces))
    return hipErrorInvalidValue;
  const bool wide = plan.bn == 192;
  const unsigned g = (unsigned)(plan.full + (plan.tiles - plan.full) * plan.ks);
  auto k = qkv ? k2_gemm_int4<128, 384, kEpiQkNormRope>
           : wide ? (epi == kEpiGelu ? k2_gemm_int4<256, 192, kEpiGelu> : k2_gemm_int4<256, 192, kEpiPlain>)
                  : (epi == kEpiGelu ? k2_gemm_int4<256, 128, kEpiGelu> : k2_gemm_int4<256, 128, kEpiPlain>);
  // Y written through the L2 at device scope when every tile runs in the one round: then
  // all tiles store at the end together and nothing is left for the release at the
  // kernel's end to write back (C2, same box: 51.6-52.1 -> 51.0-51.5 us per call).  With
  // more rounds the write-through stores of finished tiles load the fabric under the
  // other tiles' main loops (QKV +1.5, MLP-up +2.2 us), so they keep plain stores.
  const int y_wt = !split && g <= (unsigned)device_cu_count();
  hipExtLaunchKernelGGL(k, dim3(g), dim3(512), 0, st, ev0, ev1, 0, A, sA, U, nsplit, B, sB, L2t,
                        bias, Y, M, N, K, M_pad, rank, qk, plan.full, plan.ks, part, y_wt);
  if (split) {
    const unsigned gt = (unsigned)((plan.tiles - plan.full) * (plan.bm / 32) * (plan.bn == 384 ? 3 : 1));
    auto kt = qkv ? k2_tail_int4<128, 384, kEpiQkNormRope>
              : wide ? (epi == kEpiGelu ? k2_tail_int4<256, 192, kEpiGelu> : k2_tail_int4<256, 192, kEpiPlain>)
                     : (epi == kEpiGelu ? k2_tail_int4<256, 128, kEpiGelu> : k2_tail_int4<256, 128, kEpiPlain>);
    hipExtLaunchKernelGGL(kt, dim3(gt), dim3(256), 0, st, ev2, ev3, 0, part, plan.ks, plan.full,
                          M_pad / plan.bm, N / plan.bn, bias, Y, M, N, qk);
  }
  return hipGetLastError();
}

}  // namespace svdq
