// K4: the AWQ W4A16 comparison layer.
//
//   Y[m,n] = bf16( sum_g s[n,g] D_g[m,n] + b[n] ),  D_g = sum_{k in g} x[m,k] (q[n,k] - z[n,g])
//
// (Diffusers docs "Nunchaku Lite", "Supported quantization types": awq_w4a16, INT4
// weight-only, group 64.)  The weights stay 4-bit in HBM and in LDS.  Per 64-group the
// workgroup expands its BN x 64 weight slice into the exact bf16 values q - z (integers
// in [-15, 15]), the bf16 MFMA forms D_g in fp32 (four k-chunks of 16 chained on one
// accumulator), and one fp32 FMA per output element applies the group scale:
// acc = fma(s, D_g, acc).
//
// Tiling: one 512-thread workgroup (8 waves, two per SIMD) per CU, tile 256 x BN with
// BN = 64 WN (192 where N allows, else 128), wave tile 64 x BN/2 (2 x WN blocks of
// 32 x 32).  The accumulators are held in the MFMA's own orientation: lane l % 32 is
// the output column, so a block's group scale and bias are one value per lane.  A
// stage is one 64-group.  LDS holds two activation tiles (256 x 64 bf16, 16-byte units
// swizzled as u = row 8 + (c ^ ((row / 2) & 7)), c = k / 8, so that the sixteen lanes
// a fragment read serves at once, two rows per 256 bytes of the 64 banks, hit distinct
// banks), three raw weight slices (BN x 32 bytes of nibbles) and two expanded weight
// tiles (BN x 64 bf16, the same swizzle by column).  At the top of stage t every wave waits for its own copies, one barrier
// publishes them together with the weight tile expanded during stage t - 1, and the
// copies of stage t + 1's activations and stage t + 2's nibbles start (LDS DMA, 16
// bytes per lane), after the global loads of the next group's scales and the zero
// points of the group after it.  A wave then reads its stage's activation fragments (kept
// in registers for the stage), then per column block its weight fragments, the MFMAs,
// the scale FMAs and one unit of its share of stage t + 1's weight expansion.
// Rows of X at or past M read row M - 1 (their outputs are not stored).  The tile
// order is XCD-aware (tile_coords in k2_common.h).
#include "common.h"
#include "k2_common.h"
#include "kernels.h"

namespace svdq {

template <int WN, int W>
__global__ void __launch_bounds__(512, 1)
k4_gemm_awq(const uint16_t* __restrict__ X, const uint8_t* __restrict__ Q,
            const uint16_t* __restrict__ Sc, const uint8_t* __restrict__ Z,
            const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y, int M, int N, int K,
            int y_wt) {
  constexpr int BM = 256, BN = 64 * WN;
  constexpr int AB = BM * 128;         // bytes of an activation tile (256 x 64 bf16)
  constexpr int QB = BN * 32;          // bytes of a raw weight slice (BN x 64 nibbles)
  constexpr int WB = BN * 128;         // bytes of an expanded weight tile (BN x 64 bf16)
  constexpr int OFF_Q = 2 * AB, OFF_W = OFF_Q + 3 * QB, LDS = OFF_W + 2 * WB;
  constexpr int UPL = WN;              // expansion units (8 values) per lane and stage
  constexpr int TS = BN / 2 + 8;       // row pitch (bf16) of a wave's staging tile
  static_assert(WN == 2 || WN == 3, "tile width 128 or 192");
  static_assert(8 * 64 * TS * 2 <= LDS, "staging tiles fit in the freed LDS");
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, lr = lane & 31, lh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_n = N / BN, tiles_m = (M + BM - 1) / BM;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int row0 = tm * BM, col0 = tn * BN;
  const int G = K >> 6;
  const uint32_t lds0 = lds_addr(lds);

  // Copies.  Activations: wave w moves 16-byte units (4w + t) 64 + lane, t < 4, i.e.
  // rows 32w + 8t + lane / 8, chunk (lane % 8) ^ ((row / 2) % 8); the source is a fixed
  // per-lane offset from a per-stage base.  Weight nibbles: wave j < QB / 1 KiB moves
  // units 64 j + lane (column u / 2, half u % 2).
  const uint8_t* xbase = reinterpret_cast<const uint8_t*>(X) + (size_t)row0 * K * 2;
  uint32_t voffA[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int r = 32 * wave + 8 * t + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    voffA[t] = (uint32_t)(min(row0 + r, M - 1) - row0) * (uint32_t)K * 2u + 16u * c;
  }
  const uint8_t* qbase = Q + (size_t)col0 * (K / 2);
  const bool q_wave = wave < QB / 1024;
  const uint32_t voffQ = (uint32_t)(((64 * wave + lane) >> 1) * (K / 2) + 16 * (lane & 1));
  auto dma_a = [&](int g, int sl) {
    const uint8_t* src = xbase + (size_t)g * 128;
    const uint32_t dst = lds0 + sl * AB + wave * 4096;
#pragma unroll
    for (int t = 0; t < 4; ++t) dma16(voffA[t], src, dst + 1024 * t);
  };
  auto dma_q = [&](int g, int sl) {
    if (q_wave) dma16(voffQ, qbase + (size_t)g * 32, lds0 + OFF_Q + sl * QB + wave * 1024);
  };

  // Expansion units of this lane: u = 64 (UPL wave + t) + lane, column u / 8, values
  // 8 (u % 8) .. + 8 of the group.  Their zero points, and this lane's output columns'
  // scales, are read from global memory W groups at a time (W = 8 when K / 64 allows,
  // else 2; scales and zero points are stored column-major, [N][K/64]) into small
  // register queues that shift by one group per stage.  The offsets are 32-bit from the
  // tile's first column (the empty asm keeps them opaque, so the compiler does not turn
  // them into per-lane 64-bit pointers that advance with the group).
  constexpr int SD = W / 2;  // dwords of scales per column and load (W bf16)
  constexpr int ZD = W / 4 > 0 ? W / 4 : 1;  // dwords of zero points per unit and load
  const uint8_t* zbase = Z + (size_t)col0 * G;
  const uint8_t* sbase = reinterpret_cast<const uint8_t*>(Sc + (size_t)col0 * G);
  uint32_t zoff[UPL], soff[WN];  // byte offsets
#pragma unroll
  for (int t = 0; t < UPL; ++t) zoff[t] = (uint32_t)(((64 * (UPL * wave + t) + lane) >> 3) * G);
#pragma unroll
  for (int j = 0; j < WN; ++j) soff[j] = (uint32_t)(((wn * WN + j) * 32 + lr) * G * 2);
  uint32_t sq[WN][SD], zq[UPL][ZD];
  auto load_s = [&](int g) {  // groups g .. g + W - 1
    const uint8_t* sg = sbase + 2 * g;
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      asm volatile("" : "+v"(soff[j]));
      if constexpr (W == 8) {
        const uint4 v = *reinterpret_cast<const uint4*>(sg + soff[j]);
        sq[j][0] = v.x; sq[j][1] = v.y; sq[j][2] = v.z; sq[j][3] = v.w;
      } else {
        sq[j][0] = *reinterpret_cast<const uint32_t*>(sg + soff[j]);
      }
    }
  };
  auto load_z = [&](int g) {
    const uint8_t* zg = zbase + g;
#pragma unroll
    for (int u = 0; u < UPL; ++u) {
      asm volatile("" : "+v"(zoff[u]));
      if constexpr (W == 8) {
        const uint2 v = *reinterpret_cast<const uint2*>(zg + zoff[u]);
        zq[u][0] = v.x; zq[u][1] = v.y;
      } else {
        zq[u][0] = *reinterpret_cast<const uint16_t*>(zg + zoff[u]);
      }
    }
  };
  // the queue heads, then a shift by one group
  auto pop_s = [&](float (&sv)[WN]) {
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      sv[j] = __uint_as_float(sq[j][0] << 16);
#pragma unroll
      for (int d = 0; d < SD - 1; ++d) sq[j][d] = __builtin_amdgcn_alignbit(sq[j][d + 1], sq[j][d], 16);
      sq[j][SD - 1] >>= 16;
    }
  };
  auto pop_z = [&](uint32_t (&zv)[UPL]) {
#pragma unroll
    for (int u = 0; u < UPL; ++u) {
      zv[u] = zq[u][0] & 0xFFu;
#pragma unroll
      for (int d = 0; d < ZD - 1; ++d) zq[u][d] = __builtin_amdgcn_alignbit(zq[u][d + 1], zq[u][d], 8);
      zq[u][ZD - 1] >>= 8;
    }
  };
  // q - z as bf16 for the 8 nibbles of dword w (value 2i in the low nibble of byte i):
  // the bytes q + 16 - z lie in [1, 31], so one subtraction serves four values with no
  // borrow, and the float of each byte minus 16 is the exact small integer.
  auto raw = [&](int g_slot, int t) {
    const int u = 64 * (UPL * wave + t) + lane;
    return *reinterpret_cast<const uint32_t*>(lds + OFF_Q + g_slot * QB + (u >> 3) * 32 + 4 * (u & 7));
  };
  auto expand = [&](uint32_t w, int buf, int t, uint32_t z) {
    const int u = 64 * (UPL * wave + t) + lane;
    const int c = u >> 3, h = u & 7;
    const uint32_t zb = z * 0x01010101u;
    const uint32_t ev = ((w & 0x0F0F0F0Fu) | 0x10101010u) - zb;
    const uint32_t od = (((w >> 4) & 0x0F0F0F0Fu) | 0x10101010u) - zb;
    uint32_t o[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float fe = (float)((ev >> (8 * b)) & 0xFFu) - 16.0f;
      const float fo = (float)((od >> (8 * b)) & 0xFFu) - 16.0f;
      o[b] = (__float_as_uint(fe) >> 16) | (__float_as_uint(fo) & 0xFFFF0000u);
    }
    *reinterpret_cast<uint4*>(lds + OFF_W + buf * WB + 16 * (c * 8 + (h ^ ((c >> 1) & 7)))) =
        make_uint4(o[0], o[1], o[2], o[3]);
  };

  // Fragment addresses: lane l reads row (or column) 32 blk + l % 32, 16-byte unit
  // (2 c + l / 32) ^ ((l % 32) / 2 % 8) of k-chunk c; the per-lane part is the same for both
  // operands.
  uint32_t foff[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) foff[c] = (uint32_t)(lr * 128 + 16 * ((2 * c + lh) ^ ((lr >> 1) & 7)));
  typedef __attribute__((address_space(3))) const v8bf lds_v8bf;
  auto frag = [&](uint32_t base, int c) { return *(lds_v8bf*)(uintptr_t)(base + foff[c]); };

  v16f acc[2][WN];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  const v16f zero = {};

  // prologue: the first scale and zero-point loads, activations of stage 0, nibbles of
  // stages 0 and 1; then the expansion of stage 0's weights
  load_s(0);
  load_z(0);
  dma_a(0, 0);
  dma_q(0, 0);
  if (G > 1) dma_q(1, 1);
  wait_vm0();
  barrier_lds();
  uint32_t zc[UPL];
  pop_z(zc);  // zero points of group 0; the queue head is now group 1
#pragma unroll
  for (int u = 0; u < UPL; ++u) expand(raw(0, u), 0, u, zc[u]);

  // Stage t: blocks b = 0 .. 2 WN - 1 (column block b / 2, row block b % 2) in turn:
  // block b's four chained MFMAs, then block b - 1's scale FMAs (so they overlap the
  // MFMA latency), and after each column block one unit of stage t + 1's weight
  // expansion, whose nibbles were read at the top of the stage.
  int qs1 = 1;  // raw slot of stage t + 1 (t + 1 mod 3)
  for (int t = 0; t < G; ++t) {
    const int qs2 = qs1 == 2 ? 0 : qs1 + 1;
    wait_vm0();
    barrier_lds();  // stage t's activations and expanded weights are visible to all
    // the stage's first fragments and the expansion's nibbles are read first, so that
    // their latency overlaps the copies issued below
    const uint32_t abase = lds0 + (t & 1) * AB + wm * 64 * 128;
    const uint32_t bbase = lds0 + OFF_W + (t & 1) * WB + wn * WN * 32 * 128;
    v8bf af[2][4], bfc[4], bfn[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) bfc[c] = frag(bbase, c);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) af[i][c] = frag(abase + i * 32 * 128, c);
    uint32_t qraw[UPL];
    if (t + 1 < G) {
#pragma unroll
      for (int u = 0; u < UPL; ++u) qraw[u] = raw(qs1, u);
    }
    float sv[WN];
    pop_s(sv);                                   // scales of group t
    if ((t + 1) % W == 0 && t + 1 < G) load_s(t + 1);
    pop_z(zc);                                   // zero points of group t + 1
    if ((t + 2) % W == 0 && t + 2 < G) load_z(t + 2);
    if (t + 1 < G) dma_a(t + 1, (t + 1) & 1);
    if (t + 2 < G) dma_q(t + 2, qs2);

    v16f d[2];
#pragma unroll
    for (int b = 0; b <= 2 * WN; ++b) {
      const int j = b >> 1, i = b & 1;
      if (b < 2 * WN) {
        if (i == 1 && j + 1 < WN) {
#pragma unroll
          for (int c = 0; c < 4; ++c) bfn[c] = frag(bbase + (j + 1) * 32 * 128, c);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c)
          d[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i][c], bfc[c], c == 0 ? zero : d[i], 0, 0, 0);
      }
      if (b > 0) {
        const int pj = (b - 1) >> 1, pi = (b - 1) & 1;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[pi][pj][e] = __builtin_fmaf(sv[pj], d[pi][e], acc[pi][pj][e]);
        // the rescale stays here (not sunk to the end of the stage, which would keep
        // every block's D alive at once)
        asm volatile("" : "+v"(acc[pi][pj]));
        if (pi == 1 && t + 1 < G) expand(qraw[pj], (t + 1) & 1, pj, zc[pj]);
      }
      if (i == 1 && b < 2 * WN) {
#pragma unroll
        for (int c = 0; c < 4; ++c) bfc[c] = bfn[c];
      }
    }
    qs1 = qs2;
  }
  wait_vm0();
  barrier_lds();  // every wave is done with the tiles: the LDS is free for staging

  // Epilogue: + bias, bf16, through a per-wave staging tile (64 rows x BN/2) so that
  // each row segment is written with 16-byte stores.  Element e of lane l is row
  // 8 (e / 4) + 4 (l / 32) + e % 4 of its block, column l % 32.
  uint16_t* tile = reinterpret_cast<uint16_t*>(lds) + wave * (64 * TS);
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    const int col = (wn * WN + j) * 32 + lr;
    const float bv = bias ? bf16_to_f32(bias[col0 + col]) : 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = 32 * i + 8 * (e >> 2) + 4 * lh + (e & 3);
        tile[r * TS + 32 * j + lr] = (uint16_t)f32_to_bf16_rne(acc[i][j][e] + bv);
      }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  constexpr int UPR = BN / 16;  // 16-byte units per staged row
#pragma unroll
  for (int k = 0; k < UPR; ++k) {
    const int idx = lane + 64 * k;
    const int r = idx / UPR, ch = idx % UPR;
    const uint4 v = *reinterpret_cast<const uint4*>(tile + r * TS + ch * 8);
    const int row = row0 + wm * 64 + r;
    if (row < M) {
      uint16_t* yp = Y + (size_t)row * N + col0 + wn * (BN / 2) + ch * 8;
      if (y_wt) store_wt(yp, v);
      else *reinterpret_cast<uint4*>(yp) = v;
    }
  }
}

hipError_t launch_k4_awq(const uint16_t* X, const uint8_t* Q, const uint16_t* Sc, const uint8_t* Z,
                         const uint16_t* bias, uint16_t* Y, int M, int N, int K, hipStream_t st,
                         hipEvent_t ev0, hipEvent_t ev1) {
  if (M <= 0 || N % 128 != 0 || K % 64 != 0) return hipErrorInvalidValue;
  const int tiles_m = (M + 255) / 256;
  const bool w8 = (K / 64) % 8 == 0;  // scale and zero-point loads of 8 groups
  const dim3 blk(512);
  // Y through the L2 at device scope when the grid is one round (as in the int4 GEMM)
  const int cus = device_cu_count();
  if (N % 192 == 0) {
    const dim3 grid((N / 192) * tiles_m);
    const int wt = grid.x <= (unsigned)cus;
    if (w8) hipExtLaunchKernelGGL(k4_gemm_awq<3, 8>, grid, blk, 0, st, ev0, ev1, 0, X, Q, Sc, Z, bias, Y, M, N, K, wt);
    else hipExtLaunchKernelGGL(k4_gemm_awq<3, 2>, grid, blk, 0, st, ev0, ev1, 0, X, Q, Sc, Z, bias, Y, M, N, K, wt);
  } else {
    const dim3 grid((N / 128) * tiles_m);
    const int wt = grid.x <= (unsigned)cus;
    if (w8) hipExtLaunchKernelGGL(k4_gemm_awq<2, 8>, grid, blk, 0, st, ev0, ev1, 0, X, Q, Sc, Z, bias, Y, M, N, K, wt);
    else hipExtLaunchKernelGGL(k4_gemm_awq<2, 2>, grid, blk, 0, st, ev0, ev1, 0, X, Q, Sc, Z, bias, Y, M, N, K, wt);
  }
  return hipGetLastError();
}

}  // namespace svdq
