// K4: the AWQ W4A16 comparison layer.
//
//   Y[m,n] = bf16( sum_g s[n,g] D_g[m,n] + b[n] ),  D_g = sum_{k in g} x[m,k] (q[n,k] - z[n,g])
//
// (Diffusers docs "Nunchaku Lite", "Supported quantization types": awq_w4a16, INT4
// weight-only, group 64.)  The weights stay 4-bit in HBM and in LDS; per stage (one
// 64-group) the workgroup expands its 128 x 64 weight slice into the exact bf16
// values q - z (integers in [-15, 15]), the bf16 MFMA forms D_g in fp32, and one fp32
// FMA per output element applies the group scale: acc = fma(s, D_g, acc).
//
// Tiling: 256 threads (2 x 2 waves), tile 128 x 128, wave tile 64 x 64 (2 x 2 blocks
// of v_mfma_f32_32x32x16_bf16), two workgroups per CU.  X tiles (bf16) and the raw
// weight nibbles are copied into LDS by global_load_lds, double-buffered; rows of X
// past M read row M - 1 (their outputs are not stored).  The bf16 tiles use the
// 16-byte unit swizzle u = row * 8 + (c ^ (row & 7)) (c = k / 8 within the group).
#include "common.h"
#include "kernels.h"

namespace svdq {

__global__ void __launch_bounds__(256, 2)
k4_gemm_awq(const uint16_t* __restrict__ X, const uint8_t* __restrict__ Q,
            const uint16_t* __restrict__ Sc, const uint8_t* __restrict__ Z,
            const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y, int M, int N, int K) {
  constexpr int BM = 128, BN = 128;
  constexpr int TILE = 128 * 64;  // bf16 elements of a 128 x 64 tile
  __shared__ __attribute__((aligned(16))) uint16_t A0[TILE], A1[TILE], Bt[TILE];
  __shared__ __attribute__((aligned(16))) uint8_t Q0[128 * 32], Q1[128 * 32];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_n = N / BN;
  const int tn = blockIdx.x % tiles_n, tm = blockIdx.x / tiles_n;
  const int row0 = tm * BM, col0 = tn * BN;
  const int G = K >> 6;

  // Per stage each wave copies 4 KiB of the X tile (4 instructions) and 1 KiB of the
  // weight nibbles (column c's 32 bytes of group g are 16-byte units 2c and 2c + 1).
  auto dma = [&](int g, uint16_t* Ab, uint8_t* Qb) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int u = 64 * (4 * wave + t) + lane;
      const int r = u >> 3, c = (u & 7) ^ (r & 7);
      const int gr = min(row0 + r, M - 1);
      __builtin_amdgcn_global_load_lds(X + (size_t)gr * K + 64 * g + 8 * c,
                                       Ab + 8 * 64 * (4 * wave + t), 16, 0, 0);
    }
    {
      const int u = 64 * wave + lane;
      const int c = u >> 1, h = u & 1;
      __builtin_amdgcn_global_load_lds(Q + (size_t)(col0 + c) * (K / 2) + 32 * g + 16 * h,
                                       Qb + 1024 * wave, 16, 0, 0);
    }
  };

  // Expansion: thread t takes column t / 2 and 32 values of k (half t % 2 of the group).
  const int ec = tid >> 1, eh = tid & 1;
  auto expand = [&](const uint8_t* Qb, int z) {
    const uint4 v = *reinterpret_cast<const uint4*>(Qb + 16 * tid);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    const uint32_t zb = (uint32_t)z * 0x01010101u;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      // bytes of (q + 16 - z) for the even and the odd elements: no borrows, as
      // q + 16 - z lies in [1, 31]
      const uint32_t ev = ((w[d] & 0x0F0F0F0Fu) | 0x10101010u) - zb;
      const uint32_t od = (((w[d] >> 4) & 0x0F0F0F0Fu) | 0x10101010u) - zb;
      uint32_t o[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float fe = (float)((ev >> (8 * b)) & 0xFFu) - 16.0f;
        const float fo = (float)((od >> (8 * b)) & 0xFFu) - 16.0f;
        o[b] = (__float_as_uint(fe) >> 16) | (__float_as_uint(fo) & 0xFFFF0000u);
      }
      const int c = 4 * eh + d;  // 8-value chunk within the group
      *reinterpret_cast<uint4*>(Bt + 8 * (ec * 8 + (c ^ (ec & 7)))) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  };

  auto frag = [&](const uint16_t* T, int row, int kk) {
    const int c = 2 * kk + (lane >> 5);
    return *reinterpret_cast<const v8bf*>(T + 8 * (row * 8 + (c ^ (row & 7))));
  };

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  const v16f zero = {};

  // this lane's output columns (one per 32-column block j) and this thread's
  // expansion column: scales and zero points of the next group are prefetched
  const int ocol[2] = {col0 + wn * 64 + (lane & 31), col0 + wn * 64 + 32 + (lane & 31)};
  uint16_t s_nxt[2] = {Sc[(size_t)ocol[0] * G], Sc[(size_t)ocol[1] * G]};
  int z_nxt = Z[(size_t)(col0 + ec) * G];

  auto compute = [&](const uint16_t* Ab, float s0, float s1) {
    v16f d[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) d[i][j] = zero;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      v8bf a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = frag(Ab, wm * 64 + 32 * i + (lane & 31), kk);
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = frag(Bt, wn * 64 + 32 * j + (lane & 31), kk);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          d[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], d[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        acc[i][0][e] = __builtin_fmaf(s0, d[i][0][e], acc[i][0][e]);
        acc[i][1][e] = __builtin_fmaf(s1, d[i][1][e], acc[i][1][e]);
      }
  };

  auto sync_all = [&]() {
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
  };

  // Stage g: wait for its copies, expand the weights, synchronize, start the next
  // stage's copies (the compiler completes outstanding memory operations before a
  // barrier, so they are issued after the stage's last one), then the MFMAs and the
  // scale FMAs.
  auto stage = [&](int g, uint16_t* Ab, uint8_t* Qb, uint16_t* An, uint8_t* Qn) {
    const float s0 = bf16_to_f32(s_nxt[0]), s1 = bf16_to_f32(s_nxt[1]);
    const int z = z_nxt;
    sync_all();
    expand(Qb, z);
    sync_all();
    if (g + 1 < G) {
      dma(g + 1, An, Qn);
      s_nxt[0] = Sc[(size_t)ocol[0] * G + g + 1];
      s_nxt[1] = Sc[(size_t)ocol[1] * G + g + 1];
      z_nxt = Z[(size_t)(col0 + ec) * G + g + 1];
    }
    compute(Ab, s0, s1);
  };

  dma(0, A0, Q0);
  for (int g = 0; g < G; g += 2) {
    stage(g, A0, Q0, A1, Q1);
    if (g + 1 < G) stage(g + 1, A1, Q1, A0, Q0);
  }
  sync_all();

  // Epilogue: + bias, bf16 stores through a per-wave LDS tile (rows of 80 B).
  const int lr = lane & 31, lh = lane >> 5;
  uint16_t* tile = A0 + wave * (32 * 40);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rowb = row0 + wm * 64 + 32 * i;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int colb = col0 + wn * 64 + 32 * j;
      const float bv = bias ? bf16_to_f32(bias[colb + lr]) : 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int rin = 8 * (e >> 2) + 4 * lh + (e & 3);
        tile[rin * 40 + lr] = (uint16_t)f32_to_bf16_rne(acc[i][j][e] + bv);
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

hipError_t launch_k4_awq(const uint16_t* X, const uint8_t* Q, const uint16_t* Sc, const uint8_t* Z,
                         const uint16_t* bias, uint16_t* Y, int M, int N, int K, hipStream_t st,
                         hipEvent_t ev0, hipEvent_t ev1) {
  const int tiles_m = (M + 127) / 128;
  dim3 grid((N / 128) * tiles_m);
  hipExtLaunchKernelGGL(k4_gemm_awq, grid, dim3(256), 0, st, ev0, ev1, 0, X, Q, Sc, Z, bias, Y, M,
                        N, K);
  return hipGetLastError();
}

}  // namespace svdq
