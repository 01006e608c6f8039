// Per-head Q/K RMSNorm and rotary embedding as a separate pass over a bf16 QKV
// projection output: the unfused form of the QKV epilogue (Diffusers docs "Nunchaku
// Lite", "Fused kernels": the engine fuses these into the QKV projection; the
// infolabhq tutorial's section on structural rewrites shows the Diffusers sequence
// norm_q / norm_k, then apply_rotary_emb, after the projections).
//
//   row m, head h of Q (weights norm_q) or of K (norm_k), channels c = 0..127:
//   n_c = x_c / sqrt(mean_c x_c^2 + eps) * w_c,
//   y_2i = bf16(n_2i cos_i - n_2i+1 sin_i),   y_2i+1 = bf16(n_2i+1 cos_i + n_2i sin_i)
//
// in fp32 on the bf16 input.  Sixteen lanes hold one (row, head) at a time: 8
// channels (16 B) each, the sum of squares is a 16-lane butterfly.  They take up to
// eight heads of one row in turn, so each lane reads the (cos, sin) pairs of its 4
// channel pairs (32 B) once for all of them.  Memory-bound, grid-stride; the V third
// is copied only when the output is a different buffer.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace svdq {

namespace {

constexpr int kHeadsPerGroup = 8;

// Sixteen lanes take a group of up to kHeadsPerGroup heads of one row in turn: lane
// `sub` holds channels 8 sub .. 8 sub + 7 of every head, so its (cos, sin) values and
// both weight vectors are loaded once and serve all of the group's heads.
__global__ void __launch_bounds__(256)
k_qk_norm_rope_bf16(const uint16_t* __restrict__ x, uint16_t* __restrict__ y, int64_t M, int N,
                    const uint16_t* __restrict__ norm_q, const uint16_t* __restrict__ norm_k,
                    float eps, const float* __restrict__ rope) {
  const int heads = 2 * (N / 3) / 128;  // Q heads then K heads of one row
  const int groups = (heads + kHeadsPerGroup - 1) / kHeadsPerGroup;
  const int64_t units = M * groups;
  const int sub = threadIdx.x & 15;
  const int64_t stride = (int64_t)gridDim.x * 16;
  const uint4 wqv = *reinterpret_cast<const uint4*>(norm_q + 8 * sub);
  const uint4 wkv = *reinterpret_cast<const uint4*>(norm_k + 8 * sub);
  for (int64_t u = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4; u < units; u += stride) {
    const int64_t row = u / groups;
    const int h0 = (int)(u % groups) * kHeadsPerGroup, h1 = min(heads, h0 + kHeadsPerGroup);
    const float4 r0 = *reinterpret_cast<const float4*>(rope + row * 128 + 8 * sub);
    const float4 r1 = *reinterpret_cast<const float4*>(rope + row * 128 + 8 * sub + 4);
    const float cs[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll 4
    for (int h = h0; h < h1; ++h) {
      const int64_t off = row * N + (int64_t)h * 128 + 8 * sub;
      const uint4 xv = *reinterpret_cast<const uint4*>(x + off);
      const uint4 wv = h < heads / 2 ? wqv : wkv;
      const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
      const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
      float v[8], w[8];
      float ss = 0.f;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        v[2 * p] = __uint_as_float(xw[p] << 16);
        v[2 * p + 1] = __uint_as_float(xw[p] & 0xFFFF0000u);
        w[2 * p] = __uint_as_float(ww[p] << 16);
        w[2 * p + 1] = __uint_as_float(ww[p] & 0xFFFF0000u);
        ss = fmaf(v[2 * p], v[2 * p], ss);
        ss = fmaf(v[2 * p + 1], v[2 * p + 1], ss);
      }
#pragma unroll
      for (int d = 1; d < 16; d <<= 1) ss += __shfl_xor(ss, d, 16);
      const float inv = 1.0f / sqrtf(ss * (1.0f / 128.0f) + eps);
      uint32_t o[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float n0 = v[2 * p] * inv * w[2 * p], n1 = v[2 * p + 1] * inv * w[2 * p + 1];
        const float c = cs[2 * p], s = cs[2 * p + 1];
        o[p] = f32_to_bf16_rne(n0 * c - n1 * s) | (f32_to_bf16_rne(n1 * c + n0 * s) << 16);
      }
      *reinterpret_cast<uint4*>(y + off) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

// The V third, 16 bytes per thread, when the output is not the input.
__global__ void __launch_bounds__(256)
k_copy_v_bf16(const uint16_t* __restrict__ x, uint16_t* __restrict__ y, int64_t M, int N) {
  const int third8 = (N / 3) / 8;
  const int64_t n = M * third8;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
    const int64_t off = (i / third8) * N + 2 * (N / 3) + 8 * (i % third8);
    *reinterpret_cast<uint4*>(y + off) = *reinterpret_cast<const uint4*>(x + off);
  }
}

}  // namespace

hipError_t launch_qk_norm_rope_bf16(const uint16_t* x, uint16_t* y, int64_t M, int N,
                                    const uint16_t* norm_q, const uint16_t* norm_k, float eps,
                                    const float* rope, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  const int64_t units = M * ((2 * (N / 3) / 128 + kHeadsPerGroup - 1) / kHeadsPerGroup);
  const int64_t blocks = std::min<int64_t>((units * 16 + 255) / 256, 4096);
  hipLaunchKernelGGL(k_qk_norm_rope_bf16, dim3((unsigned)blocks), dim3(256), 0, st, x, y, M, N,
                     norm_q, norm_k, eps, rope);
  if (x != y) {
    const int64_t n = M * ((N / 3) / 8);
    const int64_t b2 = std::min<int64_t>((n + 255) / 256, 2048);
    hipLaunchKernelGGL(k_copy_v_bf16, dim3((unsigned)b2), dim3(256), 0, st, x, y, M, N);
  }
  return hipGetLastError();
}

}  // namespace svdq
