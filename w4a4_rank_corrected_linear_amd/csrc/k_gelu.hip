// Elementwise exact (erf) GELU on bf16, the activation between the MLP-up and
// MLP-down linears of a DiT block (Diffusers docs "Nunchaku Lite", "Fused kernels":
// the MLP's GELU).
//
//   y = bf16( x/2 * erfc(-x / sqrt 2) )        (= x Phi(x), one rounding)
//
// with erfc from gelu_f32 (common.h): a Chebyshev-fitted form accurate to ~1e-7
// relative on both sides, down to bf16's subnormal range.
// Memory-bound: one 16-byte load and store per 8 values, grid-stride.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace svdq {

namespace {

__device__ __forceinline__ uint32_t gelu_bits(uint32_t b16) {
  return f32_to_bf16_rne(gelu_f32(bf16_to_f32(b16)));
}

__global__ void __launch_bounds__(256)
k_gelu_bf16(const uint4* __restrict__ x, uint4* __restrict__ y, int64_t n8) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += stride) {
    const uint4 v = x[i];
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int p = 0; p < 4; ++p) w[p] = gelu_bits(w[p] & 0xFFFFu) | (gelu_bits(w[p] >> 16) << 16);
    y[i] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

__global__ void k_gelu_bf16_tail(const uint16_t* __restrict__ x, uint16_t* __restrict__ y, int n) {
  if ((int)threadIdx.x < n) y[threadIdx.x] = (uint16_t)gelu_bits(x[threadIdx.x]);
}

}  // namespace

hipError_t launch_gelu_bf16(const uint16_t* x, uint16_t* y, int64_t n, hipStream_t st) {
  const int64_t n8 = n / 8;
  if (n8 > 0) {
    const int64_t blocks = std::min<int64_t>((n8 + 255) / 256, 2048);
    hipLaunchKernelGGL(k_gelu_bf16, dim3((unsigned)blocks), dim3(256), 0, st,
                       reinterpret_cast<const uint4*>(x), reinterpret_cast<uint4*>(y), n8);
  }
  if (n % 8)
    hipLaunchKernelGGL(k_gelu_bf16_tail, dim3(1), dim3(64), 0, st, x + 8 * n8, y + 8 * n8,
                       (int)(n % 8));
  return hipGetLastError();
}

}  // namespace svdq
