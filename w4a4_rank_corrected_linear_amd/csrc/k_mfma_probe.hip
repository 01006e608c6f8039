// Measurement aid, not part of the layer: the dense MFMA rate this chip sustains for
// each matrix instruction the kernels issue (FP6 and the 32x32x8 bf16 outer product of
// the int4 GEMM, fp16 of the NVFP4 GEMM, bf16 of the low-rank terms and the AWQ GEMM)
// and for the FP4, FP8 and int8 forms the published peaks are quoted for.  It is the
// "achievable peak" beside the published one against which a kernel's roofline
// fraction is read.
//
// One 512-thread workgroup (8 waves, two per SIMD, as in the GEMMs) per CU; every wave
// runs `iters` rounds of four MFMAs on four independent accumulators (the next use of
// an accumulator is four issues later, past the instruction's dependency latency), on
// register operands that never change.  Each lane's accumulator sum goes to the sink
// so that nothing is optimised away.
#include "common.h"
#include "k2_common.h"
#include "kernels.h"

namespace svdq {

typedef _Float16 v8h_p __attribute__((ext_vector_type(8)));
typedef int v16i_p __attribute__((ext_vector_type(16)));

template <int OP>
__global__ void __launch_bounds__(512, 1) k_mfma_probe(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  // operand bits that are finite, small numbers in every format: FP6 E2M3 and FP4
  // E2M1 fields of 1.0 (001000, 0010), FP8 E4M3 bytes of 1.0 (0x38), int8 ones, and
  // fp16 / bf16 values 2^-6 (with a lane-dependent low bit)
  const uint32_t f6w[3] = {0x08208208u, 0x82082082u, 0x20820820u};  // 001000 repeated
  v8i a8, b8;
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    uint32_t w;
    if (OP == kMfmaFp6) w = d < 6 ? f6w[d % 3] : 0u;
    else if (OP == kMfmaFp4) w = d < 4 ? 0x22222222u : 0u;
    else if (OP == kMfmaFp8) w = 0x38383838u;
    else w = 0x01010101u;
    a8[d] = (int)(w ^ (uint32_t)(lane & 1));
    b8[d] = (int)w;
  }
  v16f acc[4];
  v16i_p iacc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      acc[c][e] = 0.f;
      iacc[c][e] = 0;
    }
  v8h_p h8;
  v8bf b8f;
  v4bf b4f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h8[e] = (_Float16)(0.015625f + (float)(lane & 1) * 0x1p-16f);
    b8f[e] = (__bf16)(0.015625f + (float)(lane & 1) * 0x1p-13f);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) b4f[e] = b8f[e];
  const v4i a4 = {a8[0], a8[1], a8[2], a8[3]}, bi4 = {b8[0], b8[1], b8[2], b8[3]};

  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if constexpr (OP == kMfmaFp6)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[c], 2, 2, 0, 127, 0, 127);
      else if constexpr (OP == kMfmaFp4)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[c], 4, 4, 0, 127, 0, 127);
      else if constexpr (OP == kMfmaFp8)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[c], 0, 0, 0, 127, 0, 127);
      else if constexpr (OP == kMfmaI8)
        iacc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a4, bi4, iacc[c], 0, 0, 0);
      else if constexpr (OP == kMfmaF16)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(h8, h8, acc[c], 0, 0, 0);
      else if constexpr (OP == kMfmaBf16)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b8f, b8f, acc[c], 0, 0, 0);
      else
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(b4f, b4f, acc[c], 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += OP == kMfmaI8 ? (float)iacc[c][e] : acc[c][e];
  sink[(size_t)blockIdx.x * 512 + threadIdx.x] = s;
}

double mfma_probe_flops_per_instr(int op) {
  switch (op) {
    case kMfmaFp6:
    case kMfmaFp4:
    case kMfmaFp8: return 2.0 * 32 * 32 * 64;
    case kMfmaI8: return 2.0 * 32 * 32 * 32;
    case kMfmaF16:
    case kMfmaBf16: return 2.0 * 32 * 32 * 16;
    default: return 2.0 * 32 * 32 * 8;
  }
}

hipError_t launch_mfma_probe(int op, int iters, float* sink, hipStream_t st) {
  const dim3 grid((unsigned)device_cu_count()), block(512);
  switch (op) {
    case kMfmaFp6: hipLaunchKernelGGL(k_mfma_probe<kMfmaFp6>, grid, block, 0, st, iters, sink); break;
    case kMfmaFp4: hipLaunchKernelGGL(k_mfma_probe<kMfmaFp4>, grid, block, 0, st, iters, sink); break;
    case kMfmaFp8: hipLaunchKernelGGL(k_mfma_probe<kMfmaFp8>, grid, block, 0, st, iters, sink); break;
    case kMfmaI8: hipLaunchKernelGGL(k_mfma_probe<kMfmaI8>, grid, block, 0, st, iters, sink); break;
    case kMfmaF16: hipLaunchKernelGGL(k_mfma_probe<kMfmaF16>, grid, block, 0, st, iters, sink); break;
    case kMfmaBf16: hipLaunchKernelGGL(k_mfma_probe<kMfmaBf16>, grid, block, 0, st, iters, sink); break;
    case kMfmaBf16K8: hipLaunchKernelGGL(k_mfma_probe<kMfmaBf16K8>, grid, block, 0, st, iters, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace svdq
