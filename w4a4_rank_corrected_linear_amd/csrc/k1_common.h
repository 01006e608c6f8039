// Arguments of the fused activation-side kernels (K1 feeding the GEMM), shared by the
// two skeletons (k1_rows32.h: 32 rows per workgroup, one round; k1_stream.h: resident
// workgroups streaming 16-row units) and the per-precision quantizer blocks.
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

// The layer's input value x of one bf16 activation, given as fp32 bits with the bf16 in
// the high half.  GELU_IN: the input is the MLP's hidden activation bf16(gelu(x)) of
// the bf16 x the up projection stored, formed with the same gelu_f32 and rounding as
// the separate GELU pass (k_gelu.hip), so the quantizer sees exactly the values that
// pass would have written (gelu(0) = 0 keeps zeroed padding rows zero).
template <bool GELU_IN>
__device__ __forceinline__ float k1_input(uint32_t hi) {
  if constexpr (GELU_IN) return __uint_as_float(f32_to_bf16_rne(gelu_f32(__uint_as_float(hi))) << 16);
  else return __uint_as_float(hi);
}

// QUANT::block(const K1Args&, const float (&xh)[32], int row, int k0, int q) quantizes
// the lane's 32 smoothed values (row, k0 .. k0 + 31) and writes its outputs with
// QUANT::kStores vector memory stores.

}  // namespace svdq
