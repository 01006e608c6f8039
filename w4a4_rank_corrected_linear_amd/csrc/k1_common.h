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

// QUANT::block(const K1Args&, const float (&xh)[32], int row, int k0, int q) quantizes
// the lane's 32 smoothed values (row, k0 .. k0 + 31) and writes its outputs with
// QUANT::kStores vector memory stores.

}  // namespace svdq
