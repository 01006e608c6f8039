// Kernel launchers (host functions defined next to their kernels).  Every launcher
// enqueues on `st` and returns hipGetLastError() of its launches.  Shapes were
// validated by the C ABI before any of these is called.  `ev0` / `ev1` (may be
// null) are HIP events that receive the kernel's start and end timestamps
// (hipExtLaunchKernelGGL), used by the per-kernel timing hook.  `epi` selects the GEMM
// epilogue (Epilogue below).
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

namespace svdq {

// The fused quantizers split K into pieces of at most kK1SplitK values, one
// workgroup column each; each piece writes its own partial U (fragment layout of
// common.h) and the GEMM adds the pieces in order.
constexpr int kK1SplitK = 1536;
inline int k1_splits(int K) { return (K + kK1SplitK - 1) / kK1SplitK; }

hipError_t launch_k1_int4(bool fused, bool gelu_in, const uint16_t* x, int M, int K, const uint16_t* smooth,
                          const uint16_t* ldown, int rank, uint8_t* codes, void* scales,
                          float* uact, int M_pad, hipStream_t st, hipEvent_t ev0 = nullptr,
                          hipEvent_t ev1 = nullptr);

// Epilogue of the GEMMs: plain (+ bias, bf16), exact GELU before the rounding, or the
// fused QKV epilogue (per-head RMSNorm and rotary embedding on the Q and K thirds of
// the columns, heads of 128; V plain).
enum Epilogue { kEpiPlain = 0, kEpiGelu = 1, kEpiQkNormRope = 2 };

struct QkEpi {
  const uint16_t* norm_q;  // bf16 [128]
  const uint16_t* norm_k;  // bf16 [128]
  const float* rope;       // fp32 [M][64][2]: (cos, sin) per token and pair
  float eps;
};

// Compute units of the current device (cached per device; 256 if the query fails).
int device_cu_count();

// Dense MFMA rate probe (a measurement aid): instruction types, the operations one
// instruction performs, and the launch (one 512-thread workgroup per CU, `iters`
// rounds of four instructions per wave, one float per thread into sink).
enum MfmaOp { kMfmaFp6 = 0, kMfmaFp4 = 1, kMfmaFp8 = 2, kMfmaI8 = 3, kMfmaF16 = 4, kMfmaBf16 = 5,
              kMfmaBf16K8 = 6 };
double mfma_probe_flops_per_instr(int op);
hipError_t launch_mfma_probe(int op, int iters, float* sink, hipStream_t st);

// Launch plan of the int4 GEMM: tile width, tile count, and the K-split of the tiles
// of a last, partial round on the CUs (tiles [full, tiles) split into ks pieces each,
// whose fp32 partial tiles a second, small kernel adds up and finishes).  max_pieces
// is the number of 256 x 192 fp32 partial tiles the caller has room for (0: no split).
struct K2Plan {
  int bm = 256, bn = 192;  // tile
  int tiles = 0, full = 0, ks = 1;
  int kernels() const { return ks > 1 ? 2 : 1; }
};
K2Plan plan_k2_int4(int M_pad, int N, int K, int epi, int max_pieces);
constexpr int kSplitMaxPieces = 256;
constexpr size_t kSplitTileBytes = (size_t)256 * 192 * 4;

// ev0/ev1 time the GEMM, ev2/ev3 the tail kernel (when the plan splits).
hipError_t launch_k2_int4(const K2Plan& plan, const uint8_t* A, const uint2* sA, const float* U,
                          int nsplit, const uint8_t* B, const uint2* sB, const uint16_t* L2t,
                          const uint16_t* bias, uint16_t* Y, int M, int N, int K, int M_pad,
                          int rank, int epi, const QkEpi& qk, float* part, hipStream_t st,
                          hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr,
                          hipEvent_t ev2 = nullptr, hipEvent_t ev3 = nullptr);

hipError_t launch_k1_nvfp4(bool fused, bool gelu_in, const uint16_t* x, int M, int K, const uint16_t* smooth,
                           const uint16_t* ldown, int rank, float g, uint8_t* out, uint8_t* scales,
                           float* uact, int M_pad, hipStream_t st, hipEvent_t ev0 = nullptr,
                           hipEvent_t ev1 = nullptr);

// NVFP4 GEMM on 4-bit operands (FP4 lane slots and fp16 block scales, common.h).
hipError_t launch_k2_fp4(const uint8_t* A, const uint16_t* sA, const float* U, int nsplit,
                         const uint8_t* B, const uint16_t* sB, const uint16_t* L2t,
                         const uint16_t* bias, float g, uint16_t* Y, int M, int N, int K,
                         int M_pad, int rank, int epi, const QkEpi& qk, hipStream_t st,
                         hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);

hipError_t launch_k4_awq(const uint16_t* X, const uint8_t* Q, const uint16_t* Sc, const uint8_t* Z,
                         const uint16_t* bias, uint16_t* Y, int M, int N, int K, hipStream_t st,
                         hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);

hipError_t launch_pack_lora_down(const uint16_t* in, uint16_t* out, int rank, int K, hipStream_t st);

// NVFP4 weights: interchange codes [N][K/2] and E4M3 scales [N][K/16] -> FP4 lane-slot
// chunks and fp16 scales [K/64][N][4] (common.h); an E4M3 NaN scale raises *flag.
hipError_t launch_pack_nvfp4(const uint8_t* codes, const uint8_t* scales, uint8_t* out_codes,
                             uint16_t* out_scales, int* flag, int N, int K, hipStream_t st);

hipError_t launch_pack_int4(const uint8_t* codes, const uint16_t* scales, uint8_t* out_codes,
                            void* out_scales, int* flag, int N, int K, hipStream_t st);

hipError_t launch_gelu_bf16(const uint16_t* x, uint16_t* y, int64_t n, hipStream_t st);

// Offline weight preparation on the GPU (k_prep.hip): smoothing factors, the
// randomized top-rank factorization of the smoothed weight (l = rank + oversampling
// columns, iters power iterations), the bf16 factors and the int4 or NVFP4 residual
// (NVFP4: globals_host[0..1] = g_w, g_x).  Runs on `st` and synchronizes it;
// *fail_host gets 0, or a nonzero code when the orthonormalization or the small
// eigenproblem broke down.  launch_prep_awq: the AWQ W4A16 weights (asynchronous).
size_t prep_workspace_bytes(int64_t K, int64_t N, int rank, int l);
hipError_t launch_prep(bool nvfp4, int K, int N, int rank, int l, int iters, const float* w,
                       const uint16_t* xc, int64_t Mc, const double* omega, uint8_t* qweight,
                       void* wscales, uint16_t* smooth, uint16_t* ldown, uint16_t* lup,
                       float* residual, void* ws, int* fail_host, float* globals_host,
                       hipStream_t st);
hipError_t launch_prep_awq(int K, int N, const float* w, uint8_t* qweight, uint16_t* scales,
                           uint8_t* zeros, hipStream_t st);

// Per-head Q/K RMSNorm + rotary embedding on a bf16 [M][N] QKV output (N = 3 H 128);
// the V third is copied when y != x.
hipError_t launch_qk_norm_rope_bf16(const uint16_t* x, uint16_t* y, int64_t M, int N,
                                    const uint16_t* norm_q, const uint16_t* norm_k, float eps,
                                    const float* rope, hipStream_t st);

}  // namespace svdq
