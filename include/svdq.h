/*
 * svdq.h -- C ABI of the MI355X (gfx950) SVDQuant W4A4 linear layer.
 *
 * What the layer computes (Diffusers docs "Nunchaku Lite", "Supported quantization
 * types" table and "NunchakuLiteQuantizationConfig" section; the infolabhq
 * tutorial's section on why 4-bit inference matters):
 *
 *   svdq_w4a4 linear, precision int4 (group 64) or nvfp4 (group 16), with the SVDQ
 *   low-rank correction of rank r (32 in the config example), compute_dtype bf16:
 *
 *     xhat = bf16(x * smooth)                      per-input-channel smoothing
 *     U    = xhat @ lora_down^T (fp32 accumulation) rank-r down projection
 *     codes, scales = quantize(xhat)               4-bit, one scale per group
 *     Y    = bf16( sum_g s_x s_w (codes_x . codes_w)_g  [ * g_x g_w for nvfp4 ]
 *                  + U @ lora_up^T + bias )
 *
 *   awq_w4a16 linear (INT4 weight-only, group 64), the comparison path:
 *     Y = bf16( sum_g s[n,g] sum_{k in g} x[m,k] (q[n,k] - z[n,g]) + bias[n] )
 *
 * Conventions for every entry point
 *   - bf16 values are passed as uint16_t bit patterns.
 *   - Every pointer argument is a DEVICE pointer (hipMalloc / torch CUDA tensors)
 *     unless stated otherwise.  All arrays are dense, row-major, 16-byte aligned.
 *   - The caller owns every buffer.  The library allocates no device memory; it
 *     keeps only a per-device architecture cache.
 *   - Work is enqueued on `stream` and is asynchronous: outputs are valid once the
 *     stream has been synchronized.  Nothing is launched when a call returns an
 *     error.  Errors are detected on the host, before any device access, in the
 *     order NULL -> config -> shape -> alignment -> workspace -> device; launch
 *     failures return SVDQ_ERR_HIP.  svdq_last_error() describes the last failure
 *     of the calling thread.
 *   - Weights are logically W[K, N] (Y = X W) and are stored per output column
 *     (N rows of length K), like nn.Linear.
 */
#ifndef SVDQ_H
#define SVDQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SVDQ_OK = 0,
  SVDQ_ERR_NULL = 1,      /* a required pointer is NULL                              */
  SVDQ_ERR_CONFIG = 2,    /* (method, precision, group_size, rank, dtype) unsupported */
  SVDQ_ERR_SHAPE = 3,     /* sizes violate the layer's shape rules                    */
  SVDQ_ERR_ALIGN = 4,     /* a pointer is not 16-byte aligned                         */
  SVDQ_ERR_WORKSPACE = 5, /* workspace smaller than svdq_workspace_bytes()           */
  SVDQ_ERR_DEVICE = 6,    /* no device, or the current device is not gfx950          */
  SVDQ_ERR_HIP = 7,       /* a HIP runtime call or kernel launch failed               */
  SVDQ_ERR_RANGE = 8      /* an input value is outside the supported range            */
} svdq_status;

typedef enum { SVDQ_INT4 = 0, SVDQ_NVFP4 = 1 } svdq_precision;
typedef enum { SVDQ_BF16 = 0 } svdq_dtype;

/* Mirrors the svdq_w4a4 / awq_w4a16 entries of NunchakuLiteQuantizationConfig.
 * Supported: svdq_w4a4 {int4, 64} and {nvfp4, 16} with rank 0..32 in steps of 16
 * (0, 16 or 32); awq_w4a16 {int4, 64} with rank 0.  compute_dtype: bf16 only. */
typedef struct {
  int32_t precision;     /* svdq_precision */
  int32_t group_size;    /* 64 (int4) or 16 (nvfp4) */
  int32_t rank;          /* low-rank correction rank r */
  int32_t compute_dtype; /* svdq_dtype */
} svdq_config;

/* A prepared svdq_w4a4 layer in the kernel layout (see svdq_pack_weight). */
typedef struct {
  int64_t K, N;
  const uint8_t* qweight;    /* packed codes, svdq_packed_weight_bytes() codes part      */
  const void* wscales;       /* packed scales, svdq_packed_weight_bytes() scales part    */
  float w_global;            /* NVFP4 per-tensor weight scale g_w; ignored for int4      */
  const uint16_t* smooth;    /* [K] bf16 smoothing multiplier m                          */
  const uint16_t* lora_down; /* L1^T in the packed order of svdq_pack_lora_down (r*K bf16;
                                NULL iff r == 0)                                          */
  const uint16_t* lora_up;   /* [N][r] bf16, L2^T (NULL iff r == 0)                      */
  const uint16_t* bias;      /* [N] bf16 or NULL                                         */
} svdq_w4a4_weight;

/* An awq_w4a16 layer in the interchange layout. */
typedef struct {
  int64_t K, N;
  const uint8_t* qweight;   /* [N][K/2] unsigned nibbles 0..15, element 2j in bits 3:0 */
  const uint16_t* scales;   /* [N][K/64] bf16                                          */
  const uint8_t* zeros;     /* [N][K/64] zero points 0..15                             */
  const uint16_t* bias;     /* [N] bf16 or NULL                                        */
} awq_w4a16_weight;

/* Returns SVDQ_OK if `hip_device` exists and is a gfx950 (MI355X-class) GPU, else
 * SVDQ_ERR_DEVICE with the reason in svdq_last_error().  This is the load-time
 * capability check with a clear error (infolabhq tutorial, hardware caveats
 * section: unsupported GPUs are rejected at load). */
svdq_status svdq_check_device(int hip_device);

/* Bytes of the packed weight buffers for a K x N svdq_w4a4 layer (0 on bad
 * config or shape).  *codes_bytes and *scales_bytes receive the two parts:
 *   int4:  codes N*K*3/4 (E2M3 lane slots, 6 bits per weight: the layout the GEMM's
 *          FP6 MFMA reads, chunks of 1536 bytes per 32 output columns and 64-group),
 *          scales round_up(K/128 * N * 8, 256) + 256 ([K/128][N] 8-byte records
 *          {scale of group 2p, scale of group 2p+1, 0, 0} in bf16: the rescale MFMA's
 *          operand as stored, one record per pair of groups; a 256-byte trailer the
 *          pack clears)
 *   nvfp4: codes N*K/2 (E2M1 codes in the GEMM's FP4 lane slots: chunks of 1024 bytes
 *          per 32 output columns and 64-group, dword j of lane slot l at byte
 *          256 j + 4 l, 4 bits per weight), scales
 *          round_up(N*K/8, 256) + 256 (each E4M3 block scale as its exact fp16 value,
 *          [K/64][N][4]; range flag) -- 4.5 bits per weight in all */
size_t svdq_packed_weight_bytes(const svdq_config* cfg, int64_t K, int64_t N,
                                size_t* codes_bytes, size_t* scales_bytes);

/* Converts interchange-layout weight codes and scales into the kernel layout.
 *   codes        [N][K/2]  int4: two's complement nibbles, element 2j in bits 3:0;
 *                          nvfp4: E2M1 nibbles, same order
 *   scales       [N][K/G]  int4: bf16; nvfp4: E4M3 bytes
 *   packed_codes, packed_scales: buffers of svdq_packed_weight_bytes()
 * int4 codes may take every value of the 4-bit two's complement range [-8, 7]
 * (each is an exact E2M3 operand value q/8 of the GEMM).  An nvfp4 scale byte that is
 * an E4M3 NaN (0x7F or 0xFF) makes the call return SVDQ_ERR_RANGE.  This
 * is an offline step: it synchronizes `stream` before returning. */
svdq_status svdq_pack_weight(const svdq_config* cfg, int64_t K, int64_t N,
                             const uint8_t* codes, const void* scales,
                             uint8_t* packed_codes, void* packed_scales, hipStream_t stream);

/* Reorders lora_down [r][K] bf16 (L1^T, interchange layout) into the order the layer's
 * quantizer reads it: for each 128-wide k-block, 16-rank slice and 8-value chunk c of
 * a 32-value lane slot, 64 entries of 16 bytes (entry 16 q + i holds ranks 16 sl + i,
 * k = 128 kb + 32 q + 8 c .. + 8), each group 1 KiB contiguous.  `packed` has r*K bf16
 * (same size); rank 16 or 32, K a multiple of 128.  The result is what
 * svdq_w4a4_weight.lora_down points to.  Offline step; enqueued on `stream`. */
svdq_status svdq_pack_lora_down(const svdq_config* cfg, int64_t K, const uint16_t* lora_down,
                                uint16_t* packed, hipStream_t stream);

/* Workspace bytes svdq_w4a4_linear needs for M tokens of K inputs.  For int4 this
 * includes 48 MiB for the GEMM's K-split of a last, partial round of tiles: when the
 * tile count leaves the CUs' last round part empty, those tiles are split along K,
 * their fp32 partial tiles stored here and added up (in a fixed order) by a second,
 * small kernel.  A workspace that stops short of that area (at least the size without
 * it) is accepted; the GEMM then splits only as far as the room it is given allows (no
 * split without room).  svdq_workspace_bytes_n sizes the area for one layer. */
size_t svdq_workspace_bytes(const svdq_config* cfg, int64_t M, int64_t K);

/* Workspace bytes for M tokens of a layer with K inputs and N outputs: the same areas
 * as svdq_workspace_bytes, with the int4 K-split area sized for the split the GEMM
 * takes at this (M, N, K) on the current device (the larger of the plain and the fused
 * QKV plans; none when neither splits), instead of the 48 MiB maximum.  A call given a
 * workspace of this size runs the same kernels as with the full one.  Host-only query
 * (it reads the current device's CU count, 256 when no device is visible); 0 for an
 * invalid config or shape. */
size_t svdq_workspace_bytes_n(const svdq_config* cfg, int64_t M, int64_t K, int64_t N);

/* Activation side of the layer (smoothing, low-rank down projection, quantization)
 * in the interchange layout.  Defined by the Diffusers docs "Nunchaku Lite",
 * "Supported quantization types" table (svdq_w4a4: activations quantized to int4 in
 * groups of 64 or to nvfp4 in blocks of 16, with the SVDQ low-rank branch) and the
 * infolabhq tutorial's section on why 4-bit inference matters (activations, not only
 * weights, are 4-bit); the smoothing and the unrounded U are readings of those pages.
 *   x          [M][K] bf16 activations
 *   smooth     [K] bf16 multiplier m;  lora_down [r][K] bf16 (NULL iff r == 0)
 *   act_global NVFP4 static activation scale g_x (ignored for int4)
 *   codes      [M][K/2] out: int4 two's complement / E2M1 nibbles, 2j in bits 3:0
 *   scales     [M][K/G] out: bf16 (int4) or E4M3 bytes (nvfp4)
 *   lora_act   [M][r] out: U = xhat @ lora_down^T, fp32 (NULL iff r == 0); U is
 *              accumulated in fp32 and kept unrounded for the up projection
 * int4: s = bf16(amax/7) per 64-group, q = round-half-even(xhat/s) clamped to the
 * int4 range [-8, 7] (only a subnormal bf16 s lets a quotient leave [-7.5, 7.5]).
 * nvfp4: s = E4M3(amax / (6 g_x)) per 16-block, code = E2M1(xhat / (s g_x)). */
svdq_status svdq_quantize_act(const svdq_config* cfg, const uint16_t* x, int64_t M, int64_t K,
                              const uint16_t* smooth, const uint16_t* lora_down, float act_global,
                              uint8_t* codes, void* scales, float* lora_act, hipStream_t stream);

/* The whole layer: Y[M][N] (bf16) = svdq_w4a4(X[M][K]), the formula at the top of this
 * file, as the Diffusers docs "Nunchaku Lite", "Supported quantization types" table
 * defines svdq_w4a4 (4-bit weights and activations, int4 g64 or nvfp4 g16, plus the
 * SVDQ low-rank correction; rank 32 in the "NunchakuLiteQuantizationConfig" example).
 * w: the packed layer (svdq_pack_weight, svdq_pack_lora_down); x [M][K] bf16; y
 * [M][N] bf16 out; act_global: g_x for nvfp4, ignored for int4.  `workspace` holds
 * the quantized activations between the two kernels (svdq_workspace_bytes); the
 * caller owns it and its contents on return are unspecified.  M >= 0 (M = 0 launches
 * nothing); K a multiple of 128, N of 128.  Errors as in the conventions above. */
svdq_status svdq_w4a4_linear(const svdq_config* cfg, const svdq_w4a4_weight* w,
                             const uint16_t* x, int64_t M, float act_global, uint16_t* y,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The same call with the exact GELU applied to each fp32 result before the single bf16
 * rounding (Diffusers docs "Nunchaku Lite", "Fused kernels": the DiT MLP's GELU fused
 * into its first projection):
 *   Y = bf16( gelu(r) ),  gelu(v) = v/2 * erfc(-v/sqrt(2)) in fp32 (erfc to ~1e-7),
 * with r the svdq_w4a4_linear result before rounding.  Arguments, layouts, ownership
 * and errors as for svdq_w4a4_linear. */
svdq_status svdq_w4a4_linear_gelu(const svdq_config* cfg, const svdq_w4a4_weight* w,
                                  const uint16_t* x, int64_t M, float act_global, uint16_t* y,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The same layer taking the GELU of its input: the second linear of the DiT MLP, whose
 * input is the GELU of the first linear's bf16 output (Diffusers docs "Nunchaku Lite",
 * "Fused kernels": the MLP's GELU fused with its projections).  The quantizer applies
 *   h = bf16_rne( gelu(x) )   (gelu as in svdq_gelu_bf16, bit for bit)
 * to each bf16 input value as it loads it and runs the layer on h, so
 *   Y = svdq_w4a4_linear(h)  exactly (codes, scales, low-rank sums and Y identical to
 * svdq_gelu_bf16 followed by svdq_w4a4_linear), without writing or reading h.
 * x [M][K] bf16 is the pre-GELU activation; the other arguments, layouts, ownership and
 * errors as for svdq_w4a4_linear. */
svdq_status svdq_w4a4_linear_gelu_in(const svdq_config* cfg, const svdq_w4a4_weight* w,
                                     const uint16_t* x, int64_t M, float act_global, uint16_t* y,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/* svdq_w4a4_linear for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, layouts, result and errors as svdq_w4a4_linear, without the workspace
 * arguments: the layer's intermediates (quantized activations, scales, partial
 * low-rank sums, and the GEMM's K-split partials when they fit) live in a scratch
 * array of svdq_noalloc_max_workspace_bytes() = 64 MiB that the library holds on each
 * device it runs on until the process ends.  The call allocates nothing and makes no
 * allocating library call; its first use on a device (or svdq_check_device on it)
 * looks up the array's address.  A shape whose workspace (svdq_workspace_bytes without
 * the optional K-split area) exceeds 64 MiB returns SVDQ_ERR_WORKSPACE before any device
 * access; for int4 that is about M * K <= 70 million (M = 4608 at K = 12288 fits).
 * Every call on one device shares that device's array: calls that overlap in time on
 * one device (other streams, other threads) race and give undefined results; calls
 * ordered on one stream are safe.  Nothing in the array needs to start at zero (every
 * call writes what it reads). */
size_t svdq_noalloc_max_workspace_bytes(void);
svdq_status svdq_w4a4_linear_noalloc(const svdq_config* cfg, const svdq_w4a4_weight* w,
                                     const uint16_t* x, int64_t M, float act_global, uint16_t* y,
                                     hipStream_t stream);

/* The fused QKV projection of a DiT attention block with its per-head Q/K RMSNorm and
 * rotary embedding in the GEMM epilogue (Diffusers docs "Nunchaku Lite", "Fused
 * kernels": the original engine fuses the Q, K, V projections with RMSNorm and RoPE;
 * the infolabhq tutorial's section on structural rewrites shows the unfused sequence:
 * split into heads, norm_q / norm_k, apply_rotary_emb).  The layer is the svdq_w4a4
 * linear with N = 3 H 128 output columns: [0, N/3) are Q, [N/3, 2N/3) K, [2N/3, N) V,
 * head h of Q (or K) the 128 columns [128 h, 128 h + 128) of its third.  With r the
 * linear's unrounded result (as svdq_w4a4_linear, bias included), for every token m and
 * every head of Q (weights norm_q) and of K (weights norm_k):
 *   n_c      = r_c / sqrt( mean_c(r_c^2) + eps ) * w_c        (c = 0..127, fp32)
 *   y_{2i}   = bf16_rne( n_{2i} cos[m][i] - n_{2i+1} sin[m][i] )
 *   y_{2i+1} = bf16_rne( n_{2i+1} cos[m][i] + n_{2i} sin[m][i] )  (i = 0..63)
 * and y = bf16_rne(r) on the V columns; one rounding per output.
 * norm_q, norm_k: device, bf16 [128].  rope: device, fp32 [M][64][2], (cos, sin) of
 * token m and pair i at rope[(m * 64 + i) * 2 + {0, 1}], the same for every head and
 * for Q and K.  eps: finite and positive (SVDQ_ERR_RANGE).  int4 and nvfp4 (act_global
 * as for svdq_w4a4_linear); N a multiple of 384 (SVDQ_ERR_SHAPE); every pointer
 * 16-byte aligned.  Workspace, stream and other errors as for svdq_w4a4_linear. */
svdq_status svdq_w4a4_linear_qkv_norm_rope(const svdq_config* cfg, const svdq_w4a4_weight* w,
                                           const uint16_t* x, int64_t M, float act_global,
                                           const uint16_t* norm_q, const uint16_t* norm_k,
                                           float eps, const float* rope, uint16_t* y,
                                           void* workspace, size_t workspace_bytes,
                                           hipStream_t stream);

/* The same per-head Q/K RMSNorm and rotary embedding as a separate pass over a bf16
 * QKV output x [M][N] (the unfused form: the projection is rounded to bf16 first, then
 * normalised and turned, in fp32, and rounded again).  y [M][N] receives the Q and K
 * thirds so transformed and, when y != x, a copy of the V third; y == x works in
 * place, other overlaps are undefined.  norm_q, norm_k, rope, eps and N as for
 * svdq_w4a4_linear_qkv_norm_rope; M >= 0 (M = 0 launches nothing).  Device pointers,
 * 16-byte aligned.  Errors: SVDQ_ERR_NULL, SVDQ_ERR_SHAPE, SVDQ_ERR_RANGE,
 * SVDQ_ERR_ALIGN, SVDQ_ERR_DEVICE, SVDQ_ERR_HIP.  Not recorded by the timing hook. */
svdq_status svdq_qk_norm_rope_bf16(const uint16_t* x, uint16_t* y, int64_t M, int64_t N,
                                   const uint16_t* norm_q, const uint16_t* norm_k, float eps,
                                   const float* rope, hipStream_t stream);

/* The AWQ W4A16 comparison layer: Y[M][N] (bf16) from bf16 X[M][K], the formula at
 * the top of this file.  Defined by the Diffusers docs "Nunchaku Lite", "Supported
 * quantization types" table (awq_w4a16: int4, group 64, an INT4 weight-only AWQ-style
 * kernel) and "NunchakuLiteQuantizationConfig" (awq_w4a16 targets keep bf16
 * activations).  cfg must be {int4, 64, rank 0, bf16}; the weight layout is
 * awq_w4a16_weight's; x, y device bf16, 16-byte aligned; M >= 0.  Errors as in the
 * conventions above. */
svdq_status awq_w4a16_linear(const svdq_config* cfg, const awq_w4a16_weight* w,
                             const uint16_t* x, int64_t M, uint16_t* y, hipStream_t stream);

/* Exact GELU of n bf16 values (Diffusers docs "Nunchaku Lite", "Fused kernels": the
 * activation of the DiT MLP between the MLP-up and MLP-down linears):
 *   y[i] = bf16_rne( x[i]/2 * erfc(-x[i]/sqrt(2)) ),  computed in fp32, erfc accurate to
 *   about 1e-7 relative (within 1 bf16 ulp of the exact value).
 * x, y: device pointers to n bf16 values, 16-byte aligned; y may equal x (in place),
 * other overlaps are undefined.  n in [0, 2^36]; n = 0 launches nothing.  Errors:
 * SVDQ_ERR_NULL, SVDQ_ERR_SHAPE, SVDQ_ERR_ALIGN, SVDQ_ERR_DEVICE, SVDQ_ERR_HIP.  Not
 * recorded by the timing hook below.  Enqueued on `stream`. */
svdq_status svdq_gelu_bf16(const uint16_t* x, uint16_t* y, int64_t n, hipStream_t stream);

/* Offline weight preparation on the GPU (the tutorial's calibrate -> SVDQuant ->
 * package step; Diffusers docs "Nunchaku Lite" introduction).  svdq_prepare_weight
 * prepares an svdq_w4a4 layer of cfg (int4 or nvfp4, rank cfg->rank) from W [K][N]
 * fp32 (Y = X W) and calibration activations x_cal [Mc][K] bf16:
 *   smooth[k] = bf16(fl32(1 / sqrt(max(amax_m |x_cal[m][k]|, 1e-5))))
 *   What = W / smooth (float64, per input row)
 *   What ~ L1 L2, L1 [K][r], L2 [r][N]: a randomized top-r factorization (Halko,
 *     Martinsson, Tropp 2011: range finder with power_iters power iterations on
 *     l = rank + oversample columns, CholeskyQR2, Jacobi eigen-decomposition of the
 *     projected l x l problem), each column of L1 signed so that its largest-magnitude
 *     entry is positive; lora_down [r][K] = bf16(L1^T), lora_up [N][r] = bf16(L2^T)
 *   R = What - L1_bf16 L2_bf16 (float64, stored as float32; residual [K][N] if not NULL)
 *   int4:  qweight [N][K/2] two's complement nibbles, wscales [N][K/64] bf16: R per
 *          output column in groups of 64, s = bf16(fl32(amax / 7)), q = rne(R / s)
 *   nvfp4: *w_global = fl32(amax|R| / 2688), qweight [N][K/2] E2M1 nibbles, wscales
 *          [N][K/16] E4M3 codes (the activation quantizer's rule on R per column), and
 *          *act_global = fl32(amax|bf16(x_cal smooth)| / 2688); w_global and
 *          act_global are host pointers (ignored for int4).
 * omega [N][l] float64 is the Gaussian test matrix (drawn by the caller).  The outputs
 * are the interchange layout of svdq_pack_weight / svdq_pack_lora_down.  rank 0: no
 * factorization, R = What, omega / lora pointers may be NULL.  rank + oversample <=
 * min(64, K, N); K and N multiples of 128.  Device pointers (except w_global and
 * act_global), 16-byte aligned; the workspace (svdq_prepare_workspace_bytes) is the
 * caller's.  Runs on `stream` and synchronizes it.  Errors: SVDQ_ERR_NULL,
 * SVDQ_ERR_CONFIG, SVDQ_ERR_SHAPE, SVDQ_ERR_ALIGN, SVDQ_ERR_WORKSPACE, SVDQ_ERR_DEVICE,
 * SVDQ_ERR_HIP, SVDQ_ERR_RANGE (the factorization broke down, What having rank below
 * l, or a zero NVFP4 tensor scale).
 *
 * awq_prepare_weight: the AWQ W4A16 layer's weights from W [K][N] fp32 (no smoothing,
 * no factorization): per output column and group of 64, s = bf16(fl32((max - min) /
 * 15)), z = clamp(rne(-min / s), 0, 15), q = clamp(rne(w / s) + z, 0, 15) (s = 0: all
 * zero); qweight [N][K/2], scales [N][K/64] bf16, zeros [N][K/64] u8.  Asynchronous on
 * `stream`; errors as above without SVDQ_ERR_WORKSPACE and SVDQ_ERR_RANGE. */
size_t svdq_prepare_workspace_bytes(int64_t K, int64_t N, int32_t rank, int32_t oversample);
svdq_status svdq_prepare_weight(const svdq_config* cfg, int64_t K, int64_t N, const float* w,
                                const uint16_t* x_cal, int64_t Mc, const double* omega,
                                int32_t oversample, int32_t power_iters, uint8_t* qweight,
                                void* wscales, uint16_t* smooth, uint16_t* lora_down,
                                uint16_t* lora_up, float* residual, float* w_global,
                                float* act_global, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);
svdq_status awq_prepare_weight(int64_t K, int64_t N, const float* w, uint8_t* qweight,
                               uint16_t* scales, uint8_t* zeros, hipStream_t stream);

/* Graph capture of a sequence of calls (Diffusers docs "Nunchaku Lite", "Fused kernels"
 * and the tutorial's torch.compile section: once the kernels are fused, what is left of
 * a denoise step's latency is launch overhead, which compiling the model recovers).
 * Here a caller records the launches of any sequence of the calls above, for example
 * the four linears and the GELU of a DiT block over several denoise steps, into one HIP
 * graph and replays it with one launch.
 *
 * svdq_capture_begin(stream) starts capturing `stream` in thread-local mode: until
 * svdq_capture_end, the calls that the calling thread makes on `stream` record their
 * kernels instead of running them.  `stream` must be a created stream (not the null
 * stream, which cannot be captured: SVDQ_ERR_CONFIG), per-kernel timing must be off
 * (SVDQ_ERR_CONFIG), and the calls made during capture must not allocate or
 * synchronize.  Nothing runs until the graph is launched; every buffer that a
 * recorded call names (inputs, outputs, workspace, weights) is bound by address and
 * must stay allocated, at the same address, while the graph may run.
 *
 * svdq_capture_end(stream, &graph) ends the capture, instantiates the recorded graph
 * and returns it through *graph (a handle that the caller owns; *graph is NULL on
 * error).  It must be called after every successful svdq_capture_begin, also when a
 * call during capture failed: a failed launch invalidates the capture, and then
 * svdq_capture_end returns SVDQ_ERR_HIP and no graph.  The instantiated graph holds
 * device resources of its own (HIP's), released by svdq_graph_destroy.
 *
 * svdq_graph_launch(graph, stream) enqueues one replay on `stream` (any stream of the
 * graph's device, the null stream included).  Replays on one stream run in order;
 * replays that overlap in time (on different streams) race on the shared buffers.
 *
 * svdq_graph_destroy(graph) releases the graph; NULL is allowed and does nothing.
 * Replays already enqueued complete normally.  Errors: SVDQ_ERR_NULL, SVDQ_ERR_CONFIG,
 * SVDQ_ERR_DEVICE, SVDQ_ERR_HIP. */
typedef struct svdq_graph svdq_graph;
svdq_status svdq_capture_begin(hipStream_t stream);
svdq_status svdq_capture_end(hipStream_t stream, svdq_graph** graph);
svdq_status svdq_graph_launch(const svdq_graph* graph, hipStream_t stream);
svdq_status svdq_graph_destroy(svdq_graph* graph);

/* Per-kernel timing, for measurement tools.  After svdq_timing_start(max_calls) and
 * until svdq_timing_stop, each svdq_w4a4_linear / awq_w4a16_linear call made on the
 * calling thread launches its kernels with a pair of HIP events that receive each
 * kernel's own start and end timestamps (hipExtLaunchKernelGGL; the first max_calls
 * calls only, 1 <= max_calls <= 65536).  The events are created by
 * svdq_timing_start and destroyed by svdq_timing_stop.  svdq_timing_stop waits for
 * the recorded events and returns, through host pointers, the number of recorded
 * calls, the number of kernels per call, and in mean_ms[i] (i < max_kernels) the
 * mean duration of kernel i in milliseconds.  Every recorded call must have
 * launched the same number of kernels, else SVDQ_ERR_CONFIG.  Calls made while
 * timing is off launch with null events. */
svdq_status svdq_timing_start(int max_calls);
svdq_status svdq_timing_stop(int* calls, int* kernels, float* mean_ms, int max_kernels);

/* ---- Measurement aid (not part of the layer): achievable dense MFMA rate ---------
 * The roofline of a GEMM is read against the chip's published dense matrix peak; these
 * calls measure what the matrix cores sustain for each instruction type the kernels
 * issue (FP6 and the 32x32x8 bf16 outer product in the int4 GEMM, fp16 in the NVFP4
 * GEMM, bf16 in the low-rank terms and the AWQ GEMM) and for the FP4, FP8 and int8
 * forms the published peaks are quoted for.
 *   op: 0 FP6 E2M3 32x32x64 (scaled, unit scales), 1 FP4 E2M1 32x32x64, 2 FP8 E4M3
 *       32x32x64, 3 int8 32x32x32, 4 fp16 32x32x16, 5 bf16 32x32x16, 6 bf16 32x32x8.
 * svdq_mfma_probe launches one 512-thread workgroup per CU of the current device;
 * every wave runs `iters` (1 .. 2^20) rounds of four independent MFMAs of type op on
 * register operands and writes one float per thread to `sink` (device,
 * svdq_mfma_probe_sink_floats() floats, 16-byte aligned; its values carry no meaning).
 * The caller times the launch (HIP events on `stream`); svdq_mfma_probe_ops(op, iters)
 * gives the operations (multiply and add counted separately) of one launch on the
 * current device, 0 for an invalid op or iters.  Errors: NULL sink -> SVDQ_ERR_NULL,
 * unknown op -> SVDQ_ERR_CONFIG, iters out of range -> SVDQ_ERR_RANGE, misaligned sink
 * -> SVDQ_ERR_ALIGN, no gfx950 device current -> SVDQ_ERR_DEVICE. */
int64_t svdq_mfma_probe_sink_floats(void);
double svdq_mfma_probe_ops(int op, int iters);
svdq_status svdq_mfma_probe(int op, int iters, float* sink, hipStream_t stream);

/* Human-readable name of a status code (static string). */
const char* svdq_status_str(svdq_status s);

/* Message describing the last error of the calling thread ("" if none). */
const char* svdq_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SVDQ_H */
