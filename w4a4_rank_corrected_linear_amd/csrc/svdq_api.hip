// Host side of the C ABI declared in include/svdq.h: argument validation (all on
// the host, before any device access), the per-device architecture check,
// workspace layout and kernel dispatch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "svdq.h"

#include "kernels.h"

namespace {

thread_local std::string g_last_error;

svdq_status fail(svdq_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

svdq_status ok() {
  g_last_error.clear();
  return SVDQ_OK;
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

svdq_status check_device_impl(int dev) {
  int count = 0;
  hipError_t e = hipGetDeviceCount(&count);
  if (e != hipSuccess || count <= 0)
    return fail(SVDQ_ERR_DEVICE, "no HIP device available (%s)",
                e != hipSuccess ? hipGetErrorString(e) : "device count is 0");
  if (dev < 0 || dev >= count)
    return fail(SVDQ_ERR_DEVICE, "device %d out of range (%d devices)", dev, count);
  if (dev < kMaxDevices) {
    const int st = g_arch_state[dev].load(std::memory_order_acquire);
    if (st == 1) return SVDQ_OK;
  }
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess)
    return fail(SVDQ_ERR_DEVICE, "hipGetDeviceProperties(%d) failed: %s", dev, hipGetErrorString(e));
  const bool good = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_arch_state[dev].store(good ? 1 : 2, std::memory_order_release);
  if (!good)
    return fail(SVDQ_ERR_DEVICE,
                "device %d is %s; this library is built for gfx950 (MI355X-class) only", dev,
                prop.gcnArchName);
  return SVDQ_OK;
}

svdq_status check_current_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return fail(SVDQ_ERR_DEVICE, "no current HIP device (%s)", hipGetErrorString(e));
  return check_device_impl(dev);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Device memory of the allocation-free entry point (svdq_w4a4_linear_noalloc): the
// layer's workspace lives in this array, one copy per device, held until the process
// ends.  Host code never passes the array's name to a kernel (in host code it is a
// stand-in, not a device address): its address on each device is looked up once,
// with that device current, and kept in g_scratch_addr.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];

// The scratch array's address on the current device (looked up on first use).
svdq_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return fail(SVDQ_ERR_DEVICE, "no current HIP device (%s)", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SVDQ_ERR_DEVICE, "device %d beyond the %d the library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(SVDQ_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  e != hipSuccess ? hipGetErrorString(e) : "null address");
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return SVDQ_OK;
}

int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

svdq_status check_svdq_config(const svdq_config* c) {
  if (c->compute_dtype != SVDQ_BF16)
    return fail(SVDQ_ERR_CONFIG, "compute_dtype %d unsupported (bf16 only)", c->compute_dtype);
  const bool int4 = c->precision == SVDQ_INT4 && c->group_size == 64;
  const bool nvfp4 = c->precision == SVDQ_NVFP4 && c->group_size == 16;
  if (!int4 && !nvfp4)
    return fail(SVDQ_ERR_CONFIG,
                "svdq_w4a4 supports (int4, group 64) and (nvfp4, group 16); got (precision %d, "
                "group %d)", c->precision, c->group_size);
  if (c->rank != 0 && c->rank != 16 && c->rank != 32)
    return fail(SVDQ_ERR_CONFIG, "rank %d unsupported (0, 16 or 32)", c->rank);
  return SVDQ_OK;
}

svdq_status check_k(int64_t K) {
  if (K < 128 || K % 128 != 0 || K > (int64_t(1) << 20))
    return fail(SVDQ_ERR_SHAPE, "K = %lld must be a positive multiple of 128 (<= 2^20)", (long long)K);
  return SVDQ_OK;
}

svdq_status check_n(int64_t N) {
  if (N < 128 || N % 128 != 0 || N > (int64_t(1) << 20))
    return fail(SVDQ_ERR_SHAPE, "N = %lld must be a positive multiple of 128 (<= 2^20)", (long long)N);
  return SVDQ_OK;
}

svdq_status check_m(int64_t M, int64_t K) {
  if (M < 0 || M > (int64_t(1) << 24) || M * K > (int64_t(1) << 36))
    return fail(SVDQ_ERR_SHAPE, "M = %lld out of range (0 <= M <= 2^24, M*K <= 2^36)", (long long)M);
  return SVDQ_OK;
}

svdq_status check_global(float g, const char* what) {
  if (!(g > 0.f) || !(g < 3.0e38f))
    return fail(SVDQ_ERR_RANGE, "nvfp4 %s scale %g must be finite and positive", what, (double)g);
  return SVDQ_OK;
}

struct WsLayout {
  int64_t M_pad = 0;
  size_t codes = 0, scales = 0, lora = 0, split = 0, total = 0;
};

WsLayout ws_layout(const svdq_config* c, int64_t M, int64_t K) {
  WsLayout L;
  const bool nv = c->precision == SVDQ_NVFP4;
  // row padding to the GEMMs' row tile (256)
  L.M_pad = round_up(M, 256);
  const int64_t G = K / c->group_size;
  // int4: GEMM A operand as E2M3 lane slots, 6 bits per value (3/4 byte), scale
  // records [G][M_pad] (8 bytes); nvfp4: E2M1 codes in FP4 lane slots (1/2 byte per
  // value) and fp16 block scales [K/64][M_pad][4] (1/8 byte per value)
  const size_t codes = nv ? (size_t)(L.M_pad * K / 2) : (size_t)(L.M_pad * K * 3 / 4);
  const size_t scales = nv ? (size_t)(L.M_pad * K / 8) : (size_t)(G * L.M_pad * 8);
  // fp32 partial U per k-split of the quantizer
  const size_t lora = (size_t)(svdq::k1_splits((int)K) * L.M_pad * c->rank * 4);
  L.codes = 0;
  L.scales = (size_t)round_up((int64_t)codes, 256);
  L.lora = L.scales + (size_t)round_up((int64_t)scales, 256);
  L.total = L.lora + (size_t)round_up((int64_t)lora, 256);
  if (!nv) {
    // int4: fp32 partial tiles of the GEMM's K-split of its last, partial round of
    // tiles; a workspace that stops short of this area runs without the split
    L.split = L.total;
    L.total = L.split + svdq::kSplitMaxPieces * svdq::kSplitTileBytes;
  }
  return L;
}

svdq_status hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SVDQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return SVDQ_OK;
}

#define SVDQ_TRY(expr)                    \
  do {                                    \
    const svdq_status _s = (expr);        \
    if (_s != SVDQ_OK) return _s;         \
  } while (0)

// Per-kernel timing of the calling thread (svdq_timing_start / svdq_timing_stop):
// each timed kernel gets a (start, end) event pair that hipExtLaunchKernelGGL fills
// with the kernel's own begin and end timestamps.
struct KernelTimer {
  bool on = false;
  std::vector<hipEvent_t> pool;           // created by svdq_timing_start
  size_t used = 0;
  std::vector<std::vector<int>> calls;    // per recorded call: event pairs (2i, 2i+1)
  int max_calls = 0;
  bool recording = false;                 // inside a call that is being recorded
};
thread_local KernelTimer g_timer;

void timer_begin_call() {
  KernelTimer& t = g_timer;
  t.recording = t.on && (int)t.calls.size() < t.max_calls;
  if (t.recording) t.calls.emplace_back();
}

struct EvPair {
  hipEvent_t start = nullptr, end = nullptr;
};

// Event pair for the next kernel of the current call (null events when not timing).
EvPair timer_kernel() {
  KernelTimer& t = g_timer;
  if (!t.recording) return {};
  if (t.used + 2 > t.pool.size()) {
    t.recording = false;
    t.calls.pop_back();
    return {};
  }
  const int idx = (int)t.used;
  t.used += 2;
  t.calls.back().push_back(idx);
  return {t.pool[idx], t.pool[idx + 1]};
}

void timer_release() {
  for (hipEvent_t e : g_timer.pool) (void)hipEventDestroy(e);
  g_timer = KernelTimer();
}

}  // namespace

extern "C" {

svdq_status svdq_check_device(int hip_device) {
  svdq_status s = check_device_impl(hip_device);
  if (s != SVDQ_OK) return s;
  // set-up of the allocation-free entry point: the scratch array's address on this
  // device, looked up with the device current
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return fail(SVDQ_ERR_DEVICE, "no current HIP device");
  if (cur != hip_device && hipSetDevice(hip_device) != hipSuccess)
    return fail(SVDQ_ERR_DEVICE, "cannot make device %d current", hip_device);
  void* p = nullptr;
  s = scratch_address(&p);
  if (cur != hip_device) (void)hipSetDevice(cur);
  return s == SVDQ_OK ? ok() : s;
}

size_t svdq_packed_weight_bytes(const svdq_config* cfg, int64_t K, int64_t N, size_t* codes_bytes,
                                size_t* scales_bytes) {
  if (!cfg || check_svdq_config(cfg) != SVDQ_OK || check_k(K) != SVDQ_OK || check_n(N) != SVDQ_OK) {
    if (codes_bytes) *codes_bytes = 0;
    if (scales_bytes) *scales_bytes = 0;
    return 0;
  }
  const int64_t G = K / cfg->group_size;
  // int4: E2M3 lane slots (3/4 byte per weight) and [G/2][N] 8-byte scale records,
  // one per pair of groups; nvfp4: E2M1 codes in FP4 lane slots (1/2 byte per weight)
  // and fp16 block scales [K/64][N][4] (1/8 byte per weight); both with a 256-byte
  // trailer (the range flag)
  const bool nv = cfg->precision == SVDQ_NVFP4;
  const size_t cb = nv ? (size_t)(N * K / 2) : (size_t)(N * K * 3 / 4);
  const size_t sb = (size_t)round_up(nv ? N * K / 8 : G / 2 * N * 8, 256) + 256;
  if (codes_bytes) *codes_bytes = cb;
  if (scales_bytes) *scales_bytes = sb;
  return cb + sb;
}

svdq_status svdq_pack_weight(const svdq_config* cfg, int64_t K, int64_t N, const uint8_t* codes,
                             const void* scales, uint8_t* packed_codes, void* packed_scales,
                             hipStream_t stream) {
  if (!cfg || !codes || !scales || !packed_codes || !packed_scales)
    return fail(SVDQ_ERR_NULL, "svdq_pack_weight: NULL argument");
  SVDQ_TRY(check_svdq_config(cfg));
  SVDQ_TRY(check_k(K));
  SVDQ_TRY(check_n(N));
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(packed_codes) || !aligned16(packed_scales))
    return fail(SVDQ_ERR_ALIGN, "svdq_pack_weight: pointers must be 16-byte aligned");
  SVDQ_TRY(check_current_device());
  const int64_t G = K / cfg->group_size;
  const bool nv = cfg->precision == SVDQ_NVFP4;
  int* flag = reinterpret_cast<int*>(static_cast<uint8_t*>(packed_scales) +
                                     round_up(nv ? N * K / 8 : G / 2 * N * 8, 256));
  if (nv)
    SVDQ_TRY(hip_check(svdq::launch_pack_nvfp4(codes, static_cast<const uint8_t*>(scales),
                                                packed_codes, static_cast<uint16_t*>(packed_scales),
                                                flag, (int)N, (int)K, stream),
                       "pack kernel launch"));
  else
    SVDQ_TRY(hip_check(svdq::launch_pack_int4(codes, static_cast<const uint16_t*>(scales),
                                               packed_codes, packed_scales,
                                               flag, (int)N, (int)K, stream),
                       "pack kernel launch"));
  int host_flag = 0;
  SVDQ_TRY(hip_check(hipMemcpyAsync(&host_flag, flag, sizeof(int), hipMemcpyDeviceToHost, stream),
                     "pack flag copy"));
  SVDQ_TRY(hip_check(hipStreamSynchronize(stream), "pack synchronize"));
  if (host_flag)
    return fail(SVDQ_ERR_RANGE, "nvfp4 weight scale is an E4M3 NaN code");
  return ok();
}

svdq_status svdq_pack_lora_down(const svdq_config* cfg, int64_t K, const uint16_t* lora_down,
                                uint16_t* packed, hipStream_t stream) {
  if (!cfg || !lora_down || !packed) return fail(SVDQ_ERR_NULL, "svdq_pack_lora_down: NULL argument");
  SVDQ_TRY(check_svdq_config(cfg));
  if (cfg->rank == 0) return fail(SVDQ_ERR_CONFIG, "svdq_pack_lora_down: rank 0 has no lora_down");
  SVDQ_TRY(check_k(K));
  if (!aligned16(lora_down) || !aligned16(packed))
    return fail(SVDQ_ERR_ALIGN, "svdq_pack_lora_down: pointers must be 16-byte aligned");
  SVDQ_TRY(check_current_device());
  SVDQ_TRY(hip_check(svdq::launch_pack_lora_down(lora_down, packed, cfg->rank, (int)K, stream),
                     "pack kernel launch"));
  return ok();
}

size_t svdq_workspace_bytes(const svdq_config* cfg, int64_t M, int64_t K) {
  if (!cfg || check_svdq_config(cfg) != SVDQ_OK || check_k(K) != SVDQ_OK || check_m(M, K) != SVDQ_OK)
    return 0;
  return ws_layout(cfg, M, K).total;
}

// Bytes of the int4 GEMM's K-split area for an N-column layer: the pieces of the plan
// taken with the full room, the larger of the plain (and GELU) plan and the fused-QKV
// one; 0 when neither splits.  The plan uses the current device's CU count (256 when no
// device is visible).
static size_t split_area_bytes(int64_t M_pad, int64_t N, int64_t K) {
  size_t best = 0;
  for (int epi : {svdq::kEpiPlain, svdq::kEpiQkNormRope}) {
    if (epi == svdq::kEpiQkNormRope && N % 384 != 0) continue;
    const svdq::K2Plan p =
        svdq::plan_k2_int4((int)M_pad, (int)N, (int)K, epi, svdq::kSplitMaxPieces);
    if (p.ks > 1) best = std::max(best, (size_t)(p.tiles - p.full) * p.ks * svdq::kSplitTileBytes);
  }
  return best;
}

size_t svdq_workspace_bytes_n(const svdq_config* cfg, int64_t M, int64_t K, int64_t N) {
  if (!cfg || check_svdq_config(cfg) != SVDQ_OK || check_k(K) != SVDQ_OK ||
      check_n(N) != SVDQ_OK || check_m(M, K) != SVDQ_OK)
    return 0;
  const WsLayout L = ws_layout(cfg, M, K);
  if (!L.split) return L.total;
  return L.split + split_area_bytes(L.M_pad, N, K);
}

svdq_status svdq_quantize_act(const svdq_config* cfg, const uint16_t* x, int64_t M, int64_t K,
                              const uint16_t* smooth, const uint16_t* lora_down, float act_global,
                              uint8_t* codes, void* scales, float* lora_act, hipStream_t stream) {
  if (!cfg || !x || !smooth || !codes || !scales)
    return fail(SVDQ_ERR_NULL, "svdq_quantize_act: NULL argument");
  SVDQ_TRY(check_svdq_config(cfg));
  const bool nv = cfg->precision == SVDQ_NVFP4;
  if (nv) SVDQ_TRY(check_global(act_global, "activation"));
  if (cfg->rank > 0 && (!lora_down || !lora_act))
    return fail(SVDQ_ERR_NULL, "svdq_quantize_act: rank %d needs lora_down and lora_act", cfg->rank);
  SVDQ_TRY(check_k(K));
  SVDQ_TRY(check_m(M, K));
  if (!aligned16(x) || !aligned16(smooth) || !aligned16(codes) || !aligned16(scales) ||
      (cfg->rank > 0 && (!aligned16(lora_down) || !aligned16(lora_act))))
    return fail(SVDQ_ERR_ALIGN, "svdq_quantize_act: pointers must be 16-byte aligned");
  if (M == 0) return ok();
  SVDQ_TRY(check_current_device());
  if (nv)
    SVDQ_TRY(hip_check(svdq::launch_k1_nvfp4(false, false, x, (int)M, (int)K, smooth,
                                              cfg->rank ? lora_down : nullptr, cfg->rank,
                                              act_global, codes, static_cast<uint8_t*>(scales),
                                              cfg->rank ? lora_act : nullptr, (int)M, stream),
                       "quantize kernel launch"));
  else
    SVDQ_TRY(hip_check(svdq::launch_k1_int4(false, false, x, (int)M, (int)K, smooth,
                                             cfg->rank ? lora_down : nullptr, cfg->rank, codes,
                                             static_cast<uint16_t*>(scales),
                                             cfg->rank ? lora_act : nullptr, (int)M, stream),
                       "quantize kernel launch"));
  return ok();
}

namespace {

// The layer call behind svdq_w4a4_linear and its variants: epi selects the GEMM's
// epilogue (plain, GELU on the output, the fused QKV norm and rotation); gelu_in makes
// the quantizer take bf16(gelu(x)) as the layer's input.
// The layer's workspace: the caller's buffer, or (scratch = true) the library's own
// scratch array of kScratchBytes, whose address is looked up after every host check.
struct Workspace {
  void* ptr;
  size_t bytes;
  bool scratch;
};

svdq_status linear_impl(const char* fn, const svdq_config* cfg, const svdq_w4a4_weight* w,
                        const uint16_t* x, int64_t M, float act_global, uint16_t* y,
                        Workspace wsa, int epi, const svdq::QkEpi& qk, hipStream_t stream,
                        bool gelu_in = false) {
  void* workspace = wsa.ptr;
  const size_t workspace_bytes = wsa.bytes;
  if (!cfg || !w || !x || !y || (!workspace && !wsa.scratch) || !w->qweight || !w->wscales ||
      !w->smooth)
    return fail(SVDQ_ERR_NULL, "%s: NULL argument", fn);
  if (epi == svdq::kEpiQkNormRope && (!qk.norm_q || !qk.norm_k || !qk.rope))
    return fail(SVDQ_ERR_NULL, "%s: NULL norm weight or rotary table", fn);
  SVDQ_TRY(check_svdq_config(cfg));
  const bool nv = cfg->precision == SVDQ_NVFP4;
  if (nv) {
    SVDQ_TRY(check_global(act_global, "activation"));
    SVDQ_TRY(check_global(w->w_global, "weight"));
  }
  if (cfg->rank > 0 && (!w->lora_down || !w->lora_up))
    return fail(SVDQ_ERR_NULL, "%s: rank %d needs lora_down and lora_up", fn, cfg->rank);
  SVDQ_TRY(check_k(w->K));
  SVDQ_TRY(check_n(w->N));
  SVDQ_TRY(check_m(M, w->K));
  if (M * w->N > (int64_t(1) << 36))
    return fail(SVDQ_ERR_SHAPE, "M * N too large");
  if (epi == svdq::kEpiQkNormRope && w->N % 384 != 0)
    return fail(SVDQ_ERR_SHAPE, "%s: N = %lld must be 3 x (a multiple of 128): Q, K, V of heads "
                "of 128", fn, (long long)w->N);
  if (epi == svdq::kEpiQkNormRope && !(std::isfinite(qk.eps) && qk.eps > 0.f))
    return fail(SVDQ_ERR_RANGE, "%s: eps = %g must be finite and positive", fn, (double)qk.eps);
  if (epi == svdq::kEpiQkNormRope &&
      (!aligned16(qk.norm_q) || !aligned16(qk.norm_k) || !aligned16(qk.rope)))
    return fail(SVDQ_ERR_ALIGN, "%s: pointers must be 16-byte aligned", fn);
  if (!aligned16(x) || !aligned16(y) || !aligned16(workspace) || !aligned16(w->qweight) ||
      !aligned16(w->wscales) || !aligned16(w->smooth) || (w->bias && !aligned16(w->bias)) ||
      (cfg->rank > 0 && (!aligned16(w->lora_down) || !aligned16(w->lora_up))))
    return fail(SVDQ_ERR_ALIGN, "%s: pointers must be 16-byte aligned", fn);
  const WsLayout L = ws_layout(cfg, M, w->K);
  const size_t need = L.split ? L.split : L.total;  // the split area is optional
  if (workspace_bytes < need) {
    if (wsa.scratch)
      return fail(SVDQ_ERR_WORKSPACE, "%s: M = %lld, K = %lld needs %zu bytes of workspace; the "
                  "allocation-free entry point holds at most %zu", fn, (long long)M,
                  (long long)w->K, need, workspace_bytes);
    return fail(SVDQ_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                workspace_bytes, need);
  }
  // K-split pieces the workspace has room for (the GEMM's plan splits only within them)
  const int split_pieces =
      L.split ? (int)std::min<size_t>(svdq::kSplitMaxPieces, (workspace_bytes - L.split) / svdq::kSplitTileBytes)
              : 0;
  if (M == 0) return ok();
  SVDQ_TRY(check_current_device());
  if (wsa.scratch) SVDQ_TRY(scratch_address(&workspace));
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint8_t* a_codes = ws + L.codes;
  uint2* a_scales = reinterpret_cast<uint2*>(ws + L.scales);
  float* a_lora = reinterpret_cast<float*>(ws + L.lora);
  timer_begin_call();
  const EvPair e1 = timer_kernel();
  if (nv) {
    SVDQ_TRY(hip_check(svdq::launch_k1_nvfp4(true, gelu_in, x, (int)M, (int)w->K, w->smooth,
                                              cfg->rank ? w->lora_down : nullptr, cfg->rank,
                                              act_global, a_codes, ws + L.scales,
                                              cfg->rank ? a_lora : nullptr, (int)L.M_pad, stream,
                                              e1.start, e1.end),
                       "quantize kernel launch"));
    const EvPair e2 = timer_kernel();
    const float g = act_global * w->w_global;
    SVDQ_TRY(hip_check(svdq::launch_k2_fp4(a_codes, reinterpret_cast<const uint16_t*>(ws + L.scales),
                                            a_lora, svdq::k1_splits((int)w->K), w->qweight,
                                            static_cast<const uint16_t*>(w->wscales), w->lora_up,
                                            w->bias, g, y, (int)M, (int)w->N, (int)w->K,
                                            (int)L.M_pad, cfg->rank, epi, qk, stream, e2.start,
                                            e2.end),
                       "gemm kernel launch"));
    return ok();
  }
  SVDQ_TRY(hip_check(svdq::launch_k1_int4(true, gelu_in, x, (int)M, (int)w->K, w->smooth,
                                           cfg->rank ? w->lora_down : nullptr, cfg->rank, a_codes,
                                           a_scales, cfg->rank ? a_lora : nullptr, (int)L.M_pad,
                                           stream, e1.start, e1.end),
                     "quantize kernel launch"));
  const svdq::K2Plan plan = svdq::plan_k2_int4((int)L.M_pad, (int)w->N, (int)w->K, epi,
                                               split_pieces);
  const EvPair e2 = timer_kernel();
  const EvPair e3 = plan.kernels() > 1 ? timer_kernel() : EvPair{};
  SVDQ_TRY(hip_check(svdq::launch_k2_int4(plan, a_codes, a_scales, a_lora,
                                           svdq::k1_splits((int)w->K), w->qweight,
                                           static_cast<const uint2*>(w->wscales), w->lora_up,
                                           w->bias, y, (int)M, (int)w->N, (int)w->K, (int)L.M_pad,
                                           cfg->rank, epi, qk,
                                           split_pieces ? reinterpret_cast<float*>(ws + L.split)
                                                      : nullptr,
                                           stream, e2.start, e2.end, e3.start, e3.end),
                     "gemm kernel launch"));
  return ok();
}

}  // namespace

svdq_status svdq_w4a4_linear(const svdq_config* cfg, const svdq_w4a4_weight* w, const uint16_t* x,
                             int64_t M, float act_global, uint16_t* y, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  return linear_impl("svdq_w4a4_linear", cfg, w, x, M, act_global, y,
                     Workspace{workspace, workspace_bytes, false},
                     svdq::kEpiPlain, svdq::QkEpi{}, stream);
}

svdq_status svdq_w4a4_linear_gelu(const svdq_config* cfg, const svdq_w4a4_weight* w,
                                  const uint16_t* x, int64_t M, float act_global, uint16_t* y,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return linear_impl("svdq_w4a4_linear_gelu", cfg, w, x, M, act_global, y,
                     Workspace{workspace, workspace_bytes, false}, svdq::kEpiGelu, svdq::QkEpi{},
                     stream);
}

svdq_status svdq_w4a4_linear_gelu_in(const svdq_config* cfg, const svdq_w4a4_weight* w,
                                     const uint16_t* x, int64_t M, float act_global, uint16_t* y,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return linear_impl("svdq_w4a4_linear_gelu_in", cfg, w, x, M, act_global, y,
                     Workspace{workspace, workspace_bytes, false}, svdq::kEpiPlain, svdq::QkEpi{},
                     stream, true);
}

size_t svdq_noalloc_max_workspace_bytes(void) { return kScratchBytes; }

svdq_status svdq_w4a4_linear_noalloc(const svdq_config* cfg, const svdq_w4a4_weight* w,
                                     const uint16_t* x, int64_t M, float act_global, uint16_t* y,
                                     hipStream_t stream) {
  return linear_impl("svdq_w4a4_linear_noalloc", cfg, w, x, M, act_global, y,
                     Workspace{nullptr, kScratchBytes, true}, svdq::kEpiPlain, svdq::QkEpi{},
                     stream);
}

svdq_status svdq_w4a4_linear_qkv_norm_rope(const svdq_config* cfg, const svdq_w4a4_weight* w,
                                           const uint16_t* x, int64_t M, float act_global,
                                           const uint16_t* norm_q, const uint16_t* norm_k,
                                           float eps, const float* rope, uint16_t* y,
                                           void* workspace, size_t workspace_bytes,
                                           hipStream_t stream) {
  return linear_impl("svdq_w4a4_linear_qkv_norm_rope", cfg, w, x, M, act_global, y,
                     Workspace{workspace, workspace_bytes, false}, svdq::kEpiQkNormRope,
                     svdq::QkEpi{norm_q, norm_k, rope, eps}, stream);
}

svdq_status awq_w4a16_linear(const svdq_config* cfg, const awq_w4a16_weight* w, const uint16_t* x,
                             int64_t M, uint16_t* y, hipStream_t stream) {
  if (!cfg || !w || !x || !y || !w->qweight || !w->scales || !w->zeros)
    return fail(SVDQ_ERR_NULL, "awq_w4a16_linear: NULL argument");
  if (cfg->precision != SVDQ_INT4 || cfg->group_size != 64 || cfg->rank != 0 ||
      cfg->compute_dtype != SVDQ_BF16)
    return fail(SVDQ_ERR_CONFIG, "awq_w4a16 supports (int4, group 64, rank 0, bf16) only");
  SVDQ_TRY(check_k(w->K));
  SVDQ_TRY(check_n(w->N));
  SVDQ_TRY(check_m(M, w->K));
  if (M * w->N > (int64_t(1) << 36)) return fail(SVDQ_ERR_SHAPE, "M * N too large");
  if (!aligned16(x) || !aligned16(y) || !aligned16(w->qweight) || !aligned16(w->scales) ||
      !aligned16(w->zeros) || (w->bias && !aligned16(w->bias)))
    return fail(SVDQ_ERR_ALIGN, "awq_w4a16_linear: pointers must be 16-byte aligned");
  if (M == 0) return ok();
  SVDQ_TRY(check_current_device());
  timer_begin_call();
  const EvPair e1 = timer_kernel();
  SVDQ_TRY(hip_check(svdq::launch_k4_awq(x, w->qweight, w->scales, w->zeros, w->bias, y, (int)M,
                                          (int)w->N, (int)w->K, stream, e1.start, e1.end),
                     "awq kernel launch"));
  return ok();
}

svdq_status svdq_gelu_bf16(const uint16_t* x, uint16_t* y, int64_t n, hipStream_t stream) {
  if (!x || !y) return fail(SVDQ_ERR_NULL, "svdq_gelu_bf16: NULL argument");
  if (n < 0 || n > (int64_t(1) << 36))
    return fail(SVDQ_ERR_SHAPE, "svdq_gelu_bf16: n = %lld out of [0, 2^36]", (long long)n);
  if (!aligned16(x) || !aligned16(y))
    return fail(SVDQ_ERR_ALIGN, "svdq_gelu_bf16: pointers must be 16-byte aligned");
  if (n == 0) return ok();
  SVDQ_TRY(check_current_device());
  SVDQ_TRY(hip_check(svdq::launch_gelu_bf16(x, y, n, stream), "gelu kernel launch"));
  return ok();
}

size_t svdq_prepare_workspace_bytes(int64_t K, int64_t N, int32_t rank, int32_t oversample) {
  if (K <= 0 || N <= 0 || rank < 0 || oversample < 0) return 0;
  return svdq::prep_workspace_bytes(K, N, rank, rank + oversample);
}

svdq_status svdq_prepare_weight(const svdq_config* cfg, int64_t K, int64_t N, const float* w,
                                const uint16_t* x_cal, int64_t Mc, const double* omega,
                                int32_t oversample, int32_t power_iters, uint8_t* qweight,
                                void* wscales, uint16_t* smooth, uint16_t* lora_down,
                                uint16_t* lora_up, float* residual, float* w_global,
                                float* act_global, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  if (!cfg || !w || !x_cal || !qweight || !wscales || !smooth || !workspace)
    return fail(SVDQ_ERR_NULL, "svdq_prepare_weight: NULL argument");
  SVDQ_TRY(check_svdq_config(cfg));
  const bool nv = cfg->precision == SVDQ_NVFP4;
  const int rank = cfg->rank;
  if (nv && (!w_global || !act_global))
    return fail(SVDQ_ERR_NULL, "svdq_prepare_weight: nvfp4 needs w_global and act_global");
  if (rank > 0 && (!omega || !lora_down || !lora_up))
    return fail(SVDQ_ERR_NULL, "svdq_prepare_weight: rank %d needs omega, lora_down and lora_up",
                rank);
  SVDQ_TRY(check_k(K));
  SVDQ_TRY(check_n(N));
  const int64_t l = rank + (int64_t)oversample;
  if (oversample < 0 || power_iters < 0 || power_iters > 64 || Mc < 1 || Mc > (int64_t(1) << 24) ||
      (rank > 0 && (l > 64 || l > std::min(K, N))))
    return fail(SVDQ_ERR_SHAPE, "svdq_prepare_weight: need Mc >= 1, 0 <= power_iters <= 64 and "
                "rank + oversample <= min(64, K, N)");
  if (!aligned16(w) || !aligned16(x_cal) || !aligned16(qweight) || !aligned16(wscales) ||
      !aligned16(smooth) || !aligned16(workspace) || (omega && !aligned16(omega)) ||
      (lora_down && !aligned16(lora_down)) || (lora_up && !aligned16(lora_up)) ||
      (residual && !aligned16(residual)))
    return fail(SVDQ_ERR_ALIGN, "svdq_prepare_weight: pointers must be 16-byte aligned");
  const size_t need = svdq::prep_workspace_bytes(K, N, rank, (int)l);
  if (workspace_bytes < need)
    return fail(SVDQ_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                workspace_bytes, need);
  SVDQ_TRY(check_current_device());
  int failed = 0;
  float globals[2] = {1.0f, 1.0f};
  SVDQ_TRY(hip_check(svdq::launch_prep(nv, (int)K, (int)N, rank, (int)l, power_iters, w, x_cal, Mc,
                                        omega, qweight, wscales, smooth, lora_down, lora_up,
                                        residual, workspace, &failed, globals, stream),
                     "weight preparation"));
  if (failed)
    return fail(SVDQ_ERR_RANGE, "svdq_prepare_weight: the factorization broke down (%s); the "
                "smoothed weight may have rank below rank + oversample",
                failed & 1 ? "Cholesky of a Gram matrix" : "non-positive singular value");
  if (nv) {
    if (!(globals[0] > 0.f) || !(globals[1] > 0.f))
      return fail(SVDQ_ERR_RANGE, "svdq_prepare_weight: an all-zero residual or calibration "
                  "set gives a zero NVFP4 tensor scale");
    *w_global = globals[0];
    *act_global = globals[1];
  }
  return ok();
}

svdq_status awq_prepare_weight(int64_t K, int64_t N, const float* w, uint8_t* qweight,
                               uint16_t* scales, uint8_t* zeros, hipStream_t stream) {
  if (!w || !qweight || !scales || !zeros)
    return fail(SVDQ_ERR_NULL, "awq_prepare_weight: NULL argument");
  SVDQ_TRY(check_k(K));
  SVDQ_TRY(check_n(N));
  if (!aligned16(w) || !aligned16(qweight) || !aligned16(scales) || !aligned16(zeros))
    return fail(SVDQ_ERR_ALIGN, "awq_prepare_weight: pointers must be 16-byte aligned");
  SVDQ_TRY(check_current_device());
  return hip_check(svdq::launch_prep_awq((int)K, (int)N, w, qweight, scales, zeros, stream),
                   "awq weight preparation");
}

struct svdq_graph {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

svdq_status svdq_capture_begin(hipStream_t stream) {
  if (!stream)
    return fail(SVDQ_ERR_CONFIG, "svdq_capture_begin: the null stream cannot be captured; "
                                 "pass a created stream");
  if (g_timer.on)
    return fail(SVDQ_ERR_CONFIG, "svdq_capture_begin: per-kernel timing is on; stop it first");
  SVDQ_TRY(check_current_device());
  return hip_check(hipStreamBeginCapture(stream, hipStreamCaptureModeThreadLocal),
                   "hipStreamBeginCapture");
}

svdq_status svdq_capture_end(hipStream_t stream, svdq_graph** graph) {
  if (!graph) return fail(SVDQ_ERR_NULL, "svdq_capture_end: NULL graph pointer");
  *graph = nullptr;
  if (!stream) return fail(SVDQ_ERR_CONFIG, "svdq_capture_end: the null stream is never captured");
  hipGraph_t g = nullptr;
  hipError_t e = hipStreamEndCapture(stream, &g);
  if (e != hipSuccess) {
    if (g) (void)hipGraphDestroy(g);
    return fail(SVDQ_ERR_HIP, "hipStreamEndCapture: %s", hipGetErrorString(e));
  }
  if (!g) return fail(SVDQ_ERR_HIP, "hipStreamEndCapture returned no graph");
  hipGraphExec_t x = nullptr;
  e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(g);
    return fail(SVDQ_ERR_HIP, "hipGraphInstantiate: %s", hipGetErrorString(e));
  }
  svdq_graph* h = new (std::nothrow) svdq_graph{g, x};
  if (!h) {
    (void)hipGraphExecDestroy(x);
    (void)hipGraphDestroy(g);
    return fail(SVDQ_ERR_HIP, "svdq_capture_end: out of host memory");
  }
  *graph = h;
  return ok();
}

svdq_status svdq_graph_launch(const svdq_graph* graph, hipStream_t stream) {
  if (!graph) return fail(SVDQ_ERR_NULL, "svdq_graph_launch: NULL graph");
  return hip_check(hipGraphLaunch(graph->exec, stream), "hipGraphLaunch");
}

svdq_status svdq_graph_destroy(svdq_graph* graph) {
  if (!graph) return ok();
  const hipError_t e1 = hipGraphExecDestroy(graph->exec);
  const hipError_t e2 = hipGraphDestroy(graph->graph);
  delete graph;
  SVDQ_TRY(hip_check(e1, "hipGraphExecDestroy"));
  return hip_check(e2, "hipGraphDestroy");
}

int64_t svdq_mfma_probe_sink_floats(void) { return (int64_t)svdq::device_cu_count() * 512; }

double svdq_mfma_probe_ops(int op, int iters) {
  if (op < svdq::kMfmaFp6 || op > svdq::kMfmaBf16K8 || iters < 1 || iters > (1 << 20)) return 0.0;
  // waves x rounds x four instructions x operations per instruction
  return (double)svdq::device_cu_count() * 8.0 * iters * 4.0 * svdq::mfma_probe_flops_per_instr(op);
}

svdq_status svdq_mfma_probe(int op, int iters, float* sink, hipStream_t stream) {
  if (!sink) return fail(SVDQ_ERR_NULL, "svdq_mfma_probe: NULL sink");
  if (op < svdq::kMfmaFp6 || op > svdq::kMfmaBf16K8)
    return fail(SVDQ_ERR_CONFIG, "svdq_mfma_probe: unknown instruction type %d", op);
  if (iters < 1 || iters > (1 << 20))
    return fail(SVDQ_ERR_RANGE, "svdq_mfma_probe: iters = %d outside [1, 2^20]", iters);
  if (!aligned16(sink)) return fail(SVDQ_ERR_ALIGN, "svdq_mfma_probe: sink must be 16-byte aligned");
  SVDQ_TRY(check_current_device());
  return hip_check(svdq::launch_mfma_probe(op, iters, sink, stream), "mfma probe launch");
}

svdq_status svdq_qk_norm_rope_bf16(const uint16_t* x, uint16_t* y, int64_t M, int64_t N,
                                   const uint16_t* norm_q, const uint16_t* norm_k, float eps,
                                   const float* rope, hipStream_t stream) {
  if (!x || !y || !norm_q || !norm_k || !rope)
    return fail(SVDQ_ERR_NULL, "svdq_qk_norm_rope_bf16: NULL argument");
  if (N <= 0 || N % 384 != 0 || N > (int64_t(1) << 20))
    return fail(SVDQ_ERR_SHAPE, "svdq_qk_norm_rope_bf16: N = %lld must be a positive multiple "
                "of 384 (<= 2^20)", (long long)N);
  if (M < 0 || M * N > (int64_t(1) << 36))
    return fail(SVDQ_ERR_SHAPE, "svdq_qk_norm_rope_bf16: M = %lld out of range", (long long)M);
  if (!(std::isfinite(eps) && eps > 0.f))
    return fail(SVDQ_ERR_RANGE, "svdq_qk_norm_rope_bf16: eps = %g must be finite and positive",
                (double)eps);
  if (!aligned16(x) || !aligned16(y) || !aligned16(norm_q) || !aligned16(norm_k) ||
      !aligned16(rope))
    return fail(SVDQ_ERR_ALIGN, "svdq_qk_norm_rope_bf16: pointers must be 16-byte aligned");
  if (M == 0) return ok();
  SVDQ_TRY(check_current_device());
  return hip_check(svdq::launch_qk_norm_rope_bf16(x, y, M, (int)N, norm_q, norm_k, eps, rope,
                                                  stream),
                   "qk norm kernel launch");
}

svdq_status svdq_timing_start(int max_calls) {
  if (max_calls < 1 || max_calls > 65536)
    return fail(SVDQ_ERR_SHAPE, "svdq_timing_start: max_calls = %d out of [1, 65536]", max_calls);
  timer_release();
  SVDQ_TRY(check_current_device());
  KernelTimer& t = g_timer;
  const size_t n = (size_t)max_calls * 6;  // room for up to three kernels per call
  t.pool.reserve(n);
  for (size_t i = 0; i < n; ++i) {
    hipEvent_t e;
    const hipError_t err = hipEventCreate(&e);
    if (err != hipSuccess) {
      timer_release();
      return fail(SVDQ_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(err));
    }
    t.pool.push_back(e);
  }
  t.max_calls = max_calls;
  t.on = true;
  return ok();
}

svdq_status svdq_timing_stop(int* calls, int* kernels, float* mean_ms, int max_kernels) {
  if (!calls || !kernels || (max_kernels > 0 && !mean_ms))
    return fail(SVDQ_ERR_NULL, "svdq_timing_stop: NULL argument");
  KernelTimer& t = g_timer;
  *calls = 0;
  *kernels = 0;
  if (!t.on) return fail(SVDQ_ERR_CONFIG, "svdq_timing_stop: timing was not started");
  const int nc = (int)t.calls.size();
  const int nk = nc ? (int)t.calls[0].size() : 0;
  for (const auto& c : t.calls)
    if ((int)c.size() != nk) {
      timer_release();
      return fail(SVDQ_ERR_CONFIG, "svdq_timing_stop: calls launched different kernel counts");
    }
  std::vector<double> sum(nk > 0 ? nk : 0, 0.0);
  for (const auto& c : t.calls) {
    const hipError_t e = nk ? hipEventSynchronize(t.pool[c.back() + 1]) : hipSuccess;
    if (e != hipSuccess) {
      timer_release();
      return fail(SVDQ_ERR_HIP, "hipEventSynchronize: %s", hipGetErrorString(e));
    }
    for (int i = 0; i < nk; ++i) {
      float ms = 0.f;
      const hipError_t e2 = hipEventElapsedTime(&ms, t.pool[c[i]], t.pool[c[i] + 1]);
      if (e2 != hipSuccess) {
        timer_release();
        return fail(SVDQ_ERR_HIP, "hipEventElapsedTime: %s", hipGetErrorString(e2));
      }
      sum[i] += ms;
    }
  }
  for (int i = 0; i < nk && i < max_kernels; ++i) mean_ms[i] = (float)(sum[i] / nc);
  *calls = nc;
  *kernels = nk;
  timer_release();
  return ok();
}

const char* svdq_status_str(svdq_status s) {
  switch (s) {
    case SVDQ_OK: return "SVDQ_OK";
    case SVDQ_ERR_NULL: return "SVDQ_ERR_NULL";
    case SVDQ_ERR_CONFIG: return "SVDQ_ERR_CONFIG";
    case SVDQ_ERR_SHAPE: return "SVDQ_ERR_SHAPE";
    case SVDQ_ERR_ALIGN: return "SVDQ_ERR_ALIGN";
    case SVDQ_ERR_WORKSPACE: return "SVDQ_ERR_WORKSPACE";
    case SVDQ_ERR_DEVICE: return "SVDQ_ERR_DEVICE";
    case SVDQ_ERR_HIP: return "SVDQ_ERR_HIP";
    case SVDQ_ERR_RANGE: return "SVDQ_ERR_RANGE";
  }
  return "SVDQ_ERR_UNKNOWN";
}

const char* svdq_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
