"""The C ABI on a host without a GPU: the library loads, exports every declared
symbol, and rejects bad arguments on the host before touching a device."""

import ctypes
import os
import re

import pytest
import torch

import w4a4_rank_corrected_linear_amd._lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HAVE_GPU = torch.cuda.is_available()

FAKE = 0x10000          # 16-byte aligned, never dereferenced: validation fails first
FAKE_MISALIGNED = 0x10008


def declared_functions():
    text = open(os.path.join(ROOT, "include", "svdq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = L.lib()
    names = declared_functions()
    assert {"svdq_w4a4_linear", "svdq_quantize_act", "awq_w4a16_linear"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"missing export {n}"


def test_status_strings():
    for s, name in enumerate(["SVDQ_OK", "SVDQ_ERR_NULL", "SVDQ_ERR_CONFIG", "SVDQ_ERR_SHAPE",
                              "SVDQ_ERR_ALIGN", "SVDQ_ERR_WORKSPACE", "SVDQ_ERR_DEVICE",
                              "SVDQ_ERR_HIP", "SVDQ_ERR_RANGE"]):
        assert L.status_str(s) == name


def cfg(precision=L.INT4, group=64, rank=32, dtype=L.BF16):
    return L.SvdqConfig(precision, group, rank, dtype)


def weight(K=512, N=512, rank=32, ptr=FAKE):
    lora = ptr if rank else None
    return L.SvdqW4A4Weight(K, N, ptr, ptr, 1.0, ptr, lora, lora, ptr)


def linear(c, w, M=16, ws_bytes=1 << 30, x=FAKE, y=FAKE, ws=FAKE):
    return L.lib().svdq_w4a4_linear(ctypes.byref(c), ctypes.byref(w), x, M, 1.0, y, ws, ws_bytes, None)


def test_config_table():
    """Supported (method, precision, group): svdq (int4, 64), svdq (nvfp4, 16),
    awq (int4, 64); anything else is SVDQ_ERR_CONFIG."""
    lib = L.lib()
    assert lib.svdq_workspace_bytes(ctypes.byref(cfg()), 16, 512) > 0
    for bad in [cfg(group=16), cfg(precision=L.NVFP4, group=64), cfg(group=32), cfg(rank=8),
                cfg(rank=64), cfg(dtype=1), cfg(precision=7)]:
        assert lib.svdq_workspace_bytes(ctypes.byref(bad), 16, 512) == 0
        assert linear(bad, weight()) == L.ERR_CONFIG
    awq = L.AwqW4A16Weight(512, 512, FAKE, FAKE, FAKE, None)
    assert lib.awq_w4a16_linear(ctypes.byref(cfg(rank=32)), ctypes.byref(awq), FAKE, 4, FAKE, None) == L.ERR_CONFIG
    assert lib.awq_w4a16_linear(ctypes.byref(cfg(group=16)), ctypes.byref(awq), FAKE, 4, FAKE, None) == L.ERR_CONFIG


def test_null_arguments():
    c = cfg()
    assert linear(c, weight(), x=None) == L.ERR_NULL
    assert linear(c, weight(), y=None) == L.ERR_NULL
    w = weight()
    w.lora_up = None
    assert linear(c, w) == L.ERR_NULL            # rank 32 needs both factors
    lib = L.lib()
    assert lib.svdq_quantize_act(ctypes.byref(c), None, 4, 512, FAKE, FAKE, 1.0, FAKE, FAKE, FAKE, None) == L.ERR_NULL
    assert lib.svdq_pack_weight(ctypes.byref(c), 512, 512, FAKE, None, FAKE, FAKE, None) == L.ERR_NULL
    assert "NULL" in L.last_error()


@pytest.mark.parametrize("K,N,M", [(500, 512, 4), (512, 500, 4), (64, 512, 4), (512, 64, 4),
                                   (512, 512, -1), (512, 200, 4)])
def test_shape_rules(K, N, M):
    assert linear(cfg(), weight(K, N), M=M) == L.ERR_SHAPE


def test_alignment():
    assert linear(cfg(), weight(), x=FAKE_MISALIGNED) == L.ERR_ALIGN
    assert linear(cfg(), weight(ptr=FAKE_MISALIGNED)) == L.ERR_ALIGN


def test_workspace_size_and_check():
    lib = L.lib()
    need = lib.svdq_workspace_bytes(ctypes.byref(cfg()), 100, 512)
    # M padded to 256 rows: operand 256*512*3/4, scale records 8*256*8, U 1 split x 256*32
    # fp32; then the GEMM's K-split area, 256 partial tiles of 256 x 192 fp32, which is
    # optional (a workspace without it is accepted)
    base = 98304 + 16384 + 32768
    split = 256 * 256 * 192 * 4
    assert need == base + split
    assert linear(cfg(), weight(), M=100, ws_bytes=base - 1) == L.ERR_WORKSPACE
    assert lib.svdq_workspace_bytes(ctypes.byref(cfg(rank=0)), 100, 512) == 98304 + 16384 + split
    nv = lib.svdq_workspace_bytes(ctypes.byref(cfg(precision=L.NVFP4, group=16)), 100, 512)
    # E2M1 codes (1/2 byte per value), fp16 block scales (1/8 byte per value) and U
    assert nv == 256 * 512 // 2 + 256 * 512 // 8 + 256 * 32 * 4


def test_workspace_sized_for_a_layer():
    """svdq_workspace_bytes_n: the K-split area sized for the layer's GEMM plan (on a
    host without a GPU the plan assumes 256 CUs)."""
    lib = L.lib()
    full = lib.svdq_workspace_bytes(ctypes.byref(cfg()), 4096, 3072)
    split = 256 * 256 * 192 * 4
    # 4096 x 3072 -> 3072: 256 tiles of 256 x 192, one round, no split
    assert lib.svdq_workspace_bytes_n(ctypes.byref(cfg()), 4096, 3072, 3072) == full - split
    # 4608 x 3072 -> 9216: 864 tiles leave a last round of 96, split into pieces
    qkv = lib.svdq_workspace_bytes_n(ctypes.byref(cfg()), 4608, 3072, 9216)
    full_qkv = lib.svdq_workspace_bytes(ctypes.byref(cfg()), 4608, 3072)
    assert full_qkv - split < qkv < full_qkv
    assert (qkv - (full_qkv - split)) % (256 * 192 * 4) == 0
    nv = cfg(precision=L.NVFP4, group=16)
    assert lib.svdq_workspace_bytes_n(ctypes.byref(nv), 100, 512, 384) == \
        lib.svdq_workspace_bytes(ctypes.byref(nv), 100, 512)
    assert lib.svdq_workspace_bytes_n(ctypes.byref(cfg()), 100, 512, 100) == 0     # N % 128
    assert lib.svdq_workspace_bytes_n(None, 100, 512, 384) == 0


def test_packed_weight_bytes():
    lib = L.lib()
    cb, sb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    tot = lib.svdq_packed_weight_bytes(ctypes.byref(cfg()), 3072, 3072, ctypes.byref(cb), ctypes.byref(sb))
    assert cb.value == 3072 * 3072 * 3 // 4      # E2M3 lane slots, 6 bits per weight
    assert sb.value == 24 * 3072 * 8 + 256     # 8-byte records per group pair + range flag
    assert tot == cb.value + sb.value


def test_empty_batch_is_ok_without_launch():
    assert linear(cfg(), weight(), M=0) == L.OK


@pytest.mark.skipif(HAVE_GPU, reason="a device is present: a valid call would launch")
def test_no_device_is_a_clear_error():
    assert L.lib().svdq_check_device(0) == L.ERR_DEVICE
    assert "device" in L.last_error().lower()
    assert linear(cfg(), weight(), M=16) == L.ERR_DEVICE


def test_python_layer_rejects_host_tensors():
    import w4a4_rank_corrected_linear_amd as svdq
    x = torch.zeros(4, 512, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        svdq.quantize_act(x, torch.zeros(512, dtype=torch.bfloat16))


def test_timing_hook_arguments():
    lib = L.lib()
    calls, kern = ctypes.c_int(-1), ctypes.c_int(-1)
    buf = (ctypes.c_float * 4)()
    assert lib.svdq_timing_start(0) == L.ERR_SHAPE
    assert lib.svdq_timing_start(65537) == L.ERR_SHAPE
    assert lib.svdq_timing_stop(None, ctypes.byref(kern), buf, 4) == L.ERR_NULL
    assert lib.svdq_timing_stop(ctypes.byref(calls), ctypes.byref(kern), buf, 4) == L.ERR_CONFIG
    assert calls.value == 0 and kern.value == 0


@pytest.mark.skipif(HAVE_GPU, reason="a device is present")
def test_timing_start_without_device_is_a_clear_error():
    assert L.lib().svdq_timing_start(8) == L.ERR_DEVICE


def test_nvfp4_sizes_and_global_scale_check():
    lib = L.lib()
    c = cfg(precision=L.NVFP4, group=16)
    # rows padded to the GEMM's 256-row tile: E2M1 codes 256 x 512 / 2, fp16 block
    # scales 256 x 512 / 8, U 256 x 32 x 4
    assert lib.svdq_workspace_bytes(ctypes.byref(c), 100, 512) == 65536 + 16384 + 32768
    cb, sb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    tot = lib.svdq_packed_weight_bytes(ctypes.byref(c), 512, 256, ctypes.byref(cb), ctypes.byref(sb))
    # 4 bits of code and (2 bytes / 16 =) 1 bit of scale per weight, then the flag trailer
    assert (cb.value, sb.value, tot) == (256 * 512 // 2, 256 * 512 // 8 + 256,
                                         256 * 512 // 2 + 256 * 512 // 8 + 256)
    w = weight()
    for gx, gw in [(0.0, 1.0), (1.0, 0.0), (float("nan"), 1.0), (1.0, float("inf")), (-1.0, 1.0)]:
        w.w_global = gw
        st = lib.svdq_w4a4_linear(ctypes.byref(c), ctypes.byref(w), FAKE, 16, gx, FAKE, FAKE, 1 << 30, None)
        assert st == L.ERR_RANGE, (gx, gw)
    assert lib.svdq_quantize_act(ctypes.byref(c), FAKE, 4, 512, FAKE, FAKE, 0.0, FAKE, FAKE, FAKE,
                                 None) == L.ERR_RANGE


def test_awq_argument_rules():
    lib = L.lib()
    c = cfg(rank=0)
    awq = L.AwqW4A16Weight(512, 512, FAKE, FAKE, FAKE, None)
    assert lib.awq_w4a16_linear(ctypes.byref(c), ctypes.byref(awq), FAKE, 0, FAKE, None) == L.OK
    assert lib.awq_w4a16_linear(ctypes.byref(c), ctypes.byref(awq), FAKE_MISALIGNED, 4, FAKE, None) == L.ERR_ALIGN
    bad = L.AwqW4A16Weight(500, 512, FAKE, FAKE, FAKE, None)
    assert lib.awq_w4a16_linear(ctypes.byref(c), ctypes.byref(bad), FAKE, 4, FAKE, None) == L.ERR_SHAPE
    nul = L.AwqW4A16Weight(512, 512, FAKE, None, FAKE, None)
    assert lib.awq_w4a16_linear(ctypes.byref(c), ctypes.byref(nul), FAKE, 4, FAKE, None) == L.ERR_NULL


def test_pack_lora_down_argument_rules():
    lib = L.lib()
    assert lib.svdq_pack_lora_down(ctypes.byref(cfg()), 512, None, FAKE, None) == L.ERR_NULL
    assert lib.svdq_pack_lora_down(ctypes.byref(cfg(rank=0)), 512, FAKE, FAKE, None) == L.ERR_CONFIG
    assert lib.svdq_pack_lora_down(ctypes.byref(cfg()), 500, FAKE, FAKE, None) == L.ERR_SHAPE
    assert lib.svdq_pack_lora_down(ctypes.byref(cfg()), 512, FAKE_MISALIGNED, FAKE, None) == L.ERR_ALIGN


def test_gelu_entry_points_validate_like_the_linear():
    lib = L.lib()
    c, w = cfg(), weight()
    args = lambda x=FAKE, M=16: (ctypes.byref(c), ctypes.byref(w), x, M, 1.0, FAKE, FAKE, 1 << 30, None)
    assert lib.svdq_w4a4_linear_gelu(*args(x=None)) == L.ERR_NULL
    assert lib.svdq_w4a4_linear_gelu(*args(x=FAKE_MISALIGNED)) == L.ERR_ALIGN
    assert lib.svdq_w4a4_linear_gelu(*args(M=0)) == L.OK
    assert "svdq_w4a4_linear_gelu" in (lib.svdq_w4a4_linear_gelu(*args(x=None)) and L.last_error())
    assert lib.svdq_w4a4_linear_gelu_in(*args(x=None)) == L.ERR_NULL
    assert lib.svdq_w4a4_linear_gelu_in(*args(x=FAKE_MISALIGNED)) == L.ERR_ALIGN
    assert lib.svdq_w4a4_linear_gelu_in(*args(M=0)) == L.OK
    assert "svdq_w4a4_linear_gelu_in" in (lib.svdq_w4a4_linear_gelu_in(*args(x=None)) and L.last_error())
    assert lib.svdq_gelu_bf16(None, FAKE, 8, None) == L.ERR_NULL
    assert lib.svdq_gelu_bf16(FAKE_MISALIGNED, FAKE, 8, None) == L.ERR_ALIGN
    assert lib.svdq_gelu_bf16(FAKE, FAKE, -1, None) == L.ERR_SHAPE
    assert lib.svdq_gelu_bf16(FAKE, FAKE, 0, None) == L.OK


def test_graph_entry_validation():
    """Graph capture entry points reject bad arguments on the host: the null stream
    cannot be captured, NULL handles are errors (destroying NULL is a no-op)."""
    lib = L.lib()
    assert lib.svdq_capture_begin(None) == L.ERR_CONFIG
    assert "null stream" in L.last_error()
    assert lib.svdq_capture_end(FAKE, None) == L.ERR_NULL
    g = ctypes.c_void_p(FAKE)
    assert lib.svdq_capture_end(None, ctypes.byref(g)) == L.ERR_CONFIG
    assert g.value is None
    assert lib.svdq_graph_launch(None, None) == L.ERR_NULL
    assert lib.svdq_graph_destroy(None) == L.OK


def test_qkv_norm_rope_entry_validation():
    """The fused QKV entry point: NULL norm weights or table, an unsupported config, N
    not a multiple of 384, eps not finite and positive, misaligned table."""
    lib = L.lib()

    def call(c, w, nq=FAKE, nk=FAKE, eps=1e-6, rope=FAKE):
        return lib.svdq_w4a4_linear_qkv_norm_rope(ctypes.byref(c), ctypes.byref(w), FAKE, 16, 1.0,
                                                  nq, nk, eps, rope, FAKE, FAKE, 1 << 30, None)

    w = weight(K=512, N=768)
    assert call(cfg(), w, nq=None) == L.ERR_NULL
    assert call(cfg(), w, rope=None) == L.ERR_NULL
    assert call(cfg(precision=L.NVFP4, group=16, rank=48), w) == L.ERR_CONFIG
    assert call(cfg(), weight(K=512, N=512)) == L.ERR_SHAPE
    for bad in (0.0, -1e-6, float("nan"), float("inf")):
        assert call(cfg(), w, eps=bad) == L.ERR_RANGE
    assert call(cfg(), w, rope=FAKE_MISALIGNED) == L.ERR_ALIGN


def test_mfma_probe_validation():
    lib = L.lib()
    assert lib.svdq_mfma_probe_sink_floats() % 512 == 0
    assert lib.svdq_mfma_probe_ops(0, 1) == lib.svdq_mfma_probe_sink_floats() / 64 * 4 * 2 * 32 * 32 * 64
    assert lib.svdq_mfma_probe_ops(7, 1) == 0.0 and lib.svdq_mfma_probe_ops(0, 0) == 0.0
    assert lib.svdq_mfma_probe(0, 16, None, None) == L.ERR_NULL
    assert lib.svdq_mfma_probe(7, 16, FAKE, None) == L.ERR_CONFIG
    assert lib.svdq_mfma_probe(-1, 16, FAKE, None) == L.ERR_CONFIG
    assert lib.svdq_mfma_probe(0, 0, FAKE, None) == L.ERR_RANGE
    assert lib.svdq_mfma_probe(0, (1 << 20) + 1, FAKE, None) == L.ERR_RANGE
    assert lib.svdq_mfma_probe(0, 16, FAKE_MISALIGNED, None) == L.ERR_ALIGN


def test_separate_qk_norm_rope_validation():
    lib = L.lib()

    def call(M=16, N=768, eps=1e-6, x=FAKE, rope=FAKE):
        return lib.svdq_qk_norm_rope_bf16(x, FAKE, M, N, FAKE, FAKE, eps, rope, None)

    assert call(x=None) == L.ERR_NULL
    assert call(rope=None) == L.ERR_NULL
    assert call(N=512) == L.ERR_SHAPE
    assert call(M=-1) == L.ERR_SHAPE
    assert call(eps=0.0) == L.ERR_RANGE
    assert call(rope=FAKE_MISALIGNED) == L.ERR_ALIGN
    assert call(M=0) == L.OK


def test_prepare_entry_validation():
    lib = L.lib()

    g1, g2 = ctypes.c_float(), ctypes.c_float()

    def call(K=512, N=512, rank=32, over=16, iters=4, Mc=8, w=FAKE, om=FAKE, nbytes=1 << 40,
             precision=L.INT4, glob=True):
        c = cfg(precision=precision, group=64 if precision == L.INT4 else 16, rank=rank)
        return lib.svdq_prepare_weight(ctypes.byref(c), K, N, w, FAKE, Mc, om, over, iters, FAKE,
                                       FAKE, FAKE, FAKE, FAKE, None,
                                       ctypes.byref(g1) if glob else None,
                                       ctypes.byref(g2) if glob else None, FAKE, nbytes, None)

    assert call(w=None) == L.ERR_NULL
    assert call(om=None) == L.ERR_NULL
    assert call(om=None, rank=0) != L.ERR_NULL        # rank 0 needs no test matrix
    assert call(precision=L.NVFP4, glob=False) == L.ERR_NULL
    assert call(rank=8) == L.ERR_CONFIG
    assert call(K=500) == L.ERR_SHAPE
    assert call(over=40) == L.ERR_SHAPE              # rank + oversample > 64
    assert call(Mc=0) == L.ERR_SHAPE
    assert call(nbytes=16) == L.ERR_WORKSPACE
    assert call(w=FAKE_MISALIGNED) == L.ERR_ALIGN
    need = lib.svdq_prepare_workspace_bytes(512, 512, 32, 16)
    assert need >= 512 * 512 * 12                      # float64 What and float32 residual

    assert lib.awq_prepare_weight(512, 512, None, FAKE, FAKE, FAKE, None) == L.ERR_NULL
    assert lib.awq_prepare_weight(500, 512, FAKE, FAKE, FAKE, FAKE, None) == L.ERR_SHAPE
    assert lib.awq_prepare_weight(512, 512, FAKE_MISALIGNED, FAKE, FAKE, FAKE, None) == L.ERR_ALIGN


def test_noalloc_entry_point_validates_on_the_host():
    """svdq_w4a4_linear_noalloc: the scratch maximum, NULL checks, and shapes whose
    workspace exceeds the scratch array rejected with SVDQ_ERR_WORKSPACE before any
    device access (here there is no device: a call that passed every host check would
    return SVDQ_ERR_DEVICE instead)."""
    lib = L.lib()
    assert lib.svdq_noalloc_max_workspace_bytes() == 64 << 20
    c = cfg()

    def call(w, M=16, x=FAKE, y=FAKE):
        return lib.svdq_w4a4_linear_noalloc(ctypes.byref(c), ctypes.byref(w), x, M, 1.0, y, None)

    assert call(weight(), x=None) == L.ERR_NULL
    assert call(weight(), y=None) == L.ERR_NULL
    assert call(weight(), x=FAKE_MISALIGNED) == L.ERR_ALIGN
    big = weight(K=12288, N=3072)
    assert call(big, M=8192) == L.ERR_WORKSPACE
    assert "64" in L.last_error() or "67108864" in L.last_error()
    if not HAVE_GPU:
        assert call(big, M=4608) == L.ERR_DEVICE      # fits: only the device check is left
        assert call(weight(), M=0) == L.OK            # nothing to do, no device access
