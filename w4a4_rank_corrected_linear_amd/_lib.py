"""ctypes binding of libsvdq.so (the C ABI in include/svdq.h).

Argument marshalling only: every computation runs in the library's gfx950
kernels.  Loading fails loudly when the library has not been built.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# SVDQ_LIBRARY names another build of the same ABI (the host-ASan test build)
LIB_PATH = os.environ.get("SVDQ_LIBRARY") or os.path.join(_HERE, "libsvdq.so")

# status codes (svdq_status)
OK, ERR_NULL, ERR_CONFIG, ERR_SHAPE, ERR_ALIGN, ERR_WORKSPACE, ERR_DEVICE, ERR_HIP, ERR_RANGE = range(9)
INT4, NVFP4 = 0, 1
BF16 = 0


class SvdqConfig(ctypes.Structure):
    _fields_ = [("precision", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("rank", ctypes.c_int32), ("compute_dtype", ctypes.c_int32)]


class SvdqW4A4Weight(ctypes.Structure):
    _fields_ = [("K", ctypes.c_int64), ("N", ctypes.c_int64),
                ("qweight", ctypes.c_void_p), ("wscales", ctypes.c_void_p),
                ("w_global", ctypes.c_float),
                ("smooth", ctypes.c_void_p), ("lora_down", ctypes.c_void_p),
                ("lora_up", ctypes.c_void_p), ("bias", ctypes.c_void_p)]


class AwqW4A16Weight(ctypes.Structure):
    _fields_ = [("K", ctypes.c_int64), ("N", ctypes.c_int64),
                ("qweight", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("zeros", ctypes.c_void_p), ("bias", ctypes.c_void_p)]


class SvdqError(RuntimeError):
    def __init__(self, status: int, func: str, msg: str):
        self.status = status
        super().__init__(f"{func}: {status_str(status)}: {msg}")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (loaded once).  Raises if libsvdq.so is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the gfx950 library first "
            "(python -m w4a4_rank_corrected_linear_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, f32, st = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    cfgp = ctypes.POINTER(SvdqConfig)
    szp = ctypes.POINTER(ctypes.c_size_t)
    L.svdq_check_device.argtypes = [ctypes.c_int]
    L.svdq_check_device.restype = st
    L.svdq_packed_weight_bytes.argtypes = [cfgp, i64, i64, szp, szp]
    L.svdq_packed_weight_bytes.restype = ctypes.c_size_t
    L.svdq_pack_weight.argtypes = [cfgp, i64, i64, vp, vp, vp, vp, vp]
    L.svdq_pack_weight.restype = st
    L.svdq_pack_lora_down.argtypes = [cfgp, i64, vp, vp, vp]
    L.svdq_pack_lora_down.restype = st
    L.svdq_workspace_bytes_n.argtypes = [cfgp, i64, i64, i64]
    L.svdq_workspace_bytes_n.restype = ctypes.c_size_t
    L.svdq_workspace_bytes.argtypes = [cfgp, i64, i64]
    L.svdq_workspace_bytes.restype = ctypes.c_size_t
    L.svdq_quantize_act.argtypes = [cfgp, vp, i64, i64, vp, vp, f32, vp, vp, vp, vp]
    L.svdq_quantize_act.restype = st
    L.svdq_w4a4_linear.argtypes = [cfgp, ctypes.POINTER(SvdqW4A4Weight), vp, i64, f32, vp, vp,
                                   ctypes.c_size_t, vp]
    L.svdq_w4a4_linear.restype = st
    L.svdq_w4a4_linear_gelu.argtypes = [cfgp, ctypes.POINTER(SvdqW4A4Weight), vp, i64, f32, vp, vp,
                                   ctypes.c_size_t, vp]
    L.svdq_w4a4_linear_gelu.restype = st
    L.svdq_w4a4_linear_gelu_in.argtypes = [cfgp, ctypes.POINTER(SvdqW4A4Weight), vp, i64, f32, vp,
                                           vp, ctypes.c_size_t, vp]
    L.svdq_w4a4_linear_gelu_in.restype = st
    L.svdq_w4a4_linear_noalloc.argtypes = [cfgp, ctypes.POINTER(SvdqW4A4Weight), vp, i64, f32, vp, vp]
    L.svdq_w4a4_linear_noalloc.restype = st
    L.svdq_noalloc_max_workspace_bytes.argtypes = []
    L.svdq_noalloc_max_workspace_bytes.restype = ctypes.c_size_t
    L.svdq_w4a4_linear_qkv_norm_rope.argtypes = [cfgp, ctypes.POINTER(SvdqW4A4Weight), vp, i64, f32,
                                                 vp, vp, f32, vp, vp, vp, ctypes.c_size_t, vp]
    L.svdq_w4a4_linear_qkv_norm_rope.restype = st
    L.svdq_qk_norm_rope_bf16.argtypes = [vp, vp, i64, i64, vp, vp, f32, vp, vp]
    L.svdq_qk_norm_rope_bf16.restype = st
    L.awq_w4a16_linear.argtypes = [cfgp, ctypes.POINTER(AwqW4A16Weight), vp, i64, vp, vp]
    L.awq_w4a16_linear.restype = st
    L.svdq_gelu_bf16.argtypes = [vp, vp, i64, vp]
    L.svdq_gelu_bf16.restype = st
    L.svdq_prepare_workspace_bytes.argtypes = [i64, i64, ctypes.c_int32, ctypes.c_int32]
    L.svdq_prepare_workspace_bytes.restype = ctypes.c_size_t
    fp = ctypes.POINTER(ctypes.c_float)
    L.svdq_prepare_weight.argtypes = [cfgp, i64, i64, vp, vp, i64, vp, ctypes.c_int32, ctypes.c_int32,
                                      vp, vp, vp, vp, vp, vp, fp, fp, vp, ctypes.c_size_t, vp]
    L.svdq_prepare_weight.restype = st
    L.awq_prepare_weight.argtypes = [i64, i64, vp, vp, vp, vp, vp]
    L.awq_prepare_weight.restype = st
    L.svdq_capture_begin.argtypes = [vp]
    L.svdq_capture_begin.restype = st
    L.svdq_capture_end.argtypes = [vp, ctypes.POINTER(vp)]
    L.svdq_capture_end.restype = st
    L.svdq_graph_launch.argtypes = [vp, vp]
    L.svdq_graph_launch.restype = st
    L.svdq_graph_destroy.argtypes = [vp]
    L.svdq_graph_destroy.restype = st
    L.svdq_timing_start.argtypes = [ctypes.c_int]
    L.svdq_timing_start.restype = st
    ip = ctypes.POINTER(ctypes.c_int)
    L.svdq_timing_stop.argtypes = [ip, ip, ctypes.POINTER(ctypes.c_float), ctypes.c_int]
    L.svdq_timing_stop.restype = st
    L.svdq_mfma_probe_sink_floats.argtypes = []
    L.svdq_mfma_probe_sink_floats.restype = i64
    L.svdq_mfma_probe_ops.argtypes = [ctypes.c_int, ctypes.c_int]
    L.svdq_mfma_probe_ops.restype = ctypes.c_double
    L.svdq_mfma_probe.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp]
    L.svdq_mfma_probe.restype = st
    L.svdq_status_str.argtypes = [st]
    L.svdq_status_str.restype = ctypes.c_char_p
    L.svdq_last_error.argtypes = []
    L.svdq_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def status_str(s: int) -> str:
    return lib().svdq_status_str(s).decode()


def last_error() -> str:
    return lib().svdq_last_error().decode()


def check(status: int, func: str) -> None:
    if status != OK:
        raise SvdqError(status, func, last_error())


def config(precision: str = "int4", rank: int = 32, group_size: int | None = None) -> SvdqConfig:
    p = {"int4": INT4, "nvfp4": NVFP4}[precision]
    g = group_size if group_size is not None else (64 if p == INT4 else 16)
    return SvdqConfig(p, g, rank, BF16)
