"""torch-facing wrappers of the C ABI: allocation of outputs and workspace with
torch, the current HIP stream, and argument marshalling.  No arithmetic here."""

from __future__ import annotations

import ctypes

import torch

from . import _lib as L


def _p(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _want(t: torch.Tensor, dtype, name: str, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def check_device(device: int | None = None) -> None:
    dev = torch.cuda.current_device() if device is None else device
    L.check(L.lib().svdq_check_device(dev), "svdq_check_device")


def workspace_bytes(precision: str, rank: int, M: int, K: int) -> int:
    cfg = L.config(precision, rank)
    return int(L.lib().svdq_workspace_bytes(ctypes.byref(cfg), M, K))


_SHARED_WS: dict = {}


def shared_workspace(need: int, device) -> torch.Tensor:
    """A uint8 workspace of at least `need` bytes for calls on `device`'s current stream,
    kept per (device, stream) and reused by every layer (reallocated larger when a call
    needs more).  Layers run on different streams get different buffers."""
    dev = torch.device(device)
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    key = (idx, torch.cuda.current_stream(idx).cuda_stream)
    ws = _SHARED_WS.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=torch.device("cuda", idx))
        _SHARED_WS[key] = ws
    return ws


def _scale_dtype(precision: str):
    return torch.bfloat16 if precision == "int4" else torch.uint8


def quantize_act(x: torch.Tensor, smooth: torch.Tensor, lora_down: torch.Tensor | None = None,
                 precision: str = "int4", act_global: float = 1.0):
    """svdq_quantize_act: returns (codes [M, K/2] u8, scales [M, K/G], lora_act [M, r] fp32)."""
    _want(x, torch.bfloat16, "x")
    M, K = x.shape
    _want(smooth, torch.bfloat16, "smooth", (K,))
    rank = 0 if lora_down is None else lora_down.shape[0]
    if lora_down is not None:
        _want(lora_down, torch.bfloat16, "lora_down", (rank, K))
    cfg = L.config(precision, rank)
    G = K // cfg.group_size
    codes = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((M, G), dtype=_scale_dtype(precision), device=x.device)
    lora_act = torch.empty((M, rank), dtype=torch.float32, device=x.device) if rank else None
    st = L.lib().svdq_quantize_act(ctypes.byref(cfg), _p(x), M, K, _p(smooth), _p(lora_down),
                                   float(act_global), _p(codes), _p(scales), _p(lora_act), _stream())
    L.check(st, "svdq_quantize_act")
    return codes, scales, lora_act


def pack_weight(codes: torch.Tensor, scales: torch.Tensor, precision: str = "int4"):
    """svdq_pack_weight: interchange [N, K/2] codes + [N, K/G] scales -> kernel layout.

    Returns (packed_codes, packed_scales) as uint8 tensors.  Synchronizes the stream.
    """
    _want(codes, torch.uint8, "codes")
    N, K2 = codes.shape
    K = 2 * K2
    cfg = L.config(precision, 0)
    _want(scales, _scale_dtype(precision), "scales", (N, K // cfg.group_size))
    cb, sb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    total = L.lib().svdq_packed_weight_bytes(ctypes.byref(cfg), K, N, ctypes.byref(cb), ctypes.byref(sb))
    if total == 0:
        L.check(L.ERR_SHAPE, "svdq_packed_weight_bytes")
    pc = torch.empty(cb.value, dtype=torch.uint8, device=codes.device)
    ps = torch.empty(sb.value, dtype=torch.uint8, device=codes.device)
    st = L.lib().svdq_pack_weight(ctypes.byref(cfg), K, N, _p(codes), _p(scales), _p(pc), _p(ps),
                                  _stream())
    L.check(st, "svdq_pack_weight")
    return pc, ps


def pack_lora_down(lora_down: torch.Tensor, precision: str = "int4") -> torch.Tensor:
    """svdq_pack_lora_down: [r, K] bf16 -> the quantizer's fragment order (same size)."""
    _want(lora_down, torch.bfloat16, "lora_down")
    rank, K = lora_down.shape
    cfg = L.config(precision, rank)
    out = torch.empty_like(lora_down)
    L.check(L.lib().svdq_pack_lora_down(ctypes.byref(cfg), K, _p(lora_down), _p(out), _stream()),
            "svdq_pack_lora_down")
    return out


class SvdqLinear:
    """A prepared svdq_w4a4 layer resident in device memory.

    smooth [K] bf16, lora_up [N, r] bf16, bias [N] bf16 or None; qweight/wscales and
    lora_down in the kernel layouts (see ``pack_weight`` and ``pack_lora_down``).
    """

    def __init__(self, K: int, N: int, qweight, wscales, smooth, lora_down, lora_up, bias,
                 precision: str = "int4", w_global: float = 1.0, act_global: float = 1.0):
        self.K, self.N = K, N
        self.precision = precision
        self.rank = 0 if lora_down is None else lora_down.shape[0]
        self.qweight, self.wscales = qweight, wscales
        self.smooth, self.lora_down, self.lora_up, self.bias = smooth, lora_down, lora_up, bias
        self.w_global, self.act_global = float(w_global), float(act_global)
        self.cfg = L.config(precision, self.rank)
        self._w = L.SvdqW4A4Weight(K, N, qweight.data_ptr(), wscales.data_ptr(), self.w_global,
                                   smooth.data_ptr(),
                                   None if lora_down is None else lora_down.data_ptr(),
                                   None if lora_up is None else lora_up.data_ptr(),
                                   None if bias is None else bias.data_ptr())

    @classmethod
    def from_interchange(cls, codes, scales, smooth, lora_down, lora_up, bias,
                         precision: str = "int4", w_global: float = 1.0, act_global: float = 1.0):
        N, K2 = codes.shape
        pc, ps = pack_weight(codes, scales, precision)
        ld = None if lora_down is None else pack_lora_down(lora_down, precision)
        return cls(2 * K2, N, pc, ps, smooth, ld, lora_up, bias, precision, w_global, act_global)

    def workspace_bytes(self, M: int) -> int:
        """svdq_workspace_bytes_n for M tokens of this layer (at least 256): the int4
        K-split area is sized for this layer's own GEMM plan."""
        return max(int(L.lib().svdq_workspace_bytes_n(ctypes.byref(self.cfg), M, self.K, self.N)), 256)

    def workspace(self, M: int, device) -> torch.Tensor:
        """The default workspace: one buffer per (device, current stream), shared by every
        layer and grown on demand, since calls ordered on one stream never overlap."""
        return shared_workspace(self.workspace_bytes(M), device)

    def forward(self, x: torch.Tensor, out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None, act_global: float | None = None,
                gelu: bool = False, gelu_in: bool = False):
        """y = layer(x); with gelu=True the exact GELU of each result is taken before the
        bf16 rounding (svdq_w4a4_linear_gelu); with gelu_in=True the layer runs on
        bf16(gelu(x)), formed by the quantizer as it loads x (svdq_w4a4_linear_gelu_in)."""
        if gelu and gelu_in:
            raise ValueError("gelu and gelu_in together: no entry point takes both")
        _want(x, torch.bfloat16, "x")
        M, K = x.shape
        if K != self.K:
            raise ValueError(f"x has K = {K}, layer expects {self.K}")
        y = torch.empty((M, self.N), dtype=torch.bfloat16, device=x.device) if out is None else out
        if M == 0:  # nothing to compute (empty tensors carry no device address)
            return y
        ws = self.workspace(M, x.device) if workspace is None else workspace
        g = self.act_global if act_global is None else float(act_global)
        fn = ("svdq_w4a4_linear_gelu" if gelu else
              "svdq_w4a4_linear_gelu_in" if gelu_in else "svdq_w4a4_linear")
        st = getattr(L.lib(), fn)(ctypes.byref(self.cfg), ctypes.byref(self._w), _p(x), M, g,
                                  _p(y), _p(ws), ws.numel(), _stream())
        L.check(st, fn)
        return y

    __call__ = forward

    def forward_noalloc(self, x: torch.Tensor, out: torch.Tensor | None = None,
                        act_global: float | None = None):
        """y = layer(x) through svdq_w4a4_linear_noalloc: the library's own scratch
        array holds the workspace (no device allocation in the call; ``out`` may be
        given so that nothing is allocated here either)."""
        _want(x, torch.bfloat16, "x")
        M, K = x.shape
        if K != self.K:
            raise ValueError(f"x has K = {K}, layer expects {self.K}")
        y = torch.empty((M, self.N), dtype=torch.bfloat16, device=x.device) if out is None else out
        if M == 0:  # nothing to compute (empty tensors carry no device address)
            return y
        g = self.act_global if act_global is None else float(act_global)
        fn = "svdq_w4a4_linear_noalloc"
        st = getattr(L.lib(), fn)(ctypes.byref(self.cfg), ctypes.byref(self._w), _p(x), M, g,
                                  _p(y), _stream())
        L.check(st, fn)
        return y

    def qkv_norm_rope(self, x: torch.Tensor, norm_q: torch.Tensor, norm_k: torch.Tensor,
                      eps: float, rope: torch.Tensor, out: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None, act_global: float | None = None):
        """The fused QKV projection (svdq_w4a4_linear_qkv_norm_rope): per-head RMSNorm
        (norm_q / norm_k, bf16 [128]) and the rotary turn (rope, float32 [M, 64, 2] of
        cos, sin) on the Q and K thirds of the output; V as the plain linear."""
        _want(x, torch.bfloat16, "x")
        M, K = x.shape
        if K != self.K:
            raise ValueError(f"x has K = {K}, layer expects {self.K}")
        _want(norm_q, torch.bfloat16, "norm_q", (128,))
        _want(norm_k, torch.bfloat16, "norm_k", (128,))
        _want(rope, torch.float32, "rope", (M, 64, 2))
        y = torch.empty((M, self.N), dtype=torch.bfloat16, device=x.device) if out is None else out
        if M == 0:  # nothing to compute (empty tensors carry no device address)
            return y
        ws = self.workspace(M, x.device) if workspace is None else workspace
        g = self.act_global if act_global is None else float(act_global)
        fn = "svdq_w4a4_linear_qkv_norm_rope"
        st = getattr(L.lib(), fn)(ctypes.byref(self.cfg), ctypes.byref(self._w), _p(x), M, g,
                                  _p(norm_q), _p(norm_k), float(eps), _p(rope), _p(y), _p(ws),
                                  ws.numel(), _stream())
        L.check(st, fn)
        return y


def prepare_layer(w: torch.Tensor, x_cal: torch.Tensor, bias: torch.Tensor | None = None,
                  precision: str = "int4", rank: int = 32, oversample: int = 16,
                  power_iters: int = 8, seed: int = 0) -> "SvdqLinear":
    """Prepare an svdq_w4a4 layer on the GPU (svdq_prepare_weight) from W [K, N] float32
    (Y = X W) and calibration activations x_cal [Mc, K] bf16, then pack it: smoothing,
    a randomized rank-r factorization (the Gaussian test matrix is drawn here with
    torch's generator from ``seed``) and the quantized residual."""
    _want(w, torch.float32, "w")
    _want(x_cal, torch.bfloat16, "x_cal")
    K, N = w.shape
    dev = w.device
    ell = rank + oversample
    gen = torch.Generator(device="cpu").manual_seed(seed)
    omega = torch.randn((N, ell), generator=gen, dtype=torch.float64).to(dev) if rank else None
    nv = precision == "nvfp4"
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    scales = (torch.empty((N, K // 16), dtype=torch.uint8, device=dev) if nv else
              torch.empty((N, K // 64), dtype=torch.bfloat16, device=dev))
    smooth = torch.empty((K,), dtype=torch.bfloat16, device=dev)
    ldown = torch.empty((rank, K), dtype=torch.bfloat16, device=dev) if rank else None
    lup = torch.empty((N, rank), dtype=torch.bfloat16, device=dev) if rank else None
    nbytes = int(L.lib().svdq_prepare_workspace_bytes(K, N, rank, oversample))
    work = torch.empty((nbytes,), dtype=torch.uint8, device=dev)
    gw, gx = ctypes.c_float(1.0), ctypes.c_float(1.0)
    cfg = L.config(precision, rank)
    L.check(L.lib().svdq_prepare_weight(ctypes.byref(cfg), K, N, _p(w), _p(x_cal), x_cal.shape[0],
                                        _p(omega), oversample, power_iters, _p(codes), _p(scales),
                                        _p(smooth), _p(ldown), _p(lup), None, ctypes.byref(gw),
                                        ctypes.byref(gx), _p(work), nbytes, _stream()),
            "svdq_prepare_weight")
    return SvdqLinear.from_interchange(codes, scales, smooth, ldown, lup, bias, precision,
                                       w_global=gw.value, act_global=gx.value)


def prepare_awq_layer(w: torch.Tensor, bias: torch.Tensor | None = None) -> "AwqLinear":
    """AWQ W4A16 weights prepared on the GPU (awq_prepare_weight) from W [K, N] float32."""
    _want(w, torch.float32, "w")
    K, N = w.shape
    dev = w.device
    q = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    s = torch.empty((N, K // 64), dtype=torch.bfloat16, device=dev)
    z = torch.empty((N, K // 64), dtype=torch.uint8, device=dev)
    L.check(L.lib().awq_prepare_weight(K, N, _p(w), _p(q), _p(s), _p(z), _stream()),
            "awq_prepare_weight")
    return AwqLinear(q, s, z, bias)


class AwqLinear:
    """An awq_w4a16 layer: qweight [N, K/2] u8, scales [N, K/64] bf16, zeros [N, K/64] u8."""

    def __init__(self, qweight, scales, zeros, bias=None):
        N, K2 = qweight.shape
        self.K, self.N = 2 * K2, N
        self.qweight, self.scales, self.zeros, self.bias = qweight, scales, zeros, bias
        self.cfg = L.config("int4", 0)
        self._w = L.AwqW4A16Weight(self.K, N, qweight.data_ptr(), scales.data_ptr(),
                                   zeros.data_ptr(), None if bias is None else bias.data_ptr())

    def forward(self, x: torch.Tensor, out: torch.Tensor | None = None):
        return awq_w4a16_linear(x, self, out)

    __call__ = forward


def awq_w4a16_linear(x: torch.Tensor, layer: AwqLinear, out: torch.Tensor | None = None):
    _want(x, torch.bfloat16, "x")
    M, K = x.shape
    y = torch.empty((M, layer.N), dtype=torch.bfloat16, device=x.device) if out is None else out
    st = L.lib().awq_w4a16_linear(ctypes.byref(layer.cfg), ctypes.byref(layer._w), _p(x), M, _p(y),
                                  _stream())
    L.check(st, "awq_w4a16_linear")
    return y


def gelu(x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """svdq_gelu_bf16: exact (erf) GELU of a contiguous bf16 device tensor; `out` may
    be `x` (in place)."""
    _want(x, torch.bfloat16, "x")
    y = torch.empty_like(x) if out is None else _want(out, torch.bfloat16, "out", tuple(x.shape))
    L.check(L.lib().svdq_gelu_bf16(_p(x), _p(y), x.numel(), _stream()), "svdq_gelu_bf16")
    return y


class Graph:
    """An instantiated HIP graph of recorded library calls (svdq_capture_end); replay it
    with ``launch``.  The buffers the recorded calls named must stay alive while it may
    run; ``keep`` holds references to them."""

    def __init__(self, handle: int, keep=()):
        self._h = ctypes.c_void_p(handle)
        self.keep = tuple(keep)

    def launch(self) -> None:
        """Enqueue one replay on the current stream."""
        if not self._h.value:
            raise RuntimeError("graph was destroyed")
        L.check(L.lib().svdq_graph_launch(self._h, _stream()), "svdq_graph_launch")

    def destroy(self) -> None:
        if self._h.value:
            L.check(L.lib().svdq_graph_destroy(self._h), "svdq_graph_destroy")
            self._h = ctypes.c_void_p(None)
        self.keep = ()

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def capture(fn, keep=()) -> Graph:
    """Record the library calls that fn() makes into one HIP graph.  fn runs on a side
    stream under thread-local capture (the null stream cannot be captured); it must not
    allocate device memory or synchronize, so create its buffers before (one eager call
    does).  Returns the instantiated Graph; nothing has run yet."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st = _stream()
        L.check(L.lib().svdq_capture_begin(st), "svdq_capture_begin")
        err = None
        try:
            fn()
        except BaseException as e:  # the capture must still be ended
            err = e
        h = ctypes.c_void_p()
        st_end = L.lib().svdq_capture_end(st, ctypes.byref(h))
    torch.cuda.current_stream().wait_stream(side)
    if err is not None:
        if h.value:
            L.lib().svdq_graph_destroy(h)
        raise err
    L.check(st_end, "svdq_capture_end")
    return Graph(h.value, keep)


def qk_norm_rope(x: torch.Tensor, norm_q: torch.Tensor, norm_k: torch.Tensor, eps: float,
                 rope: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """svdq_qk_norm_rope_bf16: per-head Q/K RMSNorm + rotary embedding of a bf16 QKV
    output [M, N] (out=x works in place; V is copied when out is another tensor)."""
    _want(x, torch.bfloat16, "x")
    M, N = x.shape
    _want(norm_q, torch.bfloat16, "norm_q", (128,))
    _want(norm_k, torch.bfloat16, "norm_k", (128,))
    _want(rope, torch.float32, "rope", (M, 64, 2))
    y = torch.empty_like(x) if out is None else _want(out, torch.bfloat16, "out", (M, N))
    if M == 0:
        return y
    L.check(L.lib().svdq_qk_norm_rope_bf16(_p(x), _p(y), M, N, _p(norm_q), _p(norm_k),
                                           float(eps), _p(rope), _stream()),
            "svdq_qk_norm_rope_bf16")
    return y


def timing_start(max_calls: int) -> None:
    """svdq_timing_start: record per-kernel HIP events in the next `max_calls` layer
    calls made on this thread."""
    L.check(L.lib().svdq_timing_start(int(max_calls)), "svdq_timing_start")


def timing_stop(max_kernels: int = 4):
    """svdq_timing_stop: returns (calls, [mean ms of kernel i])."""
    calls, kernels = ctypes.c_int(0), ctypes.c_int(0)
    buf = (ctypes.c_float * max_kernels)()
    L.check(L.lib().svdq_timing_stop(ctypes.byref(calls), ctypes.byref(kernels), buf, max_kernels),
            "svdq_timing_stop")
    return calls.value, [float(buf[i]) for i in range(min(kernels.value, max_kernels))]


# Instruction types of the dense MFMA rate probe (svdq_mfma_probe), by name.
MFMA_OPS = {"fp6": 0, "fp4": 1, "fp8": 2, "int8": 3, "fp16": 4, "bf16": 5, "bf16_k8": 6}


def mfma_probe(op: str, iters: int, sink: torch.Tensor | None = None) -> tuple[torch.Tensor, float]:
    """svdq_mfma_probe: one launch of the dense MFMA rate probe for instruction type
    `op` (a key of MFMA_OPS) on the current stream; returns (sink, operations of the
    launch).  The caller times it."""
    n = int(L.lib().svdq_mfma_probe_sink_floats())
    if sink is None:
        sink = torch.empty(n, dtype=torch.float32, device="cuda")
    _want(sink, torch.float32, "sink", (n,))
    L.check(L.lib().svdq_mfma_probe(MFMA_OPS[op], int(iters), _p(sink), _stream()), "svdq_mfma_probe")
    return sink, float(L.lib().svdq_mfma_probe_ops(MFMA_OPS[op], int(iters)))
