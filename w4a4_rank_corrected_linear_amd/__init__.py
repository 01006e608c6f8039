"""MI355X (gfx950) SVDQuant W4A4 linear layer.

Thin Python layer over libsvdq.so (include/svdq.h): torch supplies device memory
and the current HIP stream; all arithmetic runs in the library's kernels.

    import w4a4_rank_corrected_linear_amd as svdq
    layer = svdq.SvdqLinear.from_interchange(codes, scales, smooth, lora_down,
                                             lora_up, bias, precision="int4")
    y = layer(x)            # x: [M, K] bf16 CUDA tensor -> y: [M, N] bf16
"""

from ._lib import SvdqError, lib  # noqa: F401
from .api import (  # noqa: F401
    AwqLinear,
    Graph,
    SvdqLinear,
    awq_w4a16_linear,
    capture,
    check_device,
    gelu,
    MFMA_OPS,
    mfma_probe,
    pack_lora_down,
    pack_weight,
    prepare_awq_layer,
    prepare_layer,
    qk_norm_rope,
    quantize_act,
    timing_start,
    timing_stop,
    workspace_bytes,
)
from .chain import DitBlockChain  # noqa: F401
