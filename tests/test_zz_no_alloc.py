"""svdq_w4a4_linear_noalloc (the entry point for callers that cannot allocate device
memory) against svdq_w4a4_linear on the same inputs: identical outputs bit for bit,
and within the oracle's tolerance, on two calls in a row whose second input is smaller
(the scratch array keeps the first call's contents)."""

import numpy as np
import pytest
import torch

import w4a4_rank_corrected_linear_amd as svdq
from helpers import check_y, dev_bf16, dev_u8, host_bits
from oracle import linear as OL
from oracle import prep as P
from synth import inputs as I

pytestmark = pytest.mark.gpu


def _dev(layer):
    scales = dev_bf16(layer.wscales) if layer.precision == "int4" else dev_u8(layer.wscales)
    return svdq.SvdqLinear.from_interchange(
        dev_u8(layer.qweight), scales, dev_bf16(layer.smooth), dev_bf16(layer.lora_down),
        dev_bf16(layer.lora_up), dev_bf16(layer.bias), precision=layer.precision,
        w_global=layer.w_global, act_global=layer.act_global)


@pytest.mark.parametrize("precision", ["int4", "nvfp4"])
def test_noalloc_matches_linear_on_two_calls(precision):
    # K = 3072, N = 768: at 600 tokens the int4 GEMM splits every tile along K, and its
    # split area fits in the scratch array next to the quantized activations
    li = I.layer_inputs(config_id=1, M=600, K=3072, N=768, outlier_count=31, factor=30.0)
    layer = P.prepare_svdq(li.w, li.x_cal, li.bias, rank=32, precision=precision)
    dl = _dev(layer)
    assert int(svdq.lib().svdq_noalloc_max_workspace_bytes()) == 64 << 20
    for M in (600, 37):
        x = dev_bf16(li.x[:M])
        y_ref = host_bits(dl(x))
        out = torch.full((M, layer.N), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        y = host_bits(dl.forward_noalloc(x, out=out))
        assert np.array_equal(y, y_ref), (precision, M)
        check_y(y, OL.w4a4_linear(precision, li.x[:M], layer)["r"])


def test_noalloc_dit_shape_sampled_rows():
    """The largest DiT layer that fits the scratch array: MLP-down, M = 4608, K = 12288
    (about 54 MB of workspace, so the GEMM's optional K-split area does not fit and every
    tile runs whole); sampled rows against the oracle, and all rows against the workspace
    entry point given a workspace without the split area (the same launch plan)."""
    pb = I.prepared_int4_bytes(3, 12288, 3072, 32)
    sd = I.seeds(3)
    x = I.activations(4608, 12288, sd.x, I.outlier_channels(12288, 123, sd.outliers), 30.0)
    layer = P.SvdqLayer(precision="int4", K=12288, N=3072, rank=32, qweight=pb.qweight,
                        wscales=pb.wscales, w_global=1.0, act_global=1.0, smooth=pb.smooth,
                        lora_down=pb.lora_down, lora_up=pb.lora_up, bias=pb.bias)
    dl = _dev(layer)
    full = svdq.workspace_bytes("int4", 32, 4608, 12288)
    base = full - 256 * 256 * 192 * 4     # without the split area
    assert base <= 64 << 20 < full
    xd = dev_bf16(x)
    y = host_bits(dl.forward_noalloc(xd))
    rows = np.unique(np.concatenate([np.arange(11, 4608, 397), [4607]]))
    check_y(y[rows], OL.w4a4_linear_rows("int4", x, layer, rows)["r"])
    ws = torch.empty(base, dtype=torch.uint8, device="cuda")
    assert np.array_equal(y, host_bits(dl(xd, workspace=ws)))
