"""The C ABI's largest shapes on the GPU, against the oracle.

- K = 2^20, the longest reduction the ABI takes: 683 quantizer k-splits summed by the
  GEMM, 8192 (int4) or 16384 (nvfp4, AWQ) stages in one tile, which the int4 GEMM
  splits along K.
- N = 2^20, the widest layer: 8192 column tiles of 128.
- M = 2^24, the most tokens: 65536 row tiles, byte offsets past 2^32 into X, the
  workspace and Y.  X repeats a block of 4099 rows (a prime, so a row index that
  wrapped around a power of two would land on a different block row), and sampled rows
  from the whole range, the last one included, are checked.
"""

import numpy as np
import pytest
import torch

import w4a4_rank_corrected_linear_amd as svdq
from helpers import check_y, dev_bf16, dev_u8, host_bits
from oracle import linear as OL
from oracle import prep as P
from synth import inputs as I

pytestmark = pytest.mark.gpu

CID = 8  # seeds of its own


def _svdq_layer(precision, K, N):
    if precision == "int4":
        pb = I.prepared_int4_bytes(CID, K, N, 32)
        g = dict(w_global=1.0, act_global=1.0)
    else:
        pb = I.prepared_nvfp4_bytes(CID, K, N, 32)
        g = dict(w_global=pb.w_global, act_global=pb.act_global)
    return P.SvdqLayer(precision=precision, K=K, N=N, rank=32, qweight=pb.qweight,
                       wscales=pb.wscales, smooth=pb.smooth, lora_down=pb.lora_down,
                       lora_up=pb.lora_up, bias=pb.bias, **g)


def _svdq_dev(layer):
    scales = dev_bf16(layer.wscales) if layer.precision == "int4" else dev_u8(layer.wscales)
    return svdq.SvdqLinear.from_interchange(
        dev_u8(layer.qweight), scales, dev_bf16(layer.smooth), dev_bf16(layer.lora_down),
        dev_bf16(layer.lora_up), dev_bf16(layer.bias), precision=layer.precision,
        w_global=layer.w_global, act_global=layer.act_global)


def _x(M, K):
    sd = I.seeds(CID)
    return I.activations(M, K, sd.x, I.outlier_channels(K, I.default_outlier_count(K), sd.outliers),
                         30.0)


@pytest.mark.parametrize("precision", ["int4", "nvfp4"])
@pytest.mark.parametrize("K,N", [(1 << 20, 128), (128, 1 << 20)])
def test_svdq_longest_k_and_widest_n(precision, K, N):
    layer = _svdq_layer(precision, K, N)
    x = _x(3, K)
    y = host_bits(_svdq_dev(layer)(dev_bf16(x)))
    check_y(y, OL.w4a4_linear(precision, x, layer)["r"])


@pytest.mark.parametrize("K,N", [(1 << 20, 128), (128, 1 << 20)])
def test_awq_longest_k_and_widest_n(K, N):
    pb = I.prepared_awq_bytes(CID, K, N)
    awq = P.AwqLayer(K=K, N=N, group=64, qweight=pb.qweight, scales=pb.scales, zeros=pb.zeros,
                     bias=pb.bias)
    x = _x(3, K)
    dev = svdq.AwqLinear(dev_u8(pb.qweight), dev_bf16(pb.scales), dev_u8(pb.zeros), dev_bf16(pb.bias))
    check_y(host_bits(dev(dev_bf16(x))), OL.awq_w4a16_linear(x, awq)["r"])


def test_svdq_most_tokens():
    M, K, N, P0 = 1 << 24, 128, 128, 4099
    layer = _svdq_layer("int4", K, N)
    x0 = _x(P0, K)
    xd = dev_bf16(x0).repeat((M + P0 - 1) // P0, 1)[:M].contiguous()
    y = _svdq_dev(layer)(xd)
    rows = np.array([0, 1, P0, (1 << 21) + 7, (1 << 22) + 5, (1 << 23) + 12345,
                     (1 << 24) - P0 - 1, (1 << 24) - 2, (1 << 24) - 1])
    ys = host_bits(y[torch.from_numpy(rows).cuda()])
    del xd, y
    check_y(ys, OL.w4a4_linear("int4", x0[rows % P0], layer)["r"])
