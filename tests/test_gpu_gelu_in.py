"""The second MLP linear taking the GELU of its input in the quantizer
(svdq_w4a4_linear_gelu_in): its workspace (4-bit codes, scales, low-rank partial sums)
and Y are byte-identical to svdq_gelu_bf16 followed by svdq_w4a4_linear, for both
precisions and both quantizer skeletons (32-row workgroups in one round, and resident
workgroups streaming 16-row units), with the full workspace and a guard region after
it compared; Y also against the oracle on the GELU'd input."""

import numpy as np
import pytest
import torch

import w4a4_rank_corrected_linear_amd as svdq
from helpers import check_y, dev_bf16, dev_u8, host_bits
from oracle import activation as A
from oracle import formats as F
from oracle import linear as OL
from oracle import prep as P
from synth import inputs as I

pytestmark = pytest.mark.gpu

GUARD = 1 << 20


def _int4_down():
    pb = I.chain_layer_bytes()["down"]                      # K = 12288 -> N = 3072
    oracle = P.SvdqLayer(precision="int4", K=pb.K, N=pb.N, rank=pb.rank, qweight=pb.qweight,
                         wscales=pb.wscales, w_global=1.0, act_global=1.0, smooth=pb.smooth,
                         lora_down=pb.lora_down, lora_up=pb.lora_up, bias=pb.bias)
    dev = svdq.SvdqLinear.from_interchange(dev_u8(pb.qweight), dev_bf16(pb.wscales),
                                           dev_bf16(pb.smooth), dev_bf16(pb.lora_down),
                                           dev_bf16(pb.lora_up), dev_bf16(pb.bias))
    return oracle, dev


def _nvfp4_square():
    pb = I.prepared_nvfp4_bytes(4, 3072, 3072, 32)          # K = 3072 -> N = 3072
    oracle = P.SvdqLayer(precision="nvfp4", K=3072, N=3072, rank=32, qweight=pb.qweight,
                         wscales=pb.wscales, w_global=pb.w_global, act_global=pb.act_global,
                         smooth=pb.smooth, lora_down=pb.lora_down, lora_up=pb.lora_up,
                         bias=pb.bias)
    dev = svdq.SvdqLinear.from_interchange(dev_u8(pb.qweight), dev_u8(pb.wscales),
                                           dev_bf16(pb.smooth), dev_bf16(pb.lora_down),
                                           dev_bf16(pb.lora_up), dev_bf16(pb.bias),
                                           precision="nvfp4", w_global=pb.w_global,
                                           act_global=pb.act_global)
    return oracle, dev


@pytest.fixture(scope="module")
def layers():
    return {"int4": _int4_down(), "nvfp4": _nvfp4_square()}


def _pre_gelu(M, K, seed):
    """MLP-up outputs stand-in: N(0, 1) with outlier channels x30 (both GELU tails)."""
    return I.activations(M, K, seed, I.outlier_channels(K, max(1, K // 100), seed + 1), 30.0)


# (precision, M): M = 200 runs the 32-row skeleton (7 row blocks x 8 or 2 k-splits);
# M = 4608 the row stream (144 row blocks x 8 or 2 k-splits > 256 CUs); M = 1 the
# smallest call.
CASES = [("int4", 1), ("int4", 200), ("int4", 4608), ("nvfp4", 200), ("nvfp4", 4608)]


@pytest.mark.parametrize("precision,M", CASES)
def test_gelu_in_equals_separate_gelu_then_linear(layers, precision, M):
    oracle, layer = layers[precision]
    print(f"[gelu_in] {precision} M={M} K={layer.K} N={layer.N}", flush=True)
    x_bits = _pre_gelu(M, layer.K, 7100 + M)
    x = dev_bf16(x_bits)
    need = layer.workspace_bytes(M)
    ws = [torch.full((need + GUARD,), 0xA5, dtype=torch.uint8, device=x.device) for _ in range(2)]
    h = svdq.gelu(x)
    y_sep = layer(h, workspace=ws[0][:need])
    y_fused = layer(x, workspace=ws[1][:need], gelu_in=True)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(y_fused), host_bits(y_sep))
    w0, w1 = ws[0].cpu().numpy(), ws[1].cpu().numpy()
    assert np.array_equal(w1[:need], w0[:need]), "workspace (codes, scales, U) differs"
    assert np.all(w1[need:] == 0xA5), "write past the workspace"
    # the hidden activation against the oracle's GELU, and Y against the oracle on it
    h_bits = host_bits(h)
    rows = np.unique(np.array([0, M // 3, M // 2, M - 1]))
    _, h_ref = A.gelu_bf16(x_bits[rows])
    assert int(F.bf16_ulp_distance(h_bits[rows], h_ref).max()) <= 1
    ref = OL.w4a4_linear_rows(precision, h_bits, oracle, rows)
    check_y(host_bits(y_fused)[rows], ref["r"])


def test_gelu_in_rejects_gelu_on_the_output_too(layers):
    _, layer = layers["int4"]
    x = dev_bf16(_pre_gelu(4, layer.K, 3))
    with pytest.raises(ValueError):
        layer(x, gelu=True, gelu_in=True)


@pytest.mark.parametrize("rank,M", [(0, 200), (0, 4608), (16, 200), (16, 4608)])
def test_gelu_in_low_ranks_and_no_bias(rank, M):
    """Ranks 0 (no low-rank branch, no bias) and 16 (one rank slice) on both quantizer
    skeletons: the same byte identity with the separate GELU pass."""
    K, N = 3072, 384
    pb = I.prepared_int4_bytes(12, K, N, rank=rank)
    bias = None if rank == 0 else pb.bias
    layer = svdq.SvdqLinear.from_interchange(
        dev_u8(pb.qweight), dev_bf16(pb.wscales), dev_bf16(pb.smooth),
        dev_bf16(pb.lora_down) if rank else None, dev_bf16(pb.lora_up) if rank else None,
        dev_bf16(bias) if bias is not None else None)
    print(f"[gelu_in] int4 rank={rank} M={M} K={K} N={N}", flush=True)
    x = dev_bf16(_pre_gelu(M, K, 7300 + rank + M))
    need = layer.workspace_bytes(M)
    ws = [torch.full((need + GUARD,), 0xA5, dtype=torch.uint8, device=x.device) for _ in range(2)]
    y_sep = layer(svdq.gelu(x), workspace=ws[0][:need])
    y_fused = layer(x, workspace=ws[1][:need], gelu_in=True)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(y_fused), host_bits(y_sep))
    w0, w1 = ws[0].cpu().numpy(), ws[1].cpu().numpy()
    assert np.array_equal(w1, w0)
    assert np.all(w1[need:] == 0xA5)
