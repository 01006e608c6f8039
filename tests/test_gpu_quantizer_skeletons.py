"""Bit-exact checks of every quantizer kernel that svdq_w4a4_linear launches, at the
shapes where each one runs.  The layer's quantizer has two skeletons per precision, picked
by whether (rows / 32) x (k-splits) workgroups fit one round on the 256 CUs:

  int4   k1_int4_fused (32 rows)    at M = 4096, K = 3072   (128 x 2 = 256)
         k1_int4_stream (16-row units streamed through resident workgroups)
                                    at M = 4608, K = 3072  (144 x 2 = 288; 128 workgroups
                                    per k-split, two or three units each)
                                    and M = 4608, K = 12288 (144 x 8; 32 per split, 9 each)
  nvfp4  k1_nvfp4_fused32 (32 rows) at M = 4096, K = 3072
         k1_nvfp4_stream            at M = 4608, K = 3072 and M = 4096, K = 12288

The workspace the linear leaves behind (filled with 0xA5 beforehand, followed by a guard
region) is decoded and compared with the oracle: codes and scales bit for bit, the
partial low-rank sums within the fp32 bound, zeros in the padding rows.  The
standalone svdq_quantize_act (interchange layout) runs on the same rows, so the fused
and unfused quantizers are checked against each other as well."""

import numpy as np
import pytest
import torch

import w4a4_rank_corrected_linear_amd as svdq
from helpers import (check_u, dev_bf16, dev_u8, host_bits, int4_workspace,
                     nvfp4_workspace_values)
from oracle import formats as F
from oracle import prep as P
from oracle import quant as Q
from synth import inputs as I

pytestmark = pytest.mark.gpu

GUARD = 1 << 20


def _run_linear(dl, x, M):
    need = dl.workspace_bytes(M)
    buf = torch.full((need + GUARD,), 0xA5, dtype=torch.uint8, device="cuda")
    dl(dev_bf16(x), workspace=buf[:need])
    torch.cuda.synchronize()
    assert bool((buf[need:] == 0xA5).all()), "the linear wrote past its workspace"
    return host_bits(buf[:need])


def _inputs(cid, M, K, N, precision, rank=32):
    sd = I.seeds(cid)
    x = I.activations(M, K, sd.x, I.outlier_channels(K, I.default_outlier_count(K), sd.outliers),
                      30.0)
    if precision == "int4":
        pb = I.prepared_int4_bytes(cid, K, N, rank)
        gw = gx = 1.0
    else:
        pb = I.prepared_nvfp4_bytes(cid, K, N, rank)
        gw, gx = pb.w_global, pb.act_global
    layer = P.SvdqLayer(precision=precision, K=K, N=N, rank=rank, qweight=pb.qweight,
                        wscales=pb.wscales, w_global=gw, act_global=gx, smooth=pb.smooth,
                        lora_down=pb.lora_down, lora_up=pb.lora_up, bias=pb.bias)
    return x, layer


def _dev(layer):
    scales = dev_bf16(layer.wscales) if layer.precision == "int4" else dev_u8(layer.wscales)
    return svdq.SvdqLinear.from_interchange(
        dev_u8(layer.qweight), scales, dev_bf16(layer.smooth),
        dev_bf16(layer.lora_down) if layer.rank else None,
        dev_bf16(layer.lora_up) if layer.rank else None, dev_bf16(layer.bias),
        precision=layer.precision, w_global=layer.w_global, act_global=layer.act_global)


@pytest.mark.parametrize("M,K", [(4096, 3072), (4608, 3072), (4608, 12288)])
def test_int4_layer_quantizer_bitexact(M, K):
    x, layer = _inputs(3 if M == 4608 else 2, M, K, 384, "int4")
    M_pad = -(-M // 256) * 256
    w = _run_linear(_dev(layer), x, M)
    ref = Q.quantize_act_int4(x, layer.smooth, layer.lora_down)
    q, s, u = int4_workspace(w, M_pad, K, 32)
    assert np.array_equal(q[:M], ref["q"])
    assert np.array_equal(s[:, :M], ref["scales"].T)
    assert np.all(q[M:] == 0) and np.all(s[:, M:] == 0)
    usum = u.astype(np.float64).sum(axis=0)
    check_u(usum[:M], ref, layer.lora_down)
    assert np.all(u[:, M:] == 0)
    # the standalone quantizer on the same rows: the interchange form of the same codes
    codes, scales, ua = svdq.quantize_act(dev_bf16(x), dev_bf16(layer.smooth),
                                          dev_bf16(layer.lora_down))
    assert np.array_equal(host_bits(codes), ref["codes"])
    assert np.array_equal(host_bits(scales), ref["scales"])
    check_u(host_bits(ua), ref, layer.lora_down)


@pytest.mark.parametrize("M,K", [(4096, 3072), (4608, 3072), (4096, 12288)])
def test_nvfp4_layer_quantizer_bitexact(M, K):
    x, layer = _inputs(4, M, K, 384, "nvfp4")
    M_pad = -(-M // 256) * 256
    w = _run_linear(_dev(layer), x, M)
    ref = Q.quantize_act_nvfp4(x, layer.smooth, layer.act_global, layer.lora_down)
    a = nvfp4_workspace_values(w, M_pad, K)
    expect = F.e2m1_decode(ref["e2m1"]) * np.repeat(F.e4m3_decode(ref["scales"]), 16, axis=1)
    assert np.array_equal(a[:M], expect)
    assert np.all(a[M:] == 0)
    codes, scales, ua = svdq.quantize_act(dev_bf16(x), dev_bf16(layer.smooth),
                                          dev_bf16(layer.lora_down), precision="nvfp4",
                                          act_global=layer.act_global)
    assert np.array_equal(host_bits(codes), ref["codes"])
    assert np.array_equal(host_bits(scales), ref["scales"])
    check_u(host_bits(ua), ref, layer.lora_down)


# The row-stream skeleton with padding rows (M = 4500: M_pad = 4608, so the 16-row unit
# 281 holds 4 real rows and units 282..287 none) and every rank it supports: its wait
# counts depend on the rank (which waves store a partial-U float4) and it has no barrier
# at rank 0.  K = 3200 ends in a k-split of one 128-wide block, where eleven of the
# twelve waves own no block and only take part in the barriers.
@pytest.mark.parametrize("rank,K", [(0, 3072), (16, 3072), (32, 3072), (32, 3200)])
def test_int4_stream_quantizer_ragged_rows(rank, K):
    M = 4500
    x, layer = _inputs(9, M, K, 384, "int4", rank=rank)
    M_pad = -(-M // 256) * 256
    assert (M_pad // 32) * (K // 1536) > 256     # the row-stream skeleton
    w = _run_linear(_dev(layer), x, M)
    ref = Q.quantize_act_int4(x, layer.smooth, layer.lora_down if rank else None)
    q, s, u = int4_workspace(w, M_pad, K, rank)
    assert np.array_equal(q[:M], ref["q"])
    assert np.array_equal(s[:, :M], ref["scales"].T)
    assert np.all(q[M:] == 0) and np.all(s[:, M:] == 0)
    if rank:
        check_u(u.astype(np.float64).sum(axis=0)[:M], ref, layer.lora_down)
        assert np.all(u[:, M:] == 0)


def test_nvfp4_stream_quantizer_ragged_rows():
    M, K = 4500, 3072
    x, layer = _inputs(9, M, K, 384, "nvfp4", rank=16)
    M_pad = -(-M // 256) * 256
    w = _run_linear(_dev(layer), x, M)
    ref = Q.quantize_act_nvfp4(x, layer.smooth, layer.act_global, layer.lora_down)
    a = nvfp4_workspace_values(w, M_pad, K)
    expect = F.e2m1_decode(ref["e2m1"]) * np.repeat(F.e4m3_decode(ref["scales"]), 16, axis=1)
    assert np.array_equal(a[:M], expect)
    assert np.all(a[M:] == 0)
