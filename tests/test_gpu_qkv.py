"""The fused QKV projection with per-head Q/K RMSNorm and rotary embedding in the GEMM
epilogue (svdq_w4a4_linear_qkv_norm_rope) against the oracle: on an oracle-prepared
layer with ragged token counts, and on the DiT block's 3072 -> 9216 projection at
M = 4608 with the 1024x1024 rotary table (sampled rows, text and image tokens)."""

import dataclasses

import numpy as np
import pytest
import torch

import w4a4_rank_corrected_linear_amd as svdq
from helpers import check_y, dev_bf16, dev_u8, host_bits
from oracle import attention as AT
from oracle import formats as F
from oracle import linear as OL
from oracle import prep as P
from synth import inputs as I

pytestmark = pytest.mark.gpu

EPS = I.QK_NORM_EPS


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _layer_dev(layer, bias=True):
    return svdq.SvdqLinear.from_interchange(
        dev_u8(layer.qweight), dev_bf16(layer.wscales), dev_bf16(layer.smooth),
        dev_bf16(layer.lora_down) if layer.rank else None,
        dev_bf16(layer.lora_up) if layer.rank else None,
        dev_bf16(layer.bias) if bias else None)


@pytest.fixture(scope="module")
def tiny_qkv():
    """K = 512, N = 768: two heads each of Q, K and V; random angles per token."""
    li = I.layer_inputs(config_id=1, M=300, K=512, N=768, outlier_count=4, factor=20.0)
    layer = P.prepare_svdq(li.w, li.x_cal, li.bias, rank=32)
    rng = np.random.default_rng(31)
    ang = rng.uniform(-np.pi, np.pi, (300, 64))
    rope = np.stack([np.cos(ang), np.sin(ang)], axis=2).astype(np.float32)
    nq, nk = I.qk_norm_weights()
    return li, layer, rope, nq, nk


@pytest.mark.parametrize("bias", [True, False])
@pytest.mark.parametrize("M", [1, 37, 256, 300])
def test_qkv_norm_rope_tiny(tiny_qkv, M, bias):
    li, layer, rope, nq, nk = tiny_qkv
    dev = _layer_dev(layer, bias)
    y = dev.qkv_norm_rope(dev_bf16(li.x[:M]), dev_bf16(nq), dev_bf16(nk), EPS, dev_f32(rope[:M]))
    torch.cuda.synchronize()
    ol = layer if bias else dataclasses.replace(layer, bias=None)
    r = OL.w4a4_linear("int4", li.x[:M], ol)["r"]
    check_y(host_bits(y), AT.qkv_norm_rope_f64(r, nq, nk, EPS, rope[:M]))


def test_qkv_v_columns_equal_the_plain_linear(tiny_qkv):
    """V is the plain linear, bit for bit; Q and K are not."""
    li, layer, rope, nq, nk = tiny_qkv
    dev = _layer_dev(layer)
    x = dev_bf16(li.x)
    plain = host_bits(dev(x))
    fused = host_bits(dev.qkv_norm_rope(x, dev_bf16(nq), dev_bf16(nk), EPS, dev_f32(rope)))
    assert np.array_equal(fused[:, 512:], plain[:, 512:])
    assert not np.array_equal(fused[:, :256], plain[:, :256])
    assert not np.array_equal(fused[:, 256:512], plain[:, 256:512])


def test_qkv_norm_rope_zero_rows_and_m0(tiny_qkv):
    """Zero activations give r = bias: heads of the bias alone are normalised; M = 0
    launches nothing."""
    li, layer, rope, nq, nk = tiny_qkv
    dev = _layer_dev(layer)
    x = np.zeros((5, 512), np.uint16)
    y = dev.qkv_norm_rope(dev_bf16(x), dev_bf16(nq), dev_bf16(nk), EPS, dev_f32(rope[:5]))
    r = OL.w4a4_linear("int4", x, layer)["r"]
    check_y(host_bits(y), AT.qkv_norm_rope_f64(r, nq, nk, EPS, rope[:5]))
    e = torch.empty((0, 512), dtype=torch.bfloat16, device="cuda")
    out = dev.qkv_norm_rope(e, dev_bf16(nq), dev_bf16(nk), EPS,
                            torch.empty((0, 64, 2), dtype=torch.float32, device="cuda"))
    assert out.shape == (0, 768)


@pytest.mark.parametrize("K,N,rank", [(4608, 1152, 32), (640, 1152, 16), (1024, 768, 0)])
def test_qkv_norm_rope_shapes(K, N, rank):
    """Tiles of three heads that are all Q, all K or all V (N = 1152), or mixed
    (N = 768); the low-rank term before the main loop (three k-splits at K = 4608, where
    the few tiles are also split along K and finished per head by the tail kernel) or
    after it, and ranks 32, 16 and 0."""
    li = I.layer_inputs(config_id=1, M=77, K=K, N=N, outlier_count=4, factor=20.0)
    layer = P.prepare_svdq(li.w, li.x_cal, li.bias, rank=rank)
    rng = np.random.default_rng(K + N + rank)
    ang = rng.uniform(-np.pi, np.pi, (77, 64))
    rope = np.stack([np.cos(ang), np.sin(ang)], axis=2).astype(np.float32)
    nq, nk = I.qk_norm_weights()
    dev = _layer_dev(layer)
    y = dev.qkv_norm_rope(dev_bf16(li.x), dev_bf16(nq), dev_bf16(nk), EPS, dev_f32(rope))
    r = OL.w4a4_linear("int4", li.x, layer)["r"]
    check_y(host_bits(y), AT.qkv_norm_rope_f64(r, nq, nk, EPS, rope))


def test_qkv_norm_rope_dit_block_full_size():
    """The block's QKV projection at M = 4608 (512 text + 4096 image tokens) with the
    1024x1024 rotary table, sampled rows of both kinds against the oracle."""
    pb = I.chain_layer_bytes()["qkv"]
    layer = P.SvdqLayer(precision="int4", K=pb.K, N=pb.N, rank=pb.rank, qweight=pb.qweight,
                        wscales=pb.wscales, w_global=1.0, act_global=1.0, smooth=pb.smooth,
                        lora_down=pb.lora_down, lora_up=pb.lora_up, bias=pb.bias)
    dev = svdq.SvdqLinear.from_interchange(dev_u8(pb.qweight), dev_bf16(pb.wscales),
                                           dev_bf16(pb.smooth), dev_bf16(pb.lora_down),
                                           dev_bf16(pb.lora_up), dev_bf16(pb.bias))
    M = 4608
    x = I.chain_step_activations(M, 0)
    rope = I.rope_table(M)
    nq, nk = I.qk_norm_weights()
    y = host_bits(dev.qkv_norm_rope(dev_bf16(x), dev_bf16(nq), dev_bf16(nk), EPS, dev_f32(rope)))
    rows = np.array([0, 1, 300, 511, 512, 513, 1000, 2222, 4000, 4606, 4607])
    r = OL.w4a4_linear_rows("int4", x, layer, rows)["r"]
    check_y(y[rows], AT.qkv_norm_rope_f64(r, nq, nk, EPS, rope[rows]))


@pytest.mark.parametrize("M,N", [(1, 384), (37, 768), (4608, 9216)])
def test_separate_qk_norm_rope_pass(M, N):
    """svdq_qk_norm_rope_bf16 on a bf16 QKV output: the oracle's norm + rotation of the
    bf16 values, once rounded; V copied out of place and untouched in place."""
    rng = np.random.default_rng(M + N)
    x = I.to_bf16_bits((rng.standard_normal((M, N)) * 3.0).astype(np.float32))
    if M > 1:
        x[M // 2, : 2 * N // 3] = 0          # an all-zero row of Q and K heads
    rope = I.rope_table(M) if N == 9216 else np.stack(
        [np.cos(a := rng.uniform(-4, 4, (M, 64))), np.sin(a)], axis=2).astype(np.float32)
    nq, nk = I.qk_norm_weights()
    xd = dev_bf16(x)
    y = host_bits(svdq.qk_norm_rope(xd, dev_bf16(nq), dev_bf16(nk), EPS, dev_f32(rope)))
    ref = AT.qkv_norm_rope_f64(F.bf16_to_f64(x), nq, nk, EPS, rope)
    check_y(y, ref)
    assert np.array_equal(y[:, 2 * N // 3:], x[:, 2 * N // 3:])
    svdq.qk_norm_rope(xd, dev_bf16(nq), dev_bf16(nk), EPS, dev_f32(rope), out=xd)
    assert np.array_equal(host_bits(xd), y)


@pytest.fixture(scope="module")
def tiny_qkv_nvfp4():
    li = I.layer_inputs(config_id=1, M=300, K=512, N=768, outlier_count=4, factor=20.0)
    layer = P.prepare_svdq(li.w, li.x_cal, li.bias, rank=32, precision="nvfp4")
    rng = np.random.default_rng(41)
    ang = rng.uniform(-np.pi, np.pi, (300, 64))
    rope = np.stack([np.cos(ang), np.sin(ang)], axis=2).astype(np.float32)
    return li, layer, rope


@pytest.mark.parametrize("M", [1, 129, 300])
def test_qkv_norm_rope_nvfp4(tiny_qkv_nvfp4, M):
    """The NVFP4 GEMM's fused QKV epilogue against the oracle; V equals the plain
    NVFP4 linear bit for bit."""
    li, layer, rope = tiny_qkv_nvfp4
    nq, nk = I.qk_norm_weights()
    dev = svdq.SvdqLinear.from_interchange(
        dev_u8(layer.qweight), dev_u8(layer.wscales), dev_bf16(layer.smooth),
        dev_bf16(layer.lora_down), dev_bf16(layer.lora_up), dev_bf16(layer.bias),
        precision="nvfp4", w_global=layer.w_global, act_global=layer.act_global)
    x = dev_bf16(li.x[:M])
    y = host_bits(dev.qkv_norm_rope(x, dev_bf16(nq), dev_bf16(nk), EPS, dev_f32(rope[:M])))
    r = OL.w4a4_linear("nvfp4", li.x[:M], layer)["r"]
    check_y(y, AT.qkv_norm_rope_f64(r, nq, nk, EPS, rope[:M]))
    assert np.array_equal(y[:, 512:], host_bits(dev(x))[:, 512:])


def test_qkv_norm_rope_nvfp4_dit_block_full_size():
    """The NVFP4 GEMM's fused QKV epilogue at the block's shape (M = 4608, 3072 -> 9216,
    1296 tiles of one head over several rounds) with the 1024x1024 rotary table:
    sampled rows of text and image tokens against the oracle, and the V columns equal
    to the plain NVFP4 linear bit for bit."""
    pb = I.prepared_nvfp4_bytes(3, 3072, 9216, 32)
    layer = P.SvdqLayer(precision="nvfp4", K=pb.K, N=pb.N, rank=pb.rank, qweight=pb.qweight,
                        wscales=pb.wscales, w_global=pb.w_global, act_global=pb.act_global,
                        smooth=pb.smooth, lora_down=pb.lora_down, lora_up=pb.lora_up, bias=pb.bias)
    dev = svdq.SvdqLinear.from_interchange(
        dev_u8(pb.qweight), dev_u8(pb.wscales), dev_bf16(pb.smooth), dev_bf16(pb.lora_down),
        dev_bf16(pb.lora_up), dev_bf16(pb.bias), precision="nvfp4", w_global=pb.w_global,
        act_global=pb.act_global)
    M = 4608
    x = I.chain_step_activations(M, 0)
    rope = I.rope_table(M)
    nq, nk = I.qk_norm_weights()
    xd = dev_bf16(x)
    y = host_bits(dev.qkv_norm_rope(xd, dev_bf16(nq), dev_bf16(nk), EPS, dev_f32(rope)))
    rows = np.array([0, 1, 511, 512, 1000, 2222, 4000, 4607])
    r = OL.w4a4_linear_rows("nvfp4", x, layer, rows)["r"]
    check_y(y[rows], AT.qkv_norm_rope_f64(r, nq, nk, EPS, rope[rows]))
    assert np.array_equal(y[:, 6144:], host_bits(dev(xd))[:, 6144:])
