"""GPU parity of the nvfp4 path against the oracle: svdq_quantize_act (E2M1 codes and
E4M3 scales bit-exact, U within the fp32 bound), svdq_pack_weight, and
svdq_w4a4_linear (Y within the stated tolerance; bit-exact on grid-exact inputs)."""

import numpy as np
import pytest
import torch

import w4a4_rank_corrected_linear_amd as svdq
from helpers import check_u, check_y, dev_bf16, dev_u8, host_bits
from oracle import activation as A
from oracle import formats as F
from oracle import linear as OL
from oracle import prep as P
from oracle import quant as Q
from synth import inputs as I

pytestmark = pytest.mark.gpu

ONE = int(F.bf16_rne(np.float32(1.0)))


def _layer_dev(layer, bias=True, w_global=None, act_global=None):
    return svdq.SvdqLinear.from_interchange(
        dev_u8(layer.qweight), dev_u8(layer.wscales), dev_bf16(layer.smooth),
        dev_bf16(layer.lora_down) if layer.rank else None,
        dev_bf16(layer.lora_up) if layer.rank else None,
        dev_bf16(layer.bias) if (bias and layer.bias is not None) else None,
        precision="nvfp4",
        w_global=layer.w_global if w_global is None else w_global,
        act_global=layer.act_global if act_global is None else act_global)


@pytest.fixture(scope="module")
def tiny():
    li = I.layer_inputs(**I.TINY)
    return li, P.prepare_svdq(li.w, li.x_cal, li.bias, rank=32, precision="nvfp4")


def _quantize(x, smooth, ld, g):
    return svdq.quantize_act(dev_bf16(x), dev_bf16(smooth), None if ld is None else dev_bf16(ld),
                             precision="nvfp4", act_global=g)


@pytest.mark.parametrize("M", [1, 17, 256])
def test_quantize_act_nvfp4_bitexact(tiny, M):
    li, layer = tiny
    x = li.x[:M]
    ref = Q.quantize_act_nvfp4(x, layer.smooth, layer.act_global, layer.lora_down)
    codes, scales, u = _quantize(x, layer.smooth, layer.lora_down, layer.act_global)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(codes), ref["codes"])
    assert np.array_equal(host_bits(scales), ref["scales"])
    check_u(host_bits(u), ref, layer.lora_down)


def test_quantize_act_nvfp4_ties_zero_and_negative_zero():
    """g = fl32(1/6) makes fl32(6 g) = 1 and, for blocks whose amax is 6 s, the
    divisor fl32(s g) = s: the quotients are the planted values, which include every
    E2M1 midpoint (ties go to the even code), zeros and negative zeros."""
    g = float(np.float32(1.0 / 6.0))
    assert np.float32(6.0) * np.float32(g) == np.float32(1.0)
    vals = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, -0.25, -0.75, -1.25, -1.75,
                     -2.5, -3.5, -5.0, 0.0], np.float64)
    M, K = 8, 128
    rows = []
    for m in range(M):
        s = 2.0 ** (m - 3)
        row = np.tile(vals, K // 16) * s
        rows.append(row)
    x = F.bf16_rne(np.array(rows, np.float32))
    x[1::2, 15::16] = 0x8000                   # negative zeros inside non-zero blocks
    x[2, 16:32] = 0x8000                       # a block of negative zeros
    x[3, 32:48] = 0                            # a zero block
    x[4, 48:64] = F.bf16_rne(np.float32(1e-30))
    one = np.full(K, ONE, np.uint16)
    ref = Q.quantize_act_nvfp4(x, one, g, None)
    codes, scales, _ = _quantize(x, one, None, g)
    assert np.array_equal(host_bits(codes), ref["codes"])
    assert np.array_equal(host_bits(scales), ref["scales"])


def test_quantize_act_nvfp4_scale_saturation_and_subnormal_scales():
    rng = np.random.default_rng(91)
    M, K = 16, 256
    x = F.bf16_rne((rng.standard_normal((M, K)) * np.exp(rng.uniform(-12, 12, (M, 1)))).astype(np.float32))
    one = np.full(K, ONE, np.uint16)
    seen = np.zeros(0, np.uint8)
    for g in [1e-6, 1e-3, 1.0, 50.0]:
        g = float(np.float32(g))
        ref = Q.quantize_act_nvfp4(x, one, g, None)
        codes, scales, _ = _quantize(x, one, None, g)
        assert np.array_equal(host_bits(codes), ref["codes"]), g
        assert np.array_equal(host_bits(scales), ref["scales"]), g
        seen = np.concatenate([seen, ref["scales"].ravel()])
    assert np.any(seen == 0x7E), "no saturated block scale exercised"
    assert np.any((seen > 0) & (seen < 8)), "no subnormal block scale exercised"


def test_pack_weight_nvfp4_layout(tiny):
    """The packed weights are the interchange codes in FP4 lane slots and the E4M3 scales
    as their exact fp16 values (4.5 bits per weight)."""
    from helpers import decode_fp4_operand
    _, layer = tiny
    pc, ps = svdq.pack_weight(dev_u8(layer.qweight), dev_u8(layer.wscales), precision="nvfp4")
    assert pc.numel() == layer.N * layer.K // 2
    buf = np.concatenate([host_bits(pc), host_bits(ps)])
    codes, scales = decode_fp4_operand(buf, layer.N, layer.K, dword_major=True)
    assert np.array_equal(codes, F.unpack_nibbles(layer.qweight))
    assert np.array_equal(scales, F.e4m3_decode(layer.wscales))


def test_pack_weight_nvfp4_rejects_nan_scale(tiny):
    _, layer = tiny
    bad = layer.wscales.copy()
    bad[3, 5] = 0x7F
    with pytest.raises(svdq.SvdqError) as ei:
        svdq.pack_weight(dev_u8(layer.qweight), dev_u8(bad), precision="nvfp4")
    assert ei.value.status == 8


def test_nonpositive_global_scale_is_rejected(tiny):
    li, layer = tiny
    with pytest.raises(svdq.SvdqError) as ei:
        _quantize(li.x[:4], layer.smooth, layer.lora_down, 0.0)
    assert ei.value.status == 8


@pytest.mark.parametrize("M", [256, 1, 17, 129])
def test_linear_nvfp4_tiny(tiny, M):
    li, layer = tiny
    y = _layer_dev(layer)(dev_bf16(li.x[:M]))
    check_y(host_bits(y), OL.w4a4_linear("nvfp4", li.x[:M], layer)["r"])


def test_linear_nvfp4_gelu_epilogue(tiny):
    li, layer = tiny
    y = _layer_dev(layer)(dev_bf16(li.x), gelu=True)
    check_y(host_bits(y), A.gelu_f64(OL.w4a4_linear("nvfp4", li.x, layer)["r"]))


def test_linear_nvfp4_rank0_no_bias_and_rank16():
    li = I.layer_inputs(config_id=9, M=96, K=1024, N=384, outlier_count=8, factor=20.0)
    for rank, bias in [(0, None), (16, li.bias)]:
        layer = P.prepare_svdq(li.w, li.x_cal, bias, rank=rank, precision="nvfp4")
        y = _layer_dev(layer)(dev_bf16(li.x))
        check_y(host_bits(y), OL.w4a4_linear("nvfp4", li.x, layer)["r"])


def test_linear_nvfp4_grid_exact_is_bit_exact():
    """Rank 0, no bias; X and W on the NVFP4 grid with block scales 1 or 2 and one 6
    per block (so each block scale is recovered exactly); power-of-two global scales.
    Every product and partial sum is exact in fp32, so Y equals bf16(r) bit for bit."""
    rng = np.random.default_rng(92)
    M, K, N = 64, 512, 256
    cx = rng.integers(0, 16, size=(M, K))
    cw = rng.integers(0, 16, size=(N, K))
    cx[:, ::16] = 7
    cw[:, ::16] = 7
    sx = rng.choice([0x38, 0x40], size=(M, K // 16))
    sw = rng.choice([0x38, 0x40], size=(N, K // 16)).astype(np.uint8)
    x = F.bf16_rne((F.e2m1_decode(cx) * np.repeat(F.e4m3_decode(sx), 16, axis=1)).astype(np.float32))
    layer = P.SvdqLayer(precision="nvfp4", K=K, N=N, rank=0,
                        qweight=F.pack_nibbles(cw.astype(np.uint8)), wscales=sw, w_global=0.5,
                        act_global=1.0,
                        smooth=np.full(K, ONE, np.uint16), lora_down=np.zeros((0, K), np.uint16),
                        lora_up=np.zeros((N, 0), np.uint16), bias=None)
    g = 1.0
    ref = OL.w4a4_linear("nvfp4", x, layer, act_global=g)
    y = _layer_dev(layer, act_global=g)(dev_bf16(x))
    assert np.array_equal(host_bits(y), ref["y"])


def test_workspace_holds_codes_and_scales(tiny):
    """The layer's quantizer leaves the E2M1 codes and the block scales (fp16) of the
    activations in the workspace, bit for bit the oracle's, zeros in the padding rows."""
    li, layer = tiny
    M = 200
    dl = _layer_dev(layer)
    # the workspace as sized, followed by a guard region the call must leave alone
    need = dl.workspace_bytes(M)
    buf = torch.full((need + (1 << 20),), 0xA5, dtype=torch.uint8, device="cuda")
    ws = buf[:need]
    dl(dev_bf16(li.x[:M]), workspace=ws)
    torch.cuda.synchronize()
    assert bool((buf[need:] == 0xA5).all()), "the NVFP4 linear wrote past its workspace"
    ref = Q.quantize_act_nvfp4(li.x[:M], layer.smooth, layer.act_global, layer.lora_down)
    from helpers import decode_fp4_operand
    codes, scales = decode_fp4_operand(host_bits(ws), 256, layer.K)
    assert np.array_equal(codes[:M], ref["e2m1"])
    assert np.array_equal(scales[:M], F.e4m3_decode(ref["scales"]))
    assert np.all(codes[M:] == 0) and np.all(scales[M:] == 0)


@pytest.fixture(scope="module")
def nvfp4_square():
    cfg = dict(I.NVFP4_SQ)
    li = I.layer_inputs(**cfg)
    return li, P.prepare_svdq(li.w, li.x_cal, li.bias, rank=32, precision="nvfp4")


def test_linear_nvfp4_full_size_square(nvfp4_square):
    """M = 4096, K = N = 3072: sampled rows against the oracle."""
    li, layer = nvfp4_square
    y = host_bits(_layer_dev(layer)(dev_bf16(li.x)))
    rows = np.unique(np.concatenate([np.arange(5, 4096, 89), [0, 4095]]))
    ref = OL.w4a4_linear_rows("nvfp4", li.x, layer, rows)
    check_y(y[rows], ref["r"])


def test_linear_nvfp4_full_size_mlp_up_synthetic():
    """M = 4096, K = 3072 -> N = 12288 on seeded prepared-layout bytes: sampled rows."""
    pb = I.prepared_nvfp4_bytes(4, 3072, 12288, 32)
    sd = I.seeds(4)
    x = I.activations(4096, 3072, sd.x, I.outlier_channels(3072, 31, sd.outliers), 30.0)
    layer = P.SvdqLayer(precision="nvfp4", K=3072, N=12288, rank=32, qweight=pb.qweight,
                        wscales=pb.wscales, w_global=pb.w_global, act_global=pb.act_global,
                        smooth=pb.smooth, lora_down=pb.lora_down, lora_up=pb.lora_up,
                        bias=pb.bias)
    y = host_bits(_layer_dev(layer)(dev_bf16(x)))
    rows = np.unique(np.concatenate([np.arange(7, 4096, 211), [4095]]))
    check_y(y[rows], OL.w4a4_linear_rows("nvfp4", x, layer, rows)["r"])


def test_quantizers_non_dyadic_tensor_scale_golden():
    """The hand-worked block with g = fl32(1/3) (tests/golden/nvfp4_tie_third.txt),
    whose quotients sit on E2M1 midpoints only when the divisor is fl32(s g): through
    svdq_quantize_act and through the layer's own quantizer (workspace values)."""
    from golden_cases import nvfp4_tie_third
    from helpers import nvfp4_workspace_values
    xb, g, c, s = nvfp4_tie_third()
    M, K, N = 40, 256, 128
    rng = np.random.default_rng(93)
    x = np.zeros((M, K), np.uint16)
    for m in range(M):                      # the block, permuted, in every block slot
        for b in range(K // 16):
            x[m, 16 * b:16 * b + 16] = xb[0, rng.permutation(16)] if (m + b) % 3 else xb[0]
    one = np.full(K, ONE, np.uint16)
    ref = Q.quantize_act_nvfp4(x, one, float(g), None)
    assert np.all(ref["scales"] == s[0, 0])
    first = ref["e2m1"][0, :16]
    assert np.array_equal(first, c[0])
    codes, scales, _ = _quantize(x, one, None, float(g))
    assert np.array_equal(host_bits(codes), ref["codes"])
    assert np.array_equal(host_bits(scales), ref["scales"])
    layer = P.SvdqLayer(precision="nvfp4", K=K, N=N, rank=0,
                        qweight=F.pack_nibbles(rng.integers(0, 16, size=(N, K)).astype(np.uint8)),
                        wscales=np.full((N, K // 16), 0x38, np.uint8), w_global=1.0,
                        act_global=float(g), smooth=one, lora_down=np.zeros((0, K), np.uint16),
                        lora_up=np.zeros((N, 0), np.uint16), bias=None)
    dl = _layer_dev(layer)
    need = dl.workspace_bytes(M)
    buf = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    dl(dev_bf16(x), workspace=buf)
    torch.cuda.synchronize()
    a = nvfp4_workspace_values(host_bits(buf), 256, K)
    expect = F.e2m1_decode(ref["e2m1"]) * np.repeat(F.e4m3_decode(ref["scales"]), 16, axis=1)
    assert np.array_equal(a[:M], expect)
    assert np.all(a[M:] == 0)
