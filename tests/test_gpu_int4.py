"""GPU parity of the int4 path against the oracle: svdq_quantize_act (codes and
scales bit-exact, U within 1 bf16 step), svdq_pack_weight, and svdq_w4a4_linear
(Y within the stated tolerance; bit-exact on grid-exact inputs)."""

import numpy as np
import pytest
import torch

import w4a4_rank_corrected_linear_amd as svdq
from helpers import (check_u, check_y, decode_fp6_operand, dev_bf16, pair_scale_records, scale_records,
                     u_partials,
                     dev_u8, host_bits, int4_interchange)
from oracle import activation as A
from oracle import formats as F
from oracle import linear as OL
from oracle import prep as P
from oracle import quant as Q
from synth import inputs as I

pytestmark = pytest.mark.gpu


def _layer_dev(layer, bias=True):
    return svdq.SvdqLinear.from_interchange(
        dev_u8(layer.qweight), dev_bf16(layer.wscales), dev_bf16(layer.smooth),
        dev_bf16(layer.lora_down) if layer.rank else None,
        dev_bf16(layer.lora_up) if layer.rank else None,
        dev_bf16(layer.bias) if (bias and layer.bias is not None) else None)


@pytest.fixture(scope="module")
def tiny():
    li = I.layer_inputs(**I.TINY)
    return li, P.prepare_svdq(li.w, li.x_cal, li.bias, rank=32)


@pytest.mark.parametrize("M", [1, 17, 255, 256])
def test_quantize_act_int4_bitexact(tiny, M):
    li, layer = tiny
    x = li.x[:M]
    ref = Q.quantize_act_int4(x, layer.smooth, layer.lora_down)
    codes, scales, u = svdq.quantize_act(dev_bf16(x), dev_bf16(layer.smooth), dev_bf16(layer.lora_down))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(codes), ref["codes"])
    assert np.array_equal(host_bits(scales), ref["scales"])
    check_u(host_bits(u), ref, layer.lora_down)


def test_quantize_act_int4_wide_k_rank16_and_outliers():
    rng = np.random.default_rng(77)
    M, K = 40, 3072
    idx = I.outlier_channels(K, 31, 5)
    x = I.activations(M, K, 99, idx, 30.0)
    m = F.bf16_rne(rng.uniform(0.05, 1.5, K).astype(np.float32))
    ld = F.bf16_rne((rng.standard_normal((16, K)) * 0.05).astype(np.float32))
    ref = Q.quantize_act_int4(x, m, ld)
    codes, scales, u = svdq.quantize_act(dev_bf16(x), dev_bf16(m), dev_bf16(ld))
    assert np.array_equal(host_bits(codes), ref["codes"])
    assert np.array_equal(host_bits(scales), ref["scales"])
    check_u(host_bits(u), ref, ld)


def test_quantize_act_ties_and_zero_groups():
    """Exact half-way quotients round to even; all-zero groups give zero scale."""
    rng = np.random.default_rng(78)
    M, K = 32, 256
    k = rng.integers(-7, 8, size=(M, K)).astype(np.float64)
    k += np.where(rng.random((M, K)) < 0.3, 0.5, 0.0)           # plant ties
    k = np.clip(k, -6.5, 6.5)
    k[:, ::64] = 7.0
    s = 2.0 ** rng.integers(-8, 4, size=(M, K // 64))
    x = k * np.repeat(s, 64, axis=1)
    x[3, 64:128] = 0.0
    xb = F.bf16_rne(x.astype(np.float32))
    assert np.array_equal(F.bf16_to_f64(xb), x)
    one = F.bf16_rne(np.ones(K, np.float32))
    ref = Q.quantize_act_int4(xb, one, None)
    codes, scales, _ = svdq.quantize_act(dev_bf16(xb), dev_bf16(one), None)
    assert np.array_equal(host_bits(codes), ref["codes"])
    assert np.array_equal(host_bits(scales), ref["scales"])


def test_pack_weight_layout(tiny):
    _, layer = tiny
    pc, ps = svdq.pack_weight(dev_u8(layer.qweight), dev_bf16(layer.wscales))
    q = decode_fp6_operand(host_bits(pc), layer.N, layer.K)
    assert np.array_equal(q, F.int4_decode(F.unpack_nibbles(layer.qweight)))
    G = layer.K // 64
    st = pair_scale_records(host_bits(ps), G, layer.N)
    assert np.array_equal(st, layer.wscales.T)


def test_pack_weight_holds_minus_eight(tiny):
    """Every int4 code, -8 included, packs to the E2M3 operand value q/8."""
    _, layer = tiny
    rng = np.random.default_rng(83)
    q = rng.integers(-8, 8, size=(layer.N, layer.K))
    q[:, ::7] = -8
    pc, _ = svdq.pack_weight(dev_u8(int4_interchange(q)), dev_bf16(layer.wscales))
    assert np.array_equal(decode_fp6_operand(host_bits(pc), layer.N, layer.K), q)


def _subnormal_golden_rows(M):
    from golden_cases import int4_subnormal_scales
    x, q, s = int4_subnormal_scales()
    K = 512
    assert x.shape[1] <= K
    xb = np.zeros((M, K), np.uint16)
    qq = np.zeros((M, K), np.int64)
    for m in range(M):          # the golden groups, rotated by a group per row
        sh = 64 * (m % 8)
        xb[m, :x.shape[1]] = x[0]
        qq[m, :x.shape[1]] = q[0]
        xb[m] = np.roll(xb[m], sh)
        qq[m] = np.roll(qq[m], sh)
    return xb, qq, s


def test_quantize_act_subnormal_scales_golden():
    """The hand-worked groups with subnormal bf16 scales (their exact-division branch
    and the clamp to [-8, 7]) through svdq_quantize_act: codes and scales equal the
    golden values and the oracle's."""
    from golden_cases import int4_subnormal_scales
    xb, qq, s = _subnormal_golden_rows(24)
    one = F.bf16_rne(np.ones(xb.shape[1], np.float32))
    ref = Q.quantize_act_int4(xb, one, None)
    assert np.array_equal(ref["q"], qq)
    codes, scales, _ = svdq.quantize_act(dev_bf16(xb), dev_bf16(one), None)
    torch.cuda.synchronize()
    assert np.array_equal(F.int4_decode(F.unpack_nibbles(host_bits(codes))), qq)
    assert np.array_equal(host_bits(scales), ref["scales"])
    assert np.array_equal(host_bits(scales)[0, :s.shape[1]], s[0])


def test_fused_quantizer_subnormal_scales_golden():
    """The same groups through the layer's own quantizer (the GEMM operand layout in
    the workspace): -8 codes become the E2M3 value -1.0."""
    xb, qq, _ = _subnormal_golden_rows(40)
    K, N = xb.shape[1], 128
    rng = np.random.default_rng(84)
    one = F.bf16_rne(np.ones(K, np.float32))
    layer = P.SvdqLayer(precision="int4", K=K, N=N, rank=0,
                        qweight=int4_interchange(rng.integers(-8, 8, size=(N, K))),
                        wscales=F.bf16_rne(np.full((N, K // 64), 0.01, np.float32)), w_global=1.0,
                        act_global=1.0, smooth=one, lora_down=np.zeros((0, K), np.uint16),
                        lora_up=np.zeros((N, 0), np.uint16), bias=None)
    dl = _layer_dev(layer)
    need = dl.workspace_bytes(40)
    buf = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    dl(dev_bf16(xb), workspace=buf)
    torch.cuda.synchronize()
    w = host_bits(buf)
    q = decode_fp6_operand(w, 256, K)
    assert np.array_equal(q[:40], qq)
    assert np.all(q[40:] == 0)
    ref = Q.quantize_act_int4(xb, one, None)
    s = scale_records(w[256 * K * 3 // 4:], K // 64, 256)
    assert np.array_equal(s[:, :40], ref["scales"].T)
    assert np.all(s[:, 40:] == 0)


@pytest.mark.parametrize("M", [256, 1, 17, 129, 255])
def test_linear_tiny(tiny, M):
    li, layer = tiny
    dl = _layer_dev(layer)
    y = dl(dev_bf16(li.x[:M]))
    ref = OL.w4a4_linear("int4", li.x[:M], layer)
    check_y(host_bits(y), ref["r"])


@pytest.mark.parametrize("M", [256, 37])
def test_linear_gelu_epilogue(tiny, M):
    """svdq_w4a4_linear_gelu: the exact GELU of the unrounded result, rounded once,
    against the oracle's gelu(r) (128-wide tiles here; the chain test covers 192)."""
    li, layer = tiny
    y = _layer_dev(layer)(dev_bf16(li.x[:M]), gelu=True)
    check_y(host_bits(y), A.gelu_f64(OL.w4a4_linear("int4", li.x[:M], layer)["r"]))


def test_linear_rank0_no_bias_and_rank16():
    li = I.layer_inputs(config_id=9, M=96, K=1024, N=384, outlier_count=8, factor=20.0)
    for rank, bias in [(0, None), (16, li.bias)]:
        layer = P.prepare_svdq(li.w, li.x_cal, bias, rank=rank)
        y = _layer_dev(layer)(dev_bf16(li.x))
        check_y(host_bits(y), OL.w4a4_linear("int4", li.x, layer)["r"])


def test_linear_grid_exact_is_bit_exact():
    """Rank 0, no bias, X and W on the int4 grid with power-of-two scales in a narrow
    range: every fp32 step on the GPU is exact, so Y equals bf16(r) bit for bit."""
    rng = np.random.default_rng(79)
    M, K, N = 200, 512, 256
    kx = rng.integers(-7, 8, size=(M, K))
    kx[:, ::64] = 7
    sx = 2.0 ** rng.integers(-3, 0, size=(M, K // 64))
    x = F.bf16_rne((kx * np.repeat(sx, 64, axis=1)).astype(np.float32))
    kw = rng.integers(-8, 8, size=(N, K))       # the whole int4 range, -8 included
    kw[:, 1::9] = -8
    sw = 2.0 ** rng.integers(-7, -5, size=(N, K // 64))
    one = F.bf16_rne(np.ones(K, np.float32))
    layer = P.SvdqLayer(precision="int4", K=K, N=N, rank=0, qweight=int4_interchange(kw),
                        wscales=F.bf16_rne(sw.astype(np.float32)), w_global=1.0, act_global=1.0,
                        smooth=one, lora_down=np.zeros((0, K), np.uint16),
                        lora_up=np.zeros((N, 0), np.uint16), bias=None)
    ref = OL.w4a4_linear("int4", x, layer)
    y = _layer_dev(layer)(dev_bf16(x))
    assert np.array_equal(host_bits(y), ref["y"])


def test_workspace_matches_standalone_quantize(tiny):
    """The fused call's quantized activations equal svdq_quantize_act's outputs."""
    li, layer = tiny
    M = 200
    dl = _layer_dev(layer)
    # the workspace as sized, filled with a non-zero pattern (so the zero codes, scales
    # and U of the padding rows must come from the kernel), then a guard region
    need = dl.workspace_bytes(M)
    buf = torch.full((need + (1 << 20),), 0xA5, dtype=torch.uint8, device="cuda")
    ws = buf[:need]
    dl(dev_bf16(li.x[:M]), workspace=ws)
    torch.cuda.synchronize()
    assert bool((buf[need:] == 0xA5).all()), "the linear wrote past its workspace"
    ref = Q.quantize_act_int4(li.x[:M], layer.smooth, layer.lora_down)
    w = host_bits(ws)
    M_pad, K, G = 256, layer.K, layer.K // 64
    q = decode_fp6_operand(w, M_pad, K)
    assert np.array_equal(q[:M], ref["q"])
    assert np.all(q[M:] == 0)
    off_s = M_pad * K * 3 // 4
    s = scale_records(w[off_s:], G, M_pad)
    assert np.array_equal(s[:, :M], ref["scales"].T)
    off_u = off_s + G * M_pad * 8
    u = u_partials(w[off_u:], 1, M_pad, 32)[0]
    check_u(u[:M], ref, layer.lora_down)
    assert np.all(u[M:] == 0)


def test_linear_deterministic_and_writes_every_output(tiny):
    li, layer = tiny
    dl = _layer_dev(layer)
    M = 255
    x = dev_bf16(li.x[:M])
    guard = torch.full((M + 8, layer.N), -1, dtype=torch.int16, device="cuda")
    y1 = guard[:M].view(torch.bfloat16)
    dl(x, out=y1)
    g = host_bits(guard.view(torch.bfloat16))
    assert not np.any(g[:M] == 0xFFFF), "an output element was not written"
    assert np.all(g[M:] == 0xFFFF), "write past the end of Y"
    y2 = dl(x)
    assert np.array_equal(host_bits(y2), g[:M])


@pytest.fixture(scope="module")
def attn_proj():
    cfg = dict(I.ATTN_PROJ)
    li = I.layer_inputs(**cfg)
    return li, P.prepare_svdq(li.w, li.x_cal, li.bias, rank=32)


def test_linear_attention_projection_full_size(attn_proj):
    """M = 4096, K = N = 3072 in the benchmarked launch; the oracle checks a sample
    of rows (rows are independent)."""
    li, layer = attn_proj
    dl = _layer_dev(layer)
    y = host_bits(dl(dev_bf16(li.x)))
    rows = np.unique(np.concatenate([np.arange(0, 4096, 61), [4094, 4095]]))
    ref = OL.w4a4_linear_rows("int4", li.x, layer, rows)
    check_y(y[rows], ref["r"])
    codes, scales, u = svdq.quantize_act(dev_bf16(li.x[rows]), dev_bf16(layer.smooth),
                                         dev_bf16(layer.lora_down))
    assert np.array_equal(host_bits(codes), ref["act"]["codes"])
    assert np.array_equal(host_bits(scales), ref["act"]["scales"])


def test_throughput_workload_sampled_rows():
    """The seeded prepared-layout layer and activations that the throughput run times
    (M = 4096, K = N = 3072, rank 32), in the same launch: sampled rows against the
    oracle."""
    pb = I.prepared_int4_bytes(2, 3072, 3072, 32)
    sd = I.seeds(2)
    x = I.activations(4096, 3072, sd.x, I.outlier_channels(3072, 31, sd.outliers), 30.0)
    layer = P.SvdqLayer(precision="int4", K=3072, N=3072, rank=32, qweight=pb.qweight,
                        wscales=pb.wscales, w_global=1.0, act_global=1.0, smooth=pb.smooth,
                        lora_down=pb.lora_down, lora_up=pb.lora_up, bias=pb.bias)
    y = host_bits(_layer_dev(layer)(dev_bf16(x)))
    rows = np.unique(np.concatenate([np.arange(3, 4096, 97), [0, 4095]]))
    check_y(y[rows], OL.w4a4_linear_rows("int4", x, layer, rows)["r"])


@pytest.mark.parametrize("K,N", [(12288, 3072), (3072, 9216)])
def test_dit_block_shapes_sampled_rows(K, N):
    """Seeded prepared-layout layers at the DiT block shapes (M = 4608: MLP-down, whose
    GEMM runs on 128-wide tiles, and QKV on 192-wide tiles), in one launch each:
    sampled rows against the oracle."""
    pb = I.prepared_int4_bytes(3, K, N, 32)
    sd = I.seeds(3)
    x = I.activations(4608, K, sd.x, I.outlier_channels(K, I.default_outlier_count(K), sd.outliers),
                      30.0)
    layer = P.SvdqLayer(precision="int4", K=K, N=N, rank=32, qweight=pb.qweight,
                        wscales=pb.wscales, w_global=1.0, act_global=1.0, smooth=pb.smooth,
                        lora_down=pb.lora_down, lora_up=pb.lora_up, bias=pb.bias)
    y = host_bits(_layer_dev(layer)(dev_bf16(x)))
    rows = np.unique(np.concatenate([np.arange(5, 4608, 331), [0, 4607]]))
    check_y(y[rows], OL.w4a4_linear_rows("int4", x, layer, rows)["r"])


def test_timing_hook_counts_two_kernels(tiny):
    li, layer = tiny
    dl = _layer_dev(layer)
    x = dev_bf16(li.x)
    svdq.timing_start(3)
    for _ in range(5):
        dl(x)
    calls, ms = svdq.timing_stop()
    assert calls == 3 and len(ms) == 2 and all(t > 0 for t in ms)


def test_workspace_with_three_k_splits():
    """K = 3200 is quantized in k-splits of 1536, 1536 and 128 values: codes and scales
    in the workspace are bit-exact, and the partial U sums add up to U."""
    rng = np.random.default_rng(81)
    M, K, N, r = 40, 3200, 128, 32
    idx = I.outlier_channels(K, 31, 7)
    x = I.activations(M, K, 101, idx, 30.0)
    m = F.bf16_rne(rng.uniform(0.05, 1.5, K).astype(np.float32))
    ld = F.bf16_rne((rng.standard_normal((r, K)) * 0.05).astype(np.float32))
    lu = F.bf16_rne((rng.standard_normal((N, r)) * 0.05).astype(np.float32))
    qw = F.pack_nibbles(F.int4_encode(rng.integers(-7, 8, size=(N, K))))
    sw = F.bf16_rne((0.01 + 0.01 * rng.random((N, K // 64))).astype(np.float32))
    layer = P.SvdqLayer(precision="int4", K=K, N=N, rank=r, qweight=qw, wscales=sw, w_global=1.0,
                        act_global=1.0, smooth=m, lora_down=ld, lora_up=lu, bias=None)
    dl = _layer_dev(layer)
    ws = torch.zeros(dl.workspace(M, torch.device("cuda")).numel(), dtype=torch.uint8, device="cuda")
    y = dl(dev_bf16(x), workspace=ws)
    torch.cuda.synchronize()
    ref = Q.quantize_act_int4(x, m, ld)
    w = host_bits(ws)
    M_pad, G, nsplit = 256, K // 64, 3
    assert np.array_equal(decode_fp6_operand(w, M_pad, K)[:M], ref["q"])
    off_s = M_pad * K * 3 // 4
    s = scale_records(w[off_s:], G, M_pad)
    assert np.array_equal(s[:, :M], ref["scales"].T)
    off_u = off_s + -(-G * M_pad * 8 // 256) * 256
    u = u_partials(w[off_u:], nsplit, M_pad, r)
    check_u(u.astype(np.float64).sum(axis=0)[:M], ref, ld)
    check_y(host_bits(y), OL.w4a4_linear("int4", x, layer)["r"])


def test_pack_lora_down_fragment_order():
    rng = np.random.default_rng(82)
    for rank, K in [(32, 512), (16, 384)]:
        ld = F.bf16_rne(rng.standard_normal((rank, K)).astype(np.float32))
        packed = host_bits(svdq.pack_lora_down(dev_bf16(ld)))
        units = packed.reshape(K // 128, rank // 16, 4, 4, 16, 8)       # kb, sl, c, q, i, 8
        expect = ld.reshape(rank // 16, 16, K // 128, 4, 4, 8)          # sl, i, kb, q, c, 8
        assert np.array_equal(units, expect.transpose(2, 0, 4, 3, 1, 5))


@pytest.fixture(scope="module")
def split_layer():
    """K = 3072 (24 stages), N = 768: at M = 600 the GEMM has 12 tiles for 256 CUs, all
    in its last partial round, so every tile is split along K (6 pieces of 4 stages)."""
    li = I.layer_inputs(config_id=1, M=600, K=3072, N=768, outlier_count=31, factor=30.0)
    return li, P.prepare_svdq(li.w, li.x_cal, li.bias, rank=32)


@pytest.mark.parametrize("mode", ["plain", "gelu", "qkv"])
def test_linear_with_tail_split(split_layer, mode):
    """Split tiles: pieces store fp32 partials, a second kernel adds them in piece order
    and runs the epilogue; against the oracle, and against the same call with a
    workspace too small for the split (every tile whole, one GEMM kernel)."""
    from oracle import attention as AT
    li, layer = split_layer
    dev = _layer_dev(layer)
    x = dev_bf16(li.x)
    M = li.x.shape[0]
    nq, nk = I.qk_norm_weights()
    rng = np.random.default_rng(5)
    ang = rng.uniform(-3, 3, (M, 64))
    rope_np = np.stack([np.cos(ang), np.sin(ang)], axis=2).astype(np.float32)
    rope = torch.from_numpy(rope_np).cuda()

    def run(ws):
        if mode == "qkv":
            return dev.qkv_norm_rope(x, dev_bf16(nq), dev_bf16(nk), I.QK_NORM_EPS, rope, workspace=ws)
        return dev(x, workspace=ws, gelu=(mode == "gelu"))

    # the full workspace (the 48 MiB K-split area), the one sized for this layer
    # (svdq_workspace_bytes_n) and one without the split area; each is followed by a
    # guard region that the calls must leave alone
    full = svdq.workspace_bytes("int4", 32, M, li.x.shape[1])
    need, guard, split_area = dev.workspace_bytes(M), 1 << 20, 256 * 256 * 192 * 4
    base = full - split_area
    assert base < need < full
    bufs = {n: torch.full((n + guard,), 0xA5, dtype=torch.uint8, device="cuda") for n in (full, need, base)}
    ys = {}
    for n, kernels in ((full, 3), (need, 3), (base, 2)):   # quantizer, GEMM (, tail kernel)
        svdq.timing_start(1)
        ys[n] = host_bits(run(bufs[n][:n]))
        assert len(svdq.timing_stop()[1]) == kernels
        assert bool((bufs[n][n:] == 0xA5).all())
    y_split, y_whole = ys[full], ys[base]
    assert np.array_equal(ys[need], y_split)   # the sized workspace takes the same split
    r = OL.w4a4_linear("int4", li.x, layer)["r"]
    ref = {"plain": r, "gelu": A.gelu_f64(r),
           "qkv": AT.qkv_norm_rope_f64(r, nq, nk, I.QK_NORM_EPS, rope_np)}[mode]
    check_y(y_split, ref)
    check_y(y_whole, ref)
