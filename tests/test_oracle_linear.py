"""Pins of the oracle's linears: brute force, grid-exact closed forms, the rank-0
identity, an exact low-rank special case and integer exactness (no GPU)."""

import numpy as np
import pytest

from oracle import formats as F
from oracle import linear as L
from oracle import prep as P
from oracle import quant as Q
from synth import inputs as I

ONE = F.bf16_rne(np.float32(1.0))


def _bits(a):
    a = np.asarray(a, np.float32)
    b = F.bf16_rne(a)
    assert np.array_equal(F.bf16_to_f32(b), a)
    return b


@pytest.fixture(scope="module")
def tiny():
    li = I.layer_inputs(**I.TINY)
    return li, P.prepare_svdq(li.w, li.x_cal, li.bias, rank=32, precision="int4")


def test_brute_force_matches_group_sum_int4(tiny):
    li, layer = tiny
    r = L.w4a4_linear("int4", li.x, layer)["r"]
    bf = L.brute_force_int4(li.x, layer)
    assert np.max(np.abs(r - bf)) <= 1e-12 * np.max(np.abs(bf))


def test_brute_force_matches_group_sum_nvfp4():
    li = I.layer_inputs(**I.TINY)
    layer = P.prepare_svdq(li.w, li.x_cal, li.bias, rank=32, precision="nvfp4")
    r = L.w4a4_linear("nvfp4", li.x, layer)["r"]
    bf = L.brute_force_nvfp4(li.x, layer)
    assert np.max(np.abs(r - bf)) <= 1e-12 * np.max(np.abs(bf))


def _manual_int4_layer(K, N, qw, sw, lora_down=None, lora_up=None, bias=None, smooth=None):
    r = 0 if lora_down is None else lora_down.shape[0]
    return P.SvdqLayer(precision="int4", K=K, N=N, rank=r,
                       qweight=F.pack_nibbles(F.int4_encode(qw)),
                       wscales=_bits(sw), w_global=1.0, act_global=1.0,
                       smooth=np.full(K, ONE, np.uint16) if smooth is None else smooth,
                       lora_down=np.zeros((0, K), np.uint16) if lora_down is None else lora_down,
                       lora_up=np.zeros((N, 0), np.uint16) if lora_up is None else lora_up,
                       bias=bias)


def test_grid_exact_int4_linear_closed_form():
    """X = kx * sx and W = kw * sw on the int4 grid: r must equal the dense fp64
    product of those values, built here from the integers and scales directly."""
    rng = np.random.default_rng(11)
    M, K, N = 24, 256, 40
    kx = rng.integers(-7, 8, size=(M, K))
    for g in range(K // 64):
        kx[:, g * 64] = 7
    sx = 2.0 ** rng.integers(-6, 3, size=(M, K // 64)).astype(np.float64)
    x = kx * np.repeat(sx, 64, axis=1)
    kw = rng.integers(-7, 8, size=(N, K))
    sw = 1.5 * 2.0 ** rng.integers(-9, -3, size=(N, K // 64)).astype(np.float64)
    layer = _manual_int4_layer(K, N, kw, sw)
    out = L.w4a4_linear("int4", _bits(x), layer)
    dense = x @ (kw * np.repeat(sw, 64, axis=1)).T
    assert np.array_equal(out["r"], dense)


def test_rank0_identity_is_plain_w4a4(tiny):
    """Rank 0 and unit smoothing: the layer is the plain quantized GEMM of X."""
    li, _ = tiny
    layer = P.prepare_svdq(li.w, li.x_cal, None, rank=0, smooth=False)
    assert layer.lora_down.shape == (0, li.K)
    out = L.w4a4_linear("int4", li.x, layer)
    # plain W4A4 built from the format helpers only: quantize X rows, quantize W
    # columns, multiply the dequantized matrices
    qx, sx = Q.int4_scales_codes(F.bf16_to_f32(li.x))
    qw, sw = Q.int4_scales_codes(np.ascontiguousarray(li.w.T))
    xd = qx * np.repeat(F.bf16_to_f64(sx), 64, axis=1)
    wd = qw * np.repeat(F.bf16_to_f64(sw), 64, axis=1)
    assert np.allclose(out["r"], xd @ wd.T, rtol=0, atol=1e-12 * np.abs(xd @ wd.T).max())


def test_exact_low_rank_special_case():
    """All-zero residual codes: Y = bf16(xhat @ L1 @ L2 + b) with exact inputs."""
    rng = np.random.default_rng(12)
    M, K, N, r = 16, 128, 48, 32
    m = _bits(2.0 ** rng.integers(-2, 3, size=K))
    x = _bits(rng.integers(-8, 9, size=(M, K)) * 0.25)
    # one power of two per row of L1^T: each U entry is one product, exact in bf16
    l1 = np.zeros((r, K))
    l1[np.arange(r), rng.permutation(K)[:r]] = 2.0 ** rng.integers(-3, 3, size=r)
    l1t = _bits(l1)
    l2t = _bits(rng.integers(-4, 5, size=(N, r)) * 0.5)
    b = _bits(rng.integers(-4, 5, size=N) * 0.0625)
    layer = _manual_int4_layer(K, N, np.zeros((N, K), np.int64), np.zeros((N, K // 64)),
                               lora_down=l1t, lora_up=l2t, bias=b, smooth=m)
    out = L.w4a4_linear("int4", x, layer)
    xhat = F.bf16_to_f64(x) * F.bf16_to_f64(m)[None, :]       # exact (powers of two)
    u = xhat @ F.bf16_to_f64(l1t).T                             # exact small dyadics
    expect = u @ F.bf16_to_f64(l2t).T + F.bf16_to_f64(b)[None, :]
    assert np.array_equal(out["r"], expect)


def test_group_products_are_exact_integers_in_range(tiny):
    li, layer = tiny
    act = Q.quantize_act_int4(li.x, layer.smooth, layer.lora_down)
    qx = F.int4_decode(F.unpack_nibbles(act["codes"]))
    qw = F.int4_decode(F.unpack_nibbles(layer.qweight))
    for g in range(li.K // 64):
        ks = slice(g * 64, (g + 1) * 64)
        Pi = qx[:, ks].astype(np.int64) @ qw[:, ks].T.astype(np.int64)
        Pf = qx[:, ks].astype(np.float64) @ qw[:, ks].T.astype(np.float64)
        assert np.array_equal(Pi, Pf)
        assert np.abs(Pi).max() <= 64 * 49


def test_awq_grid_exact_and_brute_force():
    rng = np.random.default_rng(13)
    K, N, M = 128, 24, 10
    s = 2.0 ** rng.integers(-8, -4, size=(N, K // 64)).astype(np.float64)
    z = rng.integers(0, 16, size=(N, K // 64))
    q = rng.integers(0, 16, size=(N, K))
    for g in range(K // 64):
        q[:, g * 64] = 0
        q[:, g * 64 + 1] = 15
    w = ((q - np.repeat(z, 64, axis=1)) * np.repeat(s, 64, axis=1)).T   # [K, N]
    awq = P.prepare_awq(w.astype(np.float32), None)
    assert np.array_equal(F.unpack_nibbles(awq.qweight), q.astype(np.uint8))
    assert np.array_equal(awq.zeros, z.astype(np.uint8))
    assert np.array_equal(F.bf16_to_f64(awq.scales), s)
    x = _bits(rng.integers(-8, 9, size=(M, K)) * 0.5)
    out = L.awq_w4a16_linear(x, awq)
    assert np.array_equal(out["r"], F.bf16_to_f64(x) @ w)


def test_nvfp4_grid_exact_linear_closed_form():
    rng = np.random.default_rng(14)
    M, K, N = 8, 64, 12
    cx = rng.integers(0, 16, size=(M, K))
    cw = rng.integers(0, 16, size=(N, K))
    for b in range(K // 16):
        cx[:, b * 16] = 7
        cw[:, b * 16] = 7
    sx = rng.integers(0x20, 0x50, size=(M, K // 16))
    sw = rng.integers(0x20, 0x50, size=(N, K // 16))
    x = F.e2m1_decode(cx) * np.repeat(F.e4m3_decode(sx), 16, axis=1)
    wv = F.e2m1_decode(cw) * np.repeat(F.e4m3_decode(sw), 16, axis=1)
    layer = P.SvdqLayer(precision="nvfp4", K=K, N=N, rank=0,
                        qweight=F.pack_nibbles(cw.astype(np.uint8)), wscales=sw.astype(np.uint8),
                        w_global=0.5, act_global=1.0, smooth=np.full(K, ONE, np.uint16),
                        lora_down=np.zeros((0, K), np.uint16), lora_up=np.zeros((N, 0), np.uint16),
                        bias=None)
    out = L.w4a4_linear("nvfp4", _bits(x), layer, act_global=1.0)
    assert np.array_equal(out["r"], 0.5 * (x @ wv.T))


def test_svdq_beats_plain_w4a4_on_outliers(tiny):
    """Sanity, not parity (method quality is parity unpinned: the pages give no
    accuracy figure): smoothing + rank 32 lowers the error against X @ W."""
    li, layer = tiny
    ref = F.bf16_to_f64(li.x) @ li.w.astype(np.float64) + F.bf16_to_f64(li.bias)
    e_svdq = np.linalg.norm(L.w4a4_linear("int4", li.x, layer)["r"] - ref)
    plain = P.prepare_svdq(li.w, li.x_cal, li.bias, rank=0, smooth=False)
    e_plain = np.linalg.norm(L.w4a4_linear("int4", li.x, plain)["r"] - ref)
    assert e_svdq < 0.6 * e_plain
