"""Pins of the offline weight preparation: smoothing identity, Eckart-Young for the
low-rank split, the residual bookkeeping and the weight quantizers (no GPU)."""

import numpy as np

from oracle import formats as F
from oracle import prep as P
from oracle import quant as Q
from synth import inputs as I


def test_smoothing_factors_closed_form():
    x = np.zeros((3, 4), np.float32)
    x[:, 0] = [1.0, -4.0, 2.0]      # amax 4   -> 1/sqrt(4) = 0.5
    x[:, 1] = [0.0, 0.0, 0.0]       # amax 0   -> 1/sqrt(1e-5)
    x[:, 2] = [16.0, 1.0, -1.0]     # amax 16  -> 0.25
    x[:, 3] = [-9.0, 0.5, 3.0]      # amax 9   -> 1/3
    m = F.bf16_to_f64(P.smoothing_factors(F.bf16_rne(x)))
    assert m[0] == 0.5 and m[2] == 0.25
    assert m[1] == F.bf16_to_f64(F.bf16_rne(np.float32(1 / np.sqrt(1e-5))))
    assert m[3] == F.bf16_to_f64(F.bf16_rne(np.float32(1 / 3)))


def test_smoothed_weight_identity_and_residual_bookkeeping():
    li = I.layer_inputs(config_id=1, M=64, K=128, N=96, outlier_count=2, factor=20.0)
    layer = P.prepare_svdq(li.w, li.x_cal, None, rank=8)
    m = F.bf16_to_f64(layer.smooth)
    # diag(m) @ What == W exactly up to the float64 division
    assert np.allclose(m[:, None] * layer.smoothed_w, li.w, rtol=1e-15, atol=0)
    l1 = F.bf16_to_f64(layer.lora_down).T
    l2 = F.bf16_to_f64(layer.lora_up).T
    recon = l1 @ l2 + layer.residual.astype(np.float64)
    assert np.max(np.abs(recon - layer.smoothed_w)) <= 2.0 ** -24 * np.max(np.abs(layer.residual)) * 2


def test_low_rank_eckart_young():
    rng = np.random.default_rng(21)
    K, N, r = 96, 80, 12
    w = rng.standard_normal((K, N))
    L1, L2 = P.low_rank(w, r)
    sig = np.linalg.svd(w, compute_uv=False)
    err2 = np.linalg.norm(w - L1 @ L2) ** 2
    assert abs(err2 - np.sum(sig[r:] ** 2)) <= 1e-9 * np.sum(sig ** 2)
    # sign convention: largest-magnitude entry of each L1 column is positive
    idx = np.argmax(np.abs(L1), axis=0)
    assert np.all(L1[idx, np.arange(r)] > 0)
    # full rank: nothing left
    L1f, L2f = P.low_rank(w, min(K, N))
    assert np.max(np.abs(w - L1f @ L2f)) < 1e-12


def test_exact_rank_weight_leaves_only_factor_rounding():
    rng = np.random.default_rng(22)
    K, N, r = 128, 64, 4
    w = (rng.standard_normal((K, r)) @ rng.standard_normal((r, N))).astype(np.float32)
    x_cal = F.bf16_rne(np.ones((4, K), np.float32))            # m = 1
    layer = P.prepare_svdq(w, x_cal, None, rank=r)
    # the residual holds only the bf16 rounding of the factors (~2^-8 relative)
    assert np.max(np.abs(layer.residual)) <= 2.0 ** -7 * np.max(np.abs(w))


def test_weight_int4_quantizer_per_output_column():
    """Codes of column n come from W[:, n] (residual transposed), groups along K."""
    rng = np.random.default_rng(23)
    K, N = 128, 6
    w = np.zeros((K, N), np.float32)
    for n in range(N):
        w[:, n] = (n + 1) * 0.01 * rng.integers(-7, 8, size=K)
        w[0, n] = 7 * (n + 1) * 0.01
        w[64, n] = -7 * (n + 1) * 0.01
    x_cal = F.bf16_rne(np.ones((4, K), np.float32))
    layer = P.prepare_svdq(w, x_cal, None, rank=0)
    q = F.int4_decode(F.unpack_nibbles(layer.qweight))
    s = F.bf16_to_f64(layer.wscales)
    for n in range(N):
        sn = F.bf16_to_f64(F.bf16_rne(np.float32(np.float32(7 * (n + 1) * 0.01) / np.float32(7))))
        assert np.all(s[n] == sn)
        assert np.array_equal(q[n], np.clip(np.rint(w[:, n].astype(np.float64) / sn), -7, 7))


def test_nvfp4_globals():
    assert P.nvfp4_global(2688.0) == 1.0
    assert P.nvfp4_global(6.0 * 448.0 * 0.5) == 0.5
    rng = np.random.default_rng(24)
    li = I.layer_inputs(config_id=1, M=32, K=64, N=32, outlier_count=1, factor=20.0)
    layer = P.prepare_svdq(li.w, li.x_cal, None, rank=4, precision="nvfp4")
    # the largest block scale of the residual sits at (or next to) the top of E4M3
    top = F.e4m3_decode(layer.wscales).max()
    assert 416 <= top <= 448
    assert layer.qweight.shape == (32, 32) and layer.wscales.shape == (32, 4)
    del rng


def test_nvfp4_act_global_from_smoothed_calibration():
    """g_x is the tensor scale of the smoothed, bf16-rounded calibration activations,
    hand-worked: channel 0 holds the largest raw value (8) but, with multiplier 1/4,
    only 2 after smoothing; channel 1 (multiplier 1) reaches 4; channel 2 holds
    1 + 2^-7 with multiplier 1 + 2^-7, whose exact product 1 + 2^-6 + 2^-14 rounds to
    the bf16 1 + 2^-6.  So amax |bf16(x m)| = 4 and g_x = fl32(4 / 2688) = fl32(1/672),
    not 8/2688 (raw activations) nor a value from an unrounded product."""
    x = np.array([[8.0, -4.0, 1.0078125],
                  [-6.0, 3.0, 0.5]], np.float32)
    m = np.array([0.25, 1.0, 1.0078125], np.float32)
    gx = P.nvfp4_act_global(F.bf16_rne(x), F.bf16_rne(m))
    assert gx == float(np.float32(1.0 / 672.0))
    # the top value sits in the rounded channel when the others are small
    x2 = np.array([[0.5, 0.25, 1.0078125]], np.float32)
    gx2 = P.nvfp4_act_global(F.bf16_rne(x2), F.bf16_rne(m))
    assert gx2 == float(np.float32(1.015625 / 2688.0))
    assert gx2 != float(np.float32(np.float32(1.0078125 * 1.0078125) / np.float32(2688.0)))


def test_prepare_nvfp4_act_global_uses_its_own_smoothing():
    """Through prepare_svdq: the calibration set below has channel amax 16, 4 and 9, so
    the multipliers are 1/4, 1/2 and bf16(1/3) = 0.333984375; the smoothed maxima are
    4, 2 and bf16(9 * 0.333984375) = bf16(3.005859375) = 3.0, and g_x = fl32(4 / 2688)
    (the raw maximum 16 would give four times that)."""
    K = 64
    x = np.zeros((2, K), np.float32)
    x[:, 0] = [16.0, -3.0]
    x[:, 1] = [-4.0, 1.0]
    x[:, 2] = [2.0, 9.0]
    rng = np.random.default_rng(25)
    w = rng.standard_normal((K, 32)).astype(np.float32) * 0.02
    layer = P.prepare_svdq(w, F.bf16_rne(x), None, rank=4, precision="nvfp4")
    m = F.bf16_to_f64(layer.smooth)
    assert m[0] == 0.25 and m[1] == 0.5 and m[2] == 0.333984375
    assert layer.act_global == float(np.float32(1.0 / 672.0))
