"""Pins of the Q/K RMSNorm + rotary oracle (oracle/attention.py) against closed forms,
a hand-worked case, invariants, and complex multiplication."""

import numpy as np

from oracle import attention as AT
from oracle import formats as F
from synth import inputs as I

ONE = F.bf16_rne(np.ones(128))


def _bits(v):
    return F.bf16_rne(np.asarray(v, dtype=np.float64))


def test_hand_worked_head_of_four():
    """Head of 4 channels: r = (3, 4, 0, 0) has mean square 25/4, rms 5/2, so the norm
    gives (1.2, 1.6, 0, 0); pair 0 turned by cos 0.6, sin 0.8 gives
    (1.2*0.6 - 1.6*0.8, 1.6*0.6 + 1.2*0.8) = (-0.56, 1.92)."""
    r = np.array([[3.0, 4.0, 0.0, 0.0]])
    n = AT.rms_norm_heads(r, _bits(np.ones(4)), 0.0, head_dim=4)
    assert np.allclose(n, [[1.2, 1.6, 0.0, 0.0]], rtol=0, atol=1e-15)
    rope = np.array([[[0.6, 0.8], [1.0, 0.0]]], dtype=np.float32)
    y = AT.rotary_pairs(n, rope, head_dim=4)
    c, s = float(np.float32(0.6)), float(np.float32(0.8))
    assert np.allclose(y, [[1.2 * c - 1.6 * s, 1.6 * c + 1.2 * s, 0.0, 0.0]], rtol=0, atol=1e-15)
    assert abs(y[0, 0] + 0.56) < 1e-7 and abs(y[0, 1] - 1.92) < 1e-7


def test_rms_norm_constant_head_closed_form():
    """A head of constant a: every output is a / sqrt(a^2 + eps) * w_c."""
    w = _bits(np.linspace(0.5, 1.5, 128))
    for a, eps in [(2.0, 1e-6), (-0.001, 1e-6), (3.0, 0.25)]:
        n = AT.rms_norm_heads(np.full((1, 128), a), w, eps)
        assert np.allclose(n[0], a / np.sqrt(a * a + eps) * F.bf16_to_f64(w), rtol=1e-14, atol=0)


def test_rms_norm_unit_mean_square_and_scale_invariance():
    """With eps 0 and unit weights every head comes out with mean square 1, and
    scaling a head by a positive constant does not change it."""
    rng = np.random.default_rng(1)
    v = rng.standard_normal((5, 3 * 128)) * np.array([1e-3, 1.0, 1e3]).repeat(128)
    n = AT.rms_norm_heads(v, ONE, 0.0)
    ms = np.mean(n.reshape(5, 3, 128) ** 2, axis=2)
    assert np.allclose(ms, 1.0, rtol=1e-13, atol=0)
    assert np.allclose(AT.rms_norm_heads(7.5 * v, ONE, 0.0), n, rtol=1e-13, atol=0)


def test_rms_norm_zero_head_with_eps():
    n = AT.rms_norm_heads(np.zeros((2, 128)), ONE, 1e-6)
    assert not n.any()


def test_rotary_is_complex_multiplication():
    """Pair (a, b) with angle t is the complex product (a + ib) e^{it}."""
    rng = np.random.default_rng(2)
    M = 6
    v = rng.standard_normal((M, 2 * 128))
    ang = rng.uniform(-np.pi, np.pi, size=(M, 64))
    rope = np.stack([np.cos(ang), np.sin(ang)], axis=2).astype(np.float32)
    y = AT.rotary_pairs(v, rope)
    z = (v[:, 0::2] + 1j * v[:, 1::2]).reshape(M, 2, 64)
    e = (rope[..., 0].astype(np.float64) + 1j * rope[..., 1].astype(np.float64))[:, None, :]
    ref = (z * e).reshape(M, 128)
    assert np.allclose(y[:, 0::2], ref.real, rtol=0, atol=1e-14)
    assert np.allclose(y[:, 1::2], ref.imag, rtol=0, atol=1e-14)


def test_rotary_quarter_turn_norms_and_composition():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((3, 128))
    quarter = np.tile(np.array([0.0, 1.0], dtype=np.float32), (3, 64, 1))
    y = AT.rotary_pairs(v, quarter)
    assert np.array_equal(y[:, 0::2], -v[:, 1::2]) and np.array_equal(y[:, 1::2], v[:, 0::2])
    ang1 = rng.uniform(0, 1, (3, 64))
    ang2 = rng.uniform(0, 1, (3, 64))

    def table(a):
        return np.stack([np.cos(a), np.sin(a)], axis=2).astype(np.float32)

    y1 = AT.rotary_pairs(v, table(ang1))
    assert np.allclose(np.hypot(y1[:, 0::2], y1[:, 1::2]), np.hypot(v[:, 0::2], v[:, 1::2]),
                       rtol=1e-6, atol=0)          # |cos + i sin| = 1 to float32 precision
    both = AT.rotary_pairs(y1, table(ang2))
    assert np.allclose(both, AT.rotary_pairs(v, table(ang1 + ang2)), rtol=0, atol=2e-6)
    ident = AT.rotary_pairs(v, table(np.zeros((3, 64))))
    assert np.array_equal(ident, v)


def test_qkv_split_q_k_v_columns():
    """Q uses norm_q and K norm_k; V is the projection itself; heads are 128 wide."""
    rng = np.random.default_rng(4)
    H = 2
    r = rng.standard_normal((4, 3 * H * 128))
    rope = I.rope_table(4)
    zeros = F.bf16_rne(np.zeros(128))
    out = AT.qkv_norm_rope_f64(r, ONE, zeros, 1e-6, rope)
    t = H * 128
    assert np.array_equal(out[:, 2 * t:], r[:, 2 * t:])
    assert not out[:, t:2 * t].any()
    assert np.allclose(np.mean(out[:, :t].reshape(4, H, 128) ** 2, axis=2), 1.0, rtol=1e-5)
    out2 = AT.qkv_norm_rope_f64(r, zeros, ONE, 1e-6, rope)
    assert not out2[:, :t].any() and out2[:, t:2 * t].any()
    # head h of Q depends on columns [128h, 128h + 128) only
    r2 = r.copy()
    r2[:, 128:256] *= 3.0
    out3 = AT.qkv_norm_rope_f64(r2, ONE, ONE, 0.0, rope)
    out1 = AT.qkv_norm_rope_f64(r, ONE, ONE, 0.0, rope)
    assert np.allclose(out3[:, :t], out1[:, :t], rtol=1e-13, atol=1e-13)


def test_rope_table_text_tokens_are_unrotated_and_axes_are_in_order():
    """Text tokens (rows 0..511) sit at position 0; image token 512 + 64 i + j at
    (0, i, j): its first 8 pairs (axis 0) are unrotated, pair 8 turns by i, pair 36
    by j."""
    t = I.rope_table(4608)
    assert np.array_equal(t[:512, :, 0], np.ones((512, 64), np.float32))
    assert not t[:512, :, 1].any()
    m = 512 + 64 * 5 + 9
    assert np.array_equal(t[m, :8, 0], np.ones(8, np.float32))
    assert np.isclose(t[m, 8, 1], np.sin(5.0), atol=1e-7)
    assert np.isclose(t[m, 36, 1], np.sin(9.0), atol=1e-7)
