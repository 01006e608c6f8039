"""Pins of the oracle's activation quantizers: grid-exact inputs, hand-worked ties,
invariances and the quantization error bound (no GPU)."""

import os

import numpy as np
import pytest

from oracle import formats as F
from oracle import quant as Q

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
ONE = F.bf16_rne(np.float32(1.0))


def _bits(a):
    a = np.asarray(a, np.float32)
    b = F.bf16_rne(a)
    assert np.array_equal(F.bf16_to_f32(b), a), "value not exact in bf16"
    return b


def _grid_int4(M, K, seed):
    """Rows of k * s with s in {2^e, 1.5 * 2^e} and a +-7 in every group."""
    rng = np.random.default_rng(seed)
    G = K // 64
    k = rng.integers(-7, 8, size=(M, K))
    pos = rng.integers(0, 64, size=(M, G))
    sign = rng.choice([-1, 1], size=(M, G))
    for g in range(G):
        k[np.arange(M), g * 64 + pos[:, g]] = 7 * sign[:, g]
    e = rng.integers(-12, 6, size=(M, G)).astype(np.float64)
    s = np.where(rng.random((M, G)) < 0.5, 1.0, 1.5) * 2.0 ** e
    x = k * np.repeat(s, 64, axis=1)
    return k, s, x


def test_int4_grid_exact_codes_and_scales():
    k, s, x = _grid_int4(8, 512, 0)
    out = Q.quantize_act_int4(_bits(x), np.full(512, ONE, np.uint16))
    assert np.array_equal(out["q"], k)
    assert np.array_equal(F.bf16_to_f64(out["scales"]), s)
    assert np.array_equal(F.int4_decode(F.unpack_nibbles(out["codes"])), k)


def test_int4_hand_worked_ties():
    rows = []
    with open(os.path.join(GOLDEN, "int4_ties.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                v, c = line.split()
                rows.append((float(v), int(c)))
    x = np.zeros((1, 128), np.float32)
    expect = np.zeros(128, np.int64)
    for i, (v, c) in enumerate(rows):
        x[0, i] = v
        expect[i] = c
    x[0, 64:64 + len(rows)] = x[0, :len(rows)] * 4.0     # second group: s = 4
    expect[64:64 + len(rows)] = expect[:len(rows)]
    out = Q.quantize_act_int4(_bits(x), np.full(128, ONE, np.uint16))
    assert out["q"][0].tolist() == expect.tolist()
    assert F.bf16_to_f64(out["scales"]).tolist() == [[1.0, 4.0]]


def test_int4_zero_group_and_sign_symmetry_and_power_of_two():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((16, 256)).astype(np.float32)
    x[:, 64:128] = 0.0
    xb = F.bf16_rne(x)
    one = np.full(256, ONE, np.uint16)
    a = Q.quantize_act_int4(xb, one)
    assert np.all(a["q"][:, 64:128] == 0)
    assert np.all(F.bf16_to_f64(a["scales"][:, 1]) == 0.0)
    b = Q.quantize_act_int4(xb ^ np.uint16(0x8000), one)          # negate
    assert np.array_equal(b["q"], -a["q"])
    assert np.array_equal(b["scales"], a["scales"])
    c = Q.quantize_act_int4(F.bf16_rne(x * np.float32(2.0 ** 5)), one)
    assert np.array_equal(c["q"], a["q"])
    assert np.array_equal(F.bf16_to_f64(c["scales"]), F.bf16_to_f64(a["scales"]) * 2.0 ** 5)
    perm = rng.permutation(16)
    d = Q.quantize_act_int4(xb[perm], one)
    assert np.array_equal(d["codes"], a["codes"][perm])


def test_int4_error_bound_and_range():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((32, 512)).astype(np.float32)
    x[:, ::37] *= 30.0
    m = F.bf16_rne(rng.uniform(0.1, 2.0, 512).astype(np.float32))
    out = Q.quantize_act_int4(F.bf16_rne(x), m)
    xh = F.bf16_to_f64(out["xhat"])
    s = np.repeat(F.bf16_to_f64(out["scales"]), 64, axis=1)
    assert np.all(np.abs(xh - out["q"] * s) <= s / 2)
    assert out["q"].min() >= -7 and out["q"].max() <= 7
    # every group with a nonzero value uses code +-7 somewhere (s = amax/7)
    qa = np.abs(out["q"]).reshape(32, 8, 64).max(axis=2)
    assert np.all(qa == 7)


def test_smoothing_is_one_rounding_of_exact_product():
    # m a power of two: x * m is exact in bf16, so xhat must equal it bit for bit
    rng = np.random.default_rng(5)
    x = F.bf16_rne(rng.standard_normal((4, 128)).astype(np.float32))
    m = _bits(2.0 ** rng.integers(-3, 4, size=128))
    xh = Q.smooth(x, m)
    assert np.array_equal(F.bf16_to_f64(xh), F.bf16_to_f64(x) * F.bf16_to_f64(m)[None, :])


def _grid_nvfp4(M, K, seed):
    rng = np.random.default_rng(seed)
    B = K // 16
    c = rng.integers(0, 16, size=(M, K))
    pos = rng.integers(0, 16, size=(M, B))
    for b in range(B):
        c[np.arange(M), b * 16 + pos[:, b]] = 7 | (8 * rng.integers(0, 2, size=M))
    sc = rng.integers(0x10, 0x60, size=(M, B))           # normal E4M3 scales
    v = F.e2m1_decode(c) * np.repeat(F.e4m3_decode(sc), 16, axis=1)
    return c, sc, v


def test_nvfp4_grid_exact_codes_and_scales():
    c, sc, v = _grid_nvfp4(6, 256, 6)
    out = Q.quantize_act_nvfp4(_bits(v), np.full(256, ONE, np.uint16), 1.0)
    assert np.array_equal(out["e2m1"], c.astype(np.uint8))   # incl. the sign of zero
    assert np.array_equal(out["scales"], sc.astype(np.uint8))


def test_nvfp4_global_scale_power_of_two_invariance():
    c, sc, v = _grid_nvfp4(4, 128, 7)
    one = np.full(128, ONE, np.uint16)
    a = Q.quantize_act_nvfp4(_bits(v), one, 1.0)
    b = Q.quantize_act_nvfp4(_bits(v), one, 0.25)    # g scaled by 2^-2: scales x4
    assert np.array_equal(a["e2m1"], b["e2m1"])
    assert np.array_equal(F.e4m3_decode(b["scales"]), F.e4m3_decode(a["scales"]) * 4.0)


def test_nvfp4_error_bound():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((16, 256)).astype(np.float32)
    xb = F.bf16_rne(x)
    g = float(np.float32(np.max(np.abs(x)) / 2688.0))
    out = Q.quantize_act_nvfp4(xb, np.full(256, ONE, np.uint16), g)
    xh = F.bf16_to_f64(out["xhat"])
    sg = np.repeat(F.e4m3_decode(out["scales"]), 16, axis=1) * float(np.float32(g))
    deq = F.e2m1_decode(out["e2m1"]) * sg
    # half of the widest local E2M1 gap (2, between 4 and 6) times the block scale,
    # plus the float32 rounding of the quotient
    assert np.all(np.abs(xh - deq) <= 1.0 * sg * (1 + 1e-6))
    # elementwise: within half the gap around the chosen grid point
    mags = np.abs(F.e2m1_decode(out["e2m1"]))
    gaps = np.select([mags < 2, mags < 4], [0.5, 1.0], 2.0)
    assert np.all(np.abs(xh - deq) <= gaps / 2 * sg * (1 + 1e-6) + 1e-30)


def test_nvfp4_zero_block_and_negative_zero():
    x = np.zeros((1, 32), np.float32)
    x[0, 16:] = np.linspace(-3, 3, 16)
    x[0, 17] = -1e-4                                     # rounds to zero, keeps sign
    out = Q.quantize_act_nvfp4(F.bf16_rne(x), np.full(32, ONE, np.uint16), 1.0 / 6.0)
    assert np.all(out["e2m1"][0, :16] == 0) and out["scales"][0, 0] == 0
    assert out["e2m1"][0, 17] == 8


@pytest.mark.parametrize("rank", [0, 32])
def test_lora_down_exact_sum(rank):
    rng = np.random.default_rng(9)
    # small integers times powers of two: every product and sum is exact
    x = _bits(rng.integers(-4, 5, size=(8, 128)) * 0.5)
    l1t = _bits(rng.integers(-3, 4, size=(rank, 128)) * 0.25)
    one = np.full(128, ONE, np.uint16)
    u = Q.quantize_act_int4(x, one, l1t if rank else None)["lora_act"]
    assert u.shape == (8, rank)
    if rank:
        exact = F.bf16_to_f64(x) @ F.bf16_to_f64(l1t).T
        assert np.array_equal(u, exact)


def test_lora_down_is_not_rounded_to_bf16():
    """U keeps the full sum: 1 + 2^-10 and 3 * 2^-12 + 2^-20 are not bf16 numbers."""
    x = _bits(np.array([[1.0, 2.0 ** -10, 0.0, 0.0], [0.0, 0.0, 2.0 ** -12, 2.0 ** -20]]))
    x = np.concatenate([x, np.zeros((2, 124), np.uint16)], axis=1)
    l1t = np.zeros((1, 128), np.uint16)
    l1t[0, :4] = _bits(np.array([1.0, 1.0, 3.0, 1.0]))
    one = np.full(128, ONE, np.uint16)
    u = Q.quantize_act_int4(x, one, l1t)["lora_act"]
    assert u[0, 0] == 1.0 + 2.0 ** -10 and u[1, 0] == 3 * 2.0 ** -12 + 2.0 ** -20


def test_int4_subnormal_scales_golden():
    """Hand-worked groups whose scale is a subnormal bf16 number
    (tests/golden/int4_subnormal_scales.txt): the fl32 division and bf16 rounding of
    amax / 7 on the subnormal grid, ties to even, the clamp to the int4 range [-8, 7]
    (a -8 is kept, a +8 becomes 7) and the zero scale of a group whose amax / 7 rounds
    to 0."""
    from golden_cases import int4_subnormal_scales
    x, q, s = int4_subnormal_scales()
    out = Q.quantize_act_int4(x, np.full(x.shape[1], ONE, np.uint16))
    assert np.array_equal(out["scales"], s)
    assert np.array_equal(out["q"], q)
    assert (q == -8).sum() >= 3
    assert np.array_equal(F.int4_decode(F.unpack_nibbles(out["codes"])), q)


def test_nvfp4_non_dyadic_tensor_scale_ties_golden():
    """Hand-worked block with g = fl32(1/3) (tests/golden/nvfp4_tie_third.txt): the
    divisor is fl32(s g), formed before the quotient, which puts every listed value on
    or at an E2M1 point or midpoint; dividing by s and g one after the other misses the
    midpoints and picks the odd neighbours."""
    from golden_cases import nvfp4_tie_third
    x, g, c, s = nvfp4_tie_third()
    out = Q.quantize_act_nvfp4(x, np.full(16, ONE, np.uint16), float(g))
    assert np.array_equal(out["scales"], s)
    assert np.array_equal(out["e2m1"], c)
