"""The int4 quantizer's quotient rule, checked exhaustively on the host.

The code of a value is q = round-half-even(xhat / s) (Diffusers docs "Nunchaku Lite",
"Supported quantization types": svdq_w4a4, int4, group 64; s = bf16(amax / 7)).  The
kernel does not divide: with r = v_rcp_f32(s) (within one ulp of 1/s) it takes
t = fl32(fma(xhat, r, 192)) - 192, which lies on the grid of 2^-16, and rounds t to the
nearest integer, ties to even.  The claim: this equals round-half-even(xhat / s) for
every bf16 xhat and every normal bf16 scale s with |xhat| <= 7.0137 s (the largest
|xhat| / s a bf16 scale of amax / 7 allows).  Here it is checked for all such pairs
with |xhat| >= s / 8 (below that both sides are 0: |t| < 1/8 + 2^-17) and both
neighbours of 1/s as r.  float64 holds fma(xhat, r, 192) exactly (at most 41
significant bits), so float32(...) is the single rounding the fma makes.
"""

import numpy as np

from oracle import formats as F


def _rne_quotient(xh: np.ndarray, s: np.ndarray) -> np.ndarray:
    """round-half-even(xh / s), exactly: k = floor(xh / s) in float64 is exact (a
    non-integer quotient of two bf16 numbers lies at least 2^-12 from any integer in
    this range), the remainder xh - k s is exact in float64, and 2 (xh - k s) against s
    decides the rounding."""
    k = np.floor(xh / s)
    rem = xh - k * s
    twice = 2.0 * rem
    up = (twice > s) | ((twice == s) & (np.mod(k, 2.0) == 1.0))
    return k + up


def _kernel_rule(xh: np.ndarray, r: np.ndarray) -> np.ndarray:
    t = (xh * r + 192.0).astype(np.float32).astype(np.float64) - 192.0
    return np.round(t)  # numpy rounds half to even


def test_snapped_reciprocal_quotient_is_round_half_even():
    # every positive normal bf16 scale: exponent fields 1..254, all 128 mantissas
    s_bits = np.arange(0x0080, 0x7F80, dtype=np.uint32)
    s_all = F.bf16_to_f64(s_bits.astype(np.uint16))
    s_all = s_all[s_all >= 2.0 ** -125]
    # xhat / s = m 2^e / s: every bf16 mantissa in each binade from s / 8 up to 7.0137 s
    mant = 1.0 + np.arange(128, dtype=np.float64) / 128.0
    checked = 0
    for chunk in np.array_split(s_all, 64):
        s = chunk[:, None]
        e0 = np.floor(np.log2(chunk / 8.0))[:, None]
        xs = []
        for de in range(7):
            xs.append(mant[None, :] * np.exp2(e0 + de))
        xh = np.concatenate(xs, axis=1)
        # bf16 values only (below 2^-126 bf16 is subnormal and has fewer mantissa bits)
        xh = np.where(xh < 3.0e38, xh, 0.0)
        bf = F.bf16_to_f64(F.bf16_rne(xh.astype(np.float32))) == xh
        xh = np.where(bf & (xh >= s / 8.0) & (xh <= 7.0137 * s), xh, np.nan)
        xh = np.concatenate([xh, -xh], axis=1)
        s_b = np.broadcast_to(s, xh.shape)
        ok = ~np.isnan(xh)
        xv, sv = xh[ok], s_b[ok]
        want = _rne_quotient(xv, sv)
        r0 = (1.0 / sv).astype(np.float32).astype(np.float64)
        ulp = np.spacing(r0.astype(np.float32)).astype(np.float64)
        for r in (r0 - ulp, r0, r0 + ulp):
            got = _kernel_rule(xv, r)
            bad = got != want
            assert not bad.any(), (xv[bad][:4], sv[bad][:4], got[bad][:4], want[bad][:4])
        checked += xv.size
    assert checked > 10_000_000


def test_rule_meets_every_tie():
    # exact ties xhat = (k + 1/2) s for bf16-representable products, scales with all
    # 128 mantissas: the rule must land on k + 1/2 and round it to the even neighbour
    s = F.bf16_to_f64(np.arange(0x3F80, 0x4000, dtype=np.uint16))
    for k in range(7):
        xh = (k + 0.5) * s
        exact = F.bf16_to_f64(F.bf16_rne(xh.astype(np.float32))) == xh
        xv, sv = xh[exact], s[exact]
        assert xv.size > 0
        r0 = (1.0 / sv).astype(np.float32).astype(np.float64)
        ulp = np.spacing(r0.astype(np.float32)).astype(np.float64)
        even = k if k % 2 == 0 else k + 1
        for r in (r0 - ulp, r0, r0 + ulp):
            assert np.all(_kernel_rule(xv, r) == even)
            assert np.all(_kernel_rule(-xv, r) == -even)
