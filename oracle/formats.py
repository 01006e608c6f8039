"""Number formats used by the layer (oracle side, test infrastructure only).

* bf16        1 sign, 8 exponent, 7 mantissa bits: the compute_dtype of the layer's
              floating-point buffers (Diffusers docs "Nunchaku Lite",
              "NunchakuLiteQuantizationConfig": compute_dtype, normally bfloat16).
* int4        4-bit two's complement, stored two per byte, even k in the low nibble.
* E2M1        NVFP4 element (OCP FP4): sign bit 3, exponent bits 2:1 (bias 1),
              mantissa bit 0; magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}.
* E4M3 (FN)   NVFP4 block scale: bias 7, no infinities, max 448, subnormal step 2^-9.

All rounding here is round-to-nearest, ties to the even encoding.  E2M1 and E4M3
conversions saturate to the largest finite magnitude.  Finite inputs only.
"""

from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------- bf16


def f32_bits(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def bf16_rne(a) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even.

    Adding 0x7FFF plus the lowest kept bit to the float32 bit pattern and dropping
    the low 16 bits is round-half-even on the magnitude, for normals and
    subnormals alike; values beyond the bf16 range become infinity as IEEE
    rounding does.
    """
    a = np.asarray(a, dtype=np.float32)
    assert np.all(np.isfinite(a)), "bf16_rne: finite inputs only"
    u = a.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_to_f64(bits) -> np.ndarray:
    return bf16_to_f32(bits).astype(np.float64)


def bf16_ulp_distance(a_bits, b_bits) -> np.ndarray:
    """Distance in representable bf16 steps between two arrays of bf16 patterns."""

    def ordered(bits):
        b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
        mag = b & 0x7FFF
        return np.where(b & 0x8000, -mag, mag)

    return np.abs(ordered(a_bits) - ordered(b_bits))


# ------------------------------------------------------------- small float grids


def _grid_round(v, mags: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """Round |v| to the nearest of ``mags`` (ascending), ties to the even code,
    saturating at the largest magnitude.  Returns the magnitude codes."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    n = len(mags)
    hi = np.searchsorted(mags, a, side="left")      # first grid point >= |v|
    sat = hi >= n                                    # beyond the largest point
    hi_c = np.clip(hi, 1, n - 1)
    lo_c = hi_c - 1
    dl = a - mags[lo_c]                              # exact: grid points and the
    dh = mags[hi_c] - a                              # float32 input are exact in f64
    pick_hi = (dh < dl) | ((dh == dl) & (codes[lo_c] % 2 == 1))
    out = np.where(pick_hi, codes[hi_c], codes[lo_c])
    out = np.where(a == 0.0, codes[0], out)
    out = np.where(sat, codes[-1], out)
    return out.astype(np.int64)


# E2M1 -------------------------------------------------------------------------

E2M1_MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1_CODES = np.arange(8)


def e2m1_decode(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64)
    mag = E2M1_MAGS[c & 7]
    return np.where(c & 8, -mag, mag)


def e2m1_rne_sat(v) -> np.ndarray:
    """float -> E2M1 code (0..15).  The sign bit is the sign bit of ``v`` (so a
    negative value that rounds to zero keeps code 8)."""
    v = np.asarray(v, dtype=np.float32)
    mag = _grid_round(v, E2M1_MAGS, E2M1_CODES)
    sign = np.signbit(v).astype(np.int64)
    return (mag | (sign << 3)).astype(np.uint8)


# E4M3FN -----------------------------------------------------------------------


def _e4m3_table():
    mags, codes = [], []
    for code in range(0x7F):  # 0x7F is NaN in the FN variant
        e, m = code >> 3, code & 7
        val = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
        mags.append(val)
        codes.append(code)
    return np.array(mags), np.array(codes)


E4M3_MAGS, E4M3_CODES = _e4m3_table()
E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64)
    assert np.all((c & 0x7F) != 0x7F), "E4M3 NaN code"
    mag = E4M3_MAGS[c & 0x7F]
    return np.where(c & 0x80, -mag, mag)


def e4m3_rne_sat(v) -> np.ndarray:
    """float -> E4M3FN code, round to nearest even, saturate to +-448."""
    v = np.asarray(v, dtype=np.float32)
    mag = _grid_round(v, E4M3_MAGS, E4M3_CODES)
    sign = np.signbit(v).astype(np.int64)
    return (mag | (sign << 7)).astype(np.uint8)


# ------------------------------------------------------------------- int4 / nibbles


def int4_encode(q) -> np.ndarray:
    """Signed integers in [-8, 7] -> 4-bit two's complement codes (0..15)."""
    q = np.asarray(q, dtype=np.int64)
    assert np.all((q >= -8) & (q <= 7))
    return (q & 0xF).astype(np.uint8)


def int4_decode(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64)
    return np.where(c & 8, c - 16, c)


def pack_nibbles(codes) -> np.ndarray:
    """[..., K] codes 0..15 -> [..., K/2] bytes; element 2j in bits 3:0, 2j+1 in 7:4."""
    c = np.asarray(codes, dtype=np.uint8)
    assert c.shape[-1] % 2 == 0
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out
