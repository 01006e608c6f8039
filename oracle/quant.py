"""Activation quantizers of the SVDQuant W4A4 layer (oracle, test infrastructure).

Source: Diffusers docs "Nunchaku Lite", "Supported quantization types" table --
svdq_w4a4 runs with precision int4 at group size 64 or nvfp4 at group size 16, with
an SVDQ low-rank correction, and rank 32 in the "NunchakuLiteQuantizationConfig"
example.  Both operands of the GEMM are 4-bit (infolabhq tutorial, section on why
4-bit inference matters: weights *and* activations are 4-bit).

The pages leave the steps open; the readings used (all recorded in the design doc):

1. Smoothing.  The per-input-channel smoothing multiplier m (bf16) is folded into
   the activations: xhat = bf16(x * m).  The product of two bf16 numbers is exact in
   float32, so this is one rounding.
2. Groups run along K, per token.  int4: amax over 64 values, symmetric scale
   s = bf16(fl32(amax / 7)), code q = round-half-even(xhat / s) clamped to the
   4-bit two's complement range [-8, 7] (with s = 0 every code is 0).  While s is a
   normal bf16 number it is within 2^-9 of amax / 7, so |xhat / s| < 7.02 and the
   clamp never acts: codes stay in [-7, 7].  Only a subnormal bf16 scale (amax below
   about 2^-123), whose few significant bits can round far below amax / 7, lets a
   quotient reach -8 (kept) or +8 (clamped to 7).
3. NVFP4: blocks of 16.  Per-tensor float32 scale g (calibrated offline, passed
   in).  Block scale s = E4M3(fl32(amax / fl32(6 g))) (saturating).  Element code =
   E2M1(fl32(xhat / fl32(s g))), sign taken from the quotient's sign bit; with s = 0
   the block's codes are 0.
4. Low-rank down projection on the smoothed activations: U = xhat @ L1 with
   L1 = lora_down^T.  The branch's inputs and weights are bf16 and its sum is
   accumulated in float32 on the device; U is not rounded to bf16 before the
   up-projection.  (A bf16-rounded U would let a last-bit difference in the
   accumulation move a whole output row by ulp(U) |L2|, far beyond a few bf16 steps
   of Y for small outputs, so the intermediate is kept at accumulation precision.)
   The oracle's U is the float64 sum, exact up to float64 rounding.
"""

from __future__ import annotations

import numpy as np

from . import formats as F

INT4_GROUP = 64
NVFP4_GROUP = 16


def smooth(x_bits, smooth_bits) -> np.ndarray:
    """xhat = bf16(f32(x) * f32(m)) as bf16 bits [M, K] (step 1)."""
    x = F.bf16_to_f32(x_bits)
    m = F.bf16_to_f32(smooth_bits)
    prod = (x * m[None, :]).astype(np.float32)  # exact: 8-bit x 8-bit significands
    return F.bf16_rne(prod)


def lora_down(xhat_bits, lora_down_bits) -> np.ndarray:
    """U = xhat @ lora_down^T as float64 [M, r] (not rounded; step 4).

    ``lora_down_bits`` is L1^T, shape [r, K], bf16 bits.  Rank 0 gives an empty
    [M, 0] array.
    """
    xh = F.bf16_to_f64(xhat_bits)
    if lora_down_bits is None or np.asarray(lora_down_bits).shape[0] == 0:
        return np.zeros((xh.shape[0], 0), dtype=np.float64)
    l1t = F.bf16_to_f64(lora_down_bits)
    return xh @ l1t.T


def int4_scales_codes(v_f32: np.ndarray, group: int = INT4_GROUP):
    """Symmetric int4 quantization of float32 rows [R, K] in groups along K.

    Returns (codes int [-8, 7] of shape [R, K], scales as bf16 bits [R, K/group]).
    The code is the round-half-even of the exact quotient v / s.  The quotient is
    formed in float64, which decides that rounding exactly: with a float32
    numerator and a bf16 divisor, a quotient that is not a half-integer lies at
    least 2^-25 from one (both v and (k + 1/2) s are multiples of 2^(e_s - 24) near
    a tie, e_s the exponent of s), while float64's error is below 2^-50 for
    |q| < 8; exact ties are exact in float64.
    """
    v = np.asarray(v_f32, dtype=np.float32)
    R, K = v.shape
    assert K % group == 0
    vg = v.reshape(R, K // group, group)
    amax = np.max(np.abs(vg), axis=2).astype(np.float32)
    s_bits = F.bf16_rne((amax / np.float32(7.0)).astype(np.float32))
    s = F.bf16_to_f64(s_bits)
    with np.errstate(divide="ignore", invalid="ignore"):
        quot = vg.astype(np.float64) / s[:, :, None]
    q = np.where(s[:, :, None] > 0, np.rint(quot), 0.0)
    q = np.clip(q, -8, 7).astype(np.int64)
    return q.reshape(R, K), s_bits


def nvfp4_scales_codes(v_f32: np.ndarray, g: float, group: int = NVFP4_GROUP):
    """NVFP4 quantization of float32 rows [R, K] with per-tensor scale ``g``.

    Returns (E2M1 codes 0..15 [R, K], E4M3 scale codes [R, K/group]).
    """
    v = np.asarray(v_f32, dtype=np.float32)
    R, K = v.shape
    assert K % group == 0
    g32 = np.float32(g)
    vg = v.reshape(R, K // group, group)
    amax = np.max(np.abs(vg), axis=2).astype(np.float32)
    denom = np.float32(np.float32(6.0) * g32)
    s_codes = F.e4m3_rne_sat((amax / denom).astype(np.float32))
    s = F.e4m3_decode(s_codes).astype(np.float32)
    d = (s * g32).astype(np.float32)                       # fl32(s * g)
    with np.errstate(divide="ignore", invalid="ignore"):
        quot = (vg / d[:, :, None]).astype(np.float32)     # fl32(v / d)
    codes = F.e2m1_rne_sat(np.where(s[:, :, None] > 0, quot, np.float32(0.0)))
    codes = np.where(s[:, :, None] > 0, codes, 0).astype(np.uint8)
    return codes.reshape(R, K), s_codes


def quantize_act_int4(x_bits, smooth_bits, lora_down_bits=None):
    """svdq_quantize_act, int4 group 64.

    Returns dict(codes=[M, K/2] packed bytes, scales=[M, K/64] bf16 bits,
    lora_act=[M, r] float64, q=[M, K] ints, xhat=[M, K] bf16 bits).
    """
    xhat = smooth(x_bits, smooth_bits)
    q, s_bits = int4_scales_codes(F.bf16_to_f32(xhat), INT4_GROUP)
    return dict(codes=F.pack_nibbles(F.int4_encode(q)), scales=s_bits,
                lora_act=lora_down(xhat, lora_down_bits), q=q, xhat=xhat)


def quantize_act_nvfp4(x_bits, smooth_bits, act_global: float, lora_down_bits=None):
    """svdq_quantize_act, NVFP4 group 16 with E4M3 block scales.

    Returns dict(codes=[M, K/2] packed E2M1 bytes, scales=[M, K/16] E4M3 codes,
    lora_act=[M, r] float64, e2m1=[M, K] codes, xhat=[M, K] bf16 bits).
    """
    xhat = smooth(x_bits, smooth_bits)
    c, s_codes = nvfp4_scales_codes(F.bf16_to_f32(xhat), act_global, NVFP4_GROUP)
    return dict(codes=F.pack_nibbles(c), scales=s_codes,
                lora_act=lora_down(xhat, lora_down_bits), e2m1=c, xhat=xhat)
