"""Pins of the oracle's number formats against torch, brute force and hand-worked
fixtures (no GPU)."""

import os

import numpy as np
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                yield line.split()


def test_bf16_roundtrip_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    finite = bits[exp != 0xFF]
    assert np.array_equal(F.bf16_rne(F.bf16_to_f32(finite)), finite)


def test_bf16_rne_matches_torch_cast():
    rng = np.random.default_rng(0)
    u = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    # plant exact ties (low half == 0x8000) and values next to them
    u[:20000] = (u[:20000] & 0xFFFF0000) | 0x8000
    u[20000:30000] = (u[20000:30000] & 0xFFFF0000) | 0x7FFF
    a = u.view(np.float32)
    # keep finite values whose rounding stays finite
    a = a[np.isfinite(a) & (np.abs(a) < 3.0e38)]
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.bf16_rne(a), ref)


def test_e2m1_against_argmin_over_all_codes():
    grid = np.concatenate([np.arange(0, 7, 1 / 64.0), [6.5, 7.0, 50.0]])
    vals = np.concatenate([grid, -grid]).astype(np.float32)
    codes = F.e2m1_rne_sat(vals)
    allv = F.e2m1_decode(np.arange(16))
    for v, c in zip(vals, codes):
        same_sign = [k for k in range(16) if (k >> 3) == int(np.signbit(v))]
        d = np.array([abs(float(v) - allv[k]) for k in same_sign])
        best = [same_sign[i] for i in np.flatnonzero(d == d.min())]
        # ties go to the even magnitude code
        pick = best[0] if len(best) == 1 else [k for k in best if (k & 7) % 2 == 0][0]
        assert c == pick, (v, c, pick)


def test_e2m1_golden_points():
    for v, code in _rows("e2m1_points.txt"):
        assert int(F.e2m1_rne_sat(np.float32(float(v)))) == int(code, 16), v


def test_e4m3_against_torch_below_464():
    mags = F.E4M3_MAGS
    mids = (mags[:-1] + mags[1:]) / 2.0
    rng = np.random.default_rng(1)
    rand = rng.uniform(0, 460, 100_000)
    small = rng.uniform(0, 0.05, 100_000)
    v = np.concatenate([mags, mids, rand, small]).astype(np.float32)
    v = np.concatenate([v, -v])
    v = v[np.abs(v) < 464]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = F.e4m3_rne_sat(v)
    # torch keeps the sign of zero results the same way
    assert np.array_equal(ours, ref)


def test_e4m3_golden_points_and_saturation():
    for v, code in _rows("e4m3_points.txt"):
        assert int(F.e4m3_rne_sat(np.float32(float(v)))) == int(code, 16), v
    assert int(F.e4m3_rne_sat(np.float32(-1.0e6))) == 0xFE


def test_e4m3_decode_grid():
    # 0x38 = 1.0, 0x7E = 448, 0x01 = 2^-9, 0x08 = 2^-6
    assert F.e4m3_decode(np.array([0x38, 0x7E, 0x01, 0x08, 0xB8])).tolist() == \
        [1.0, 448.0, 2.0 ** -9, 2.0 ** -6, -1.0]


def test_nibble_packing_golden():
    for q0, q1, byte in _rows("nibbles.txt"):
        codes = F.int4_encode(np.array([int(q0), int(q1)]))
        packed = F.pack_nibbles(codes)
        assert packed.tolist() == [int(byte, 16)]
        assert F.int4_decode(F.unpack_nibbles(packed)).tolist() == [int(q0), int(q1)]


def test_int4_codes_roundtrip():
    q = np.arange(-8, 8)
    assert np.array_equal(F.int4_decode(F.int4_encode(q)), q)


def test_ulp_distance():
    a = F.bf16_rne(np.array([1.0, -1.0, 0.0], np.float32))
    b = F.bf16_rne(np.array([1.0078125, -1.015625, -0.0], np.float32))
    assert F.bf16_ulp_distance(a, b).tolist() == [1, 2, 0]
