"""Parsers of the hand-worked fixtures under tests/golden/ into input bit patterns and
expected codes and scales.  No arithmetic of the method here: the values and expected
results are the files' own, with their derivations in the files' comments."""

from __future__ import annotations

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                yield line.split()


def int4_subnormal_scales():
    """-> (x bf16 bits [1, 64 G], expected codes [1, 64 G], expected scale bits [1, G]).

    Values are integer multiples of t = 2^-133, whose bf16 bit pattern is the integer
    itself (subnormal mantissa) with the sign in bit 15."""
    entries, scales = [], {}
    for tok in _lines("int4_subnormal_scales.txt"):
        if tok[0] == "scale":
            scales[int(tok[1])] = int(tok[2], 16)
        else:
            entries.append((int(tok[0]), int(tok[1]), int(tok[2])))
    G = max(scales) + 1
    x = np.zeros((1, 64 * G), np.uint16)
    q = np.zeros((1, 64 * G), np.int64)
    used = {g: 0 for g in range(G)}
    for g, v, c in entries:
        k = 64 * g + 5 * used[g]        # spread the listed values over the group
        used[g] += 1
        x[0, k] = abs(v) | (0x8000 if v < 0 else 0)
        q[0, k] = c
    s = np.array([[scales[g] for g in range(G)]], np.uint16)
    return x, q, s


def nvfp4_tie_third():
    """-> (x bf16 bits [1, 16], g (float32), expected E2M1 codes [1, 16], expected E4M3
    scale code [1, 1])."""
    g = scale = None
    vals, codes = [], []
    for tok in _lines("nvfp4_tie_third.txt"):
        if tok[0] == "g":
            g = np.uint32(int(tok[1], 16)).view(np.float32)
        elif tok[0] == "scale":
            scale = int(tok[1], 16)
        else:
            vals.append(float(tok[0]))
            codes.append(int(tok[1]))
    x = np.zeros(16, np.float32)
    c = np.zeros(16, np.uint8)
    x[: len(vals)] = vals
    c[: len(codes)] = codes
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), x), "not a bf16 value"
    return bits[None, :], np.float32(g), c[None, :], np.array([[scale]], np.uint8)
