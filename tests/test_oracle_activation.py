"""Pins of the oracle's GELU (exact erf form) against the normal distribution it is
defined by, independent of the special-function routine it calls."""

import numpy as np

from oracle import activation as A
from oracle import formats as F


def test_textbook_normal_cdf_values():
    # gelu(x) = x Phi(x); Phi(1), Phi(2), Phi(-3) from standard normal tables
    phi = {1.0: 0.8413447460685429, 2.0: 0.9772498680518208, -1.0: 0.15865525393145707,
           -3.0: 0.0013498980316300946}
    for x, p in phi.items():
        assert abs(A.gelu_f64(x) - x * p) <= 1e-15 * max(1.0, abs(x * p)), x
    assert A.gelu_f64(0.0) == 0.0


def test_odd_part_identity():
    # Phi(x) + Phi(-x) = 1  =>  gelu(x) - gelu(-x) = x
    x = np.random.default_rng(1).uniform(-9, 9, 1000)
    assert np.allclose(A.gelu_f64(x) - A.gelu_f64(-x), x, rtol=1e-14, atol=1e-300)


def test_against_integrated_density():
    # Phi(x) by composite Simpson integration of the density on [-40, x]
    for x in (-6.0, -2.5, -0.7, 0.3, 1.9, 4.0):
        t = np.linspace(-40.0, x, 400001)
        f = np.exp(-0.5 * t * t) / np.sqrt(2 * np.pi)
        h = t[1] - t[0]
        cdf = h / 3 * (f[0] + f[-1] + 4 * f[1:-1:2].sum() + 2 * f[2:-1:2].sum())
        # the sum of 4e5 terms limits the quadrature to about 1e-11 relative
        assert abs(A.gelu_f64(x) - x * cdf) <= 1e-10 * max(abs(x * cdf), 1e-300), x


def test_negative_tail_keeps_relative_accuracy():
    # Mills ratio: Phi(-z) = phi(z)/z (1 - 1/z^2 + 3/z^4 - 15/z^6 + ...) for large z
    for z in (12.0, 20.0, 30.0):
        phi = np.exp(-0.5 * z * z) / np.sqrt(2 * np.pi)
        tail = phi / z * (1 - 1 / z**2 + 3 / z**4 - 15 / z**6)
        assert abs(A.gelu_f64(-z) / (-z * tail) - 1) < 1e-6, z


def test_bf16_rounding_of_reference():
    x = F.bf16_rne(np.array([0.0, 1.0, -1.0, 3.0, -0.5], dtype=np.float32))
    r, bits = A.gelu_bf16(x)
    assert np.array_equal(bits, F.bf16_rne(r))
    assert bits[0] == 0 and F.bf16_to_f64(bits[1]) == F.bf16_to_f64(F.bf16_rne(np.float32(0.8413447460685429)))
