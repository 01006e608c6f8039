"""The DiT MLP activation between the MLP-up and MLP-down linears (oracle, test
infrastructure only).

Diffusers docs "Nunchaku Lite", "Fused kernels": the MLP of a DiT block applies GELU
between its two projections.  Exact (erf) GELU, the PyTorch default:

    gelu(x) = x Phi(x) = x/2 * erfc(-x / sqrt 2),

evaluated in float64 with the complementary error function (which stays accurate
where 1 + erf cancels, x << 0) and rounded once to bf16.
"""

from __future__ import annotations

import numpy as np
from scipy import special

from . import formats as F


def gelu_f64(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * special.erfc(-x / np.sqrt(2.0))


def gelu_bf16(x_bits) -> np.ndarray:
    """bf16 bits -> (float64 reference values, bf16 bits of the once-rounded result)."""
    r = gelu_f64(F.bf16_to_f64(x_bits))
    return r, F.bf16_rne(r)
