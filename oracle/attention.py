"""Per-head RMSNorm and rotary embedding of a fused QKV projection (oracle, test
infrastructure only).

Diffusers docs "Nunchaku Lite", "Fused kernels", and the infolabhq tutorial's section
on models that need structural rewrites: the original engine projects Q, K and V with
one matmul (to_qkv) and applies the per-head Q/K normalisation (norm_q, norm_k) and
the rotary embedding in the same operator; the Diffusers path does the same steps one
by one (split into heads, norm_q / norm_k, apply_rotary_emb).  The pages show the call
sequence only.  This oracle takes the plainest reading of it (each choice below is a
reading):

* columns of the projection output: [0, N/3) are Q, [N/3, 2N/3) K, [2N/3, N) V; head
  h of Q (or K) is the D consecutive columns [hD, hD + D) of its third, D = 128;
* RMSNorm over the D values of one token and head, with a per-channel weight w [D]:
  n_c = r_c / sqrt(mean_c r_c^2 + eps) * w_c;
* the rotary embedding turns adjacent pairs (2i, 2i+1) of a normalised head by the
  token's angle for pair i, given as a table of (cos, sin) per token and pair (the
  same for every head and for Q and K):
  y_2i = n_2i cos - n_2i+1 sin,   y_2i+1 = n_2i+1 cos + n_2i sin;
* V is the projection itself;
* all of it in float64 on the unrounded projection result r, rounded once to bf16
  (the fused operator's output).
"""

from __future__ import annotations

import numpy as np

from . import formats as F

HEAD_DIM = 128


def rms_norm_heads(v, weight_bits, eps: float, head_dim: int = HEAD_DIM) -> np.ndarray:
    """v [M, H * head_dim] float64 -> every head scaled by 1 / rms and by the weight."""
    v = np.asarray(v, dtype=np.float64)
    M, W = v.shape
    assert W % head_dim == 0
    h = v.reshape(M, W // head_dim, head_dim)
    ms = np.mean(h * h, axis=2, keepdims=True)
    w = F.bf16_to_f64(weight_bits).reshape(1, 1, head_dim)
    return (h / np.sqrt(ms + eps) * w).reshape(M, W)


def rotary_pairs(v, rope, head_dim: int = HEAD_DIM) -> np.ndarray:
    """v [M, H * head_dim] float64; rope [M, head_dim / 2, 2] float32 (cos, sin) per token
    and pair.  Pair i of every head is turned by the token's angle i."""
    v = np.asarray(v, dtype=np.float64)
    M, W = v.shape
    rope = np.asarray(rope, dtype=np.float32).astype(np.float64)
    assert rope.shape == (M, head_dim // 2, 2)
    h = v.reshape(M, W // head_dim, head_dim // 2, 2)
    c = rope[:, None, :, 0]
    s = rope[:, None, :, 1]
    out = np.empty_like(h)
    out[..., 0] = h[..., 0] * c - h[..., 1] * s
    out[..., 1] = h[..., 1] * c + h[..., 0] * s
    return out.reshape(M, W)


def qkv_norm_rope_f64(r, norm_q_bits, norm_k_bits, eps: float, rope,
                      head_dim: int = HEAD_DIM) -> np.ndarray:
    """r [M, N] float64 (the projection before rounding) -> [M, N] float64 outputs."""
    r = np.asarray(r, dtype=np.float64)
    M, N = r.shape
    assert N % (3 * head_dim) == 0
    t = N // 3
    out = r.copy()
    out[:, :t] = rotary_pairs(rms_norm_heads(r[:, :t], norm_q_bits, eps, head_dim), rope, head_dim)
    out[:, t:2 * t] = rotary_pairs(rms_norm_heads(r[:, t:2 * t], norm_k_bits, eps, head_dim), rope,
                                   head_dim)
    return out
