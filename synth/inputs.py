"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This module only draws random numbers and encodes them as the storage types the
layer takes (bf16 bit patterns, float32).  It holds none of the layer's own
arithmetic: no smoothing, no low-rank split, no quantization, no GEMM.

Distributions follow the workloads described for the DiT linears that the SVDQuant
W4A4 layer replaces (1024x1024 images, 4096 image + 512 text tokens):

* activations  X ~ N(0, 1), with a seeded set of outlier input channels scaled by a
  constant factor (x20 for the tiny case, x30 with 1 % of channels otherwise);
* weights      W ~ N(0, 0.02), float32, logical shape [K, N] (Y = X @ W);
* bias         b ~ N(0, 0.02), bf16;
* calibration  a second, independent draw of X used to set the smoothing factors.

Seeds are derived from a config id c as in ``seeds(c)``.
"""

from __future__ import annotations

import dataclasses

import numpy as np
import torch


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Encode float32 values as bf16 bit patterns (uint16) with torch's cast.

    torch rounds float32 -> bfloat16 to nearest-even; this is only the input
    encoding of synthetic data, done by the library, not by this project.
    """
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact: append 16 zero bits)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Seeds:
    x: int
    x_cal: int
    w: int
    bias: int
    outliers: int
    sketch: int

    def step(self, s: int) -> int:
        """Seed of the activations of denoise step ``s`` in a chained workload."""
        return self.x + 99 + s


def seeds(config_id: int) -> Seeds:
    c = 1000 * int(config_id)
    return Seeds(x=c + 1, x_cal=c + 2, w=c + 3, bias=c + 4, outliers=c + 5, sketch=c + 6)


def outlier_channels(K: int, count: int, seed: int) -> np.ndarray:
    """Sorted indices of ``count`` distinct outlier input channels."""
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(K, size=count, replace=False)).astype(np.int64)


def default_outlier_count(K: int) -> int:
    """1 % of the input channels, rounded (31 at K=3072, 123 at K=12288)."""
    return int(round(0.01 * K))


def activations_f32(M: int, K: int, seed: int, outliers: np.ndarray, factor: float) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K), dtype=np.float32)
    if len(outliers):
        x[:, outliers] *= np.float32(factor)
    return x


def activations(M: int, K: int, seed: int, outliers: np.ndarray, factor: float) -> np.ndarray:
    """bf16 bit patterns [M, K] of N(0,1) activations with scaled outlier channels."""
    return to_bf16_bits(activations_f32(M, K, seed, outliers, factor))


def weights(K: int, N: int, seed: int, std: float = 0.02) -> np.ndarray:
    """float32 weights, logical [K, N] (Y = X @ W)."""
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((K, N), dtype=np.float32) * np.float32(std)).astype(np.float32)


def bias(N: int, seed: int, std: float = 0.02) -> np.ndarray:
    """bf16 bit patterns [N]."""
    rng = np.random.default_rng(seed)
    return to_bf16_bits(rng.standard_normal(N, dtype=np.float32) * np.float32(std))


def sketch(N: int, width: int, seed: int) -> np.ndarray:
    """Gaussian test matrix [N, width] (float32) for a randomized range finder."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((N, width), dtype=np.float32)


@dataclasses.dataclass
class LayerInputs:
    """Raw (unprepared) inputs of one linear: activations, calibration data, W, bias."""

    M: int
    K: int
    N: int
    x: np.ndarray        # bf16 bits [M, K]
    x_cal: np.ndarray    # bf16 bits [M_cal, K]
    w: np.ndarray        # float32 [K, N]
    bias: np.ndarray     # bf16 bits [N]
    outliers: np.ndarray
    factor: float


def layer_inputs(config_id: int, M: int, K: int, N: int, *, outlier_count: int | None = None,
                 factor: float = 30.0, cal_rows: int | None = None) -> LayerInputs:
    """All raw inputs of one layer, drawn from the seeds of ``config_id``."""
    sd = seeds(config_id)
    n_out = default_outlier_count(K) if outlier_count is None else outlier_count
    idx = outlier_channels(K, n_out, sd.outliers)
    m_cal = M if cal_rows is None else cal_rows
    return LayerInputs(
        M=M, K=K, N=N,
        x=activations(M, K, sd.x, idx, factor),
        x_cal=activations(m_cal, K, sd.x_cal, idx, factor),
        w=weights(K, N, sd.w),
        bias=bias(N, sd.bias),
        outliers=idx,
        factor=factor,
    )


# The workloads: (config id, M, K, N, outlier count or None for 1 %, outlier factor).
TINY = dict(config_id=1, M=256, K=512, N=512, outlier_count=4, factor=20.0)
ATTN_PROJ = dict(config_id=2, M=4096, K=3072, N=3072, outlier_count=None, factor=30.0)
QKV = dict(config_id=3, M=4608, K=3072, N=9216, outlier_count=None, factor=30.0)
MLP_UP = dict(config_id=3, M=4608, K=3072, N=12288, outlier_count=None, factor=30.0)
MLP_DOWN = dict(config_id=3, M=4608, K=12288, N=3072, outlier_count=None, factor=30.0)
NVFP4_SQ = dict(config_id=4, M=4096, K=3072, N=3072, outlier_count=None, factor=30.0)
NVFP4_UP = dict(config_id=4, M=4096, K=3072, N=12288, outlier_count=None, factor=30.0)


def _nibble_bytes(rng: np.random.Generator, rows: int, half_k: int) -> np.ndarray:
    """Bytes whose two 4-bit fields are drawn uniformly from all 16 two's complement
    patterns, the int4 values -8..7."""
    lo = rng.integers(0, 16, size=(rows, half_k)).astype(np.uint8)
    hi = rng.integers(0, 16, size=(rows, half_k)).astype(np.uint8)
    return (lo | (hi << 4)).astype(np.uint8)


@dataclasses.dataclass
class PreparedBytes:
    """Seeded bytes in the layout of a prepared int4 svdq_w4a4 layer (stand-ins for
    the output of the offline weight preparation, for timing the forward call).

    qweight  uint8 [N, K/2]    codes uniform in -8..7
    wscales  bf16  [N, K/64]   about 0.015 (log-normal spread)
    smooth   bf16  [K]         0.4..0.6, outlier channels 0.08..0.12
    lora_down bf16 [rank, K]   N(0, 0.05);  lora_up bf16 [N, rank]  N(0, 0.05)
    bias     bf16  [N]         N(0, 0.02)
    """

    K: int
    N: int
    rank: int
    qweight: np.ndarray
    wscales: np.ndarray
    smooth: np.ndarray
    lora_down: np.ndarray
    lora_up: np.ndarray
    bias: np.ndarray


def prepared_int4_bytes(config_id: int, K: int, N: int, rank: int = 32,
                        outlier_count: int | None = None, layer: int = 0) -> PreparedBytes:
    """``layer`` tells apart the layers of one config (a block chain); 0 for a single
    layer."""
    sd = seeds(config_id)
    rng = np.random.default_rng(sd.w + 500 + 17 * layer)
    n_out = default_outlier_count(K) if outlier_count is None else outlier_count
    idx = outlier_channels(K, n_out, sd.outliers)
    smooth = rng.uniform(0.4, 0.6, K).astype(np.float32)
    smooth[idx] = rng.uniform(0.08, 0.12, len(idx)).astype(np.float32)
    wscales = (0.015 * np.exp(0.1 * rng.standard_normal((N, K // 64)))).astype(np.float32)
    return PreparedBytes(
        K=K, N=N, rank=rank,
        qweight=_nibble_bytes(rng, N, K // 2),
        wscales=to_bf16_bits(wscales),
        smooth=to_bf16_bits(smooth),
        lora_down=to_bf16_bits(rng.standard_normal((rank, K), dtype=np.float32) * np.float32(0.05)),
        lora_up=to_bf16_bits(rng.standard_normal((N, rank), dtype=np.float32) * np.float32(0.05)),
        bias=bias(N, sd.bias),
    )


@dataclasses.dataclass
class PreparedNvfp4Bytes(PreparedBytes):
    """Seeded bytes in the layout of a prepared nvfp4 svdq_w4a4 layer: E2M1 codes
    uniform over all 16 patterns, E4M3 scale codes between 0.5 and 4 (codes 0x30..0x48),
    per-tensor scales w_global (weights) and act_global (activations)."""

    w_global: float = 1.0
    act_global: float = 1.0


def prepared_nvfp4_bytes(config_id: int, K: int, N: int, rank: int = 32,
                         outlier_count: int | None = None) -> PreparedNvfp4Bytes:
    base = prepared_int4_bytes(config_id, K, N, rank, outlier_count)
    rng = np.random.default_rng(seeds(config_id).w + 700)
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint16).astype(np.uint8)
    scales = rng.integers(0x30, 0x49, size=(N, K // 16), dtype=np.uint16).astype(np.uint8)
    return PreparedNvfp4Bytes(
        K=K, N=N, rank=rank, qweight=codes, wscales=scales, smooth=base.smooth,
        lora_down=base.lora_down, lora_up=base.lora_up, bias=base.bias,
        w_global=float(np.float32(0.02 / 6.0)), act_global=float(np.float32(1.0 / 168.0)))


@dataclasses.dataclass
class PreparedAwqBytes:
    """Seeded bytes of an awq_w4a16 layer: unsigned 4-bit codes uniform over 0..15,
    bf16 group scales about 0.003, zero points uniform over 0..15, bf16 bias."""

    K: int
    N: int
    qweight: np.ndarray   # uint8 [N, K/2]
    scales: np.ndarray    # bf16 bits [N, K/64]
    zeros: np.ndarray     # uint8 [N, K/64]
    bias: np.ndarray      # bf16 bits [N]


def prepared_awq_bytes(config_id: int, K: int, N: int) -> PreparedAwqBytes:
    rng = np.random.default_rng(seeds(config_id).w + 900)
    return PreparedAwqBytes(
        K=K, N=N,
        qweight=rng.integers(0, 256, size=(N, K // 2), dtype=np.uint16).astype(np.uint8),
        scales=to_bf16_bits((0.003 * np.exp(0.1 * rng.standard_normal((N, K // 64)))).astype(np.float32)),
        zeros=rng.integers(0, 16, size=(N, K // 64), dtype=np.uint16).astype(np.uint8),
        bias=bias(N, seeds(config_id).bias))


# The four W4A4 linears of one DiT block (hidden 3072, MLP 12288): name, K, N.
CHAIN_LAYERS = (("qkv", 3072, 9216), ("out", 3072, 3072), ("up", 3072, 12288),
                ("down", 12288, 3072))
CHAIN_CONFIG = 5


def chain_layer_bytes(rank: int = 32) -> dict:
    """Prepared-layout bytes of the block's four int4 layers (config 5), one seed each."""
    return {name: prepared_int4_bytes(CHAIN_CONFIG, K, N, rank, layer=i + 1)
            for i, (name, K, N) in enumerate(CHAIN_LAYERS)}


def chain_step_activations(M: int, step: int) -> np.ndarray:
    """Fresh block input of denoise step ``step``: [M, 3072] bf16 bits, N(0, 1) with 1 %
    outlier channels x30 (the same channels in every step)."""
    sd = seeds(CHAIN_CONFIG)
    K = CHAIN_LAYERS[0][1]
    idx = outlier_channels(K, default_outlier_count(K), sd.outliers)
    return activations(M, K, sd.step(step), idx, 30.0)


# Rotary table and Q/K norm weights of the block's attention (config 3 shapes: 24 heads
# of 128 in a 3072 hidden).  The angles follow the positional layout of a 1024x1024
# DiT: 512 text tokens at position (0, 0, 0), then the 64 x 64 latent patches at
# (0, row, column); 128 = 2 (16 + 56 + 56) channels split over the three axes, each
# axis with base 10000: angle of pair j of an axis of width d at position p is
# p * 10000^(-2j/d).  Batch b repeats the table b times (one sequence per image).
ROPE_AXES = (16, 56, 56)
ROPE_THETA = 10000.0
QK_NORM_EPS = 1e-6


def _rope_positions() -> np.ndarray:
    text = np.zeros((512, 3), dtype=np.float64)
    rr, cc = np.meshgrid(np.arange(64), np.arange(64), indexing="ij")
    img = np.stack([np.zeros(4096), rr.ravel(), cc.ravel()], axis=1).astype(np.float64)
    return np.concatenate([text, img], axis=0)


def rope_table(M: int) -> np.ndarray:
    """[M, 64, 2] float32 (cos, sin) per token and pair, token m at position m % 4608."""
    pos = _rope_positions()
    ang = []
    for a, d in enumerate(ROPE_AXES):
        freq = ROPE_THETA ** (-np.arange(0, d, 2, dtype=np.float64) / d)
        ang.append(pos[:, a:a + 1] * freq[None, :])
    ang = np.concatenate(ang, axis=1)                       # [4608, 64]
    ang = ang[np.arange(M) % ang.shape[0]]
    return np.stack([np.cos(ang), np.sin(ang)], axis=2).astype(np.float32)


def qk_norm_weights(config_id: int = 3, head_dim: int = 128):
    """(norm_q, norm_k) bf16 bits [head_dim] each, 1 + 0.1 N(0, 1)."""
    rng = np.random.default_rng(seeds(config_id).w + 900)
    w = 1.0 + 0.1 * rng.standard_normal((2, head_dim))
    return to_bf16_bits(w[0].astype(np.float32)), to_bf16_bits(w[1].astype(np.float32))


def gaussian_test_matrix(N: int, cols: int, seed: int) -> np.ndarray:
    """Omega [N, cols] float64 ~ N(0, 1): the random test matrix of the randomized
    low-rank factorization in the GPU weight preparation (drawn here, passed in)."""
    return np.random.default_rng(seed).standard_normal((N, cols))
