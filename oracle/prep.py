"""Offline weight preparation (oracle side, test infrastructure only).

The step before the layer runs: the infolabhq tutorial ("quantize your own model"
section) and the Diffusers docs ("Nunchaku Lite" introduction) describe an offline
calibrate -> SVDQuant -> package flow that produces pre-quantized svdq_w4a4 and
awq_w4a16 checkpoints (rank 32 in the config example).  The pages do not give the
steps; the readings used here:

* smoothing factor per input channel k: lambda_k = sqrt(max(amax_k(X_cal), 1e-5)),
  runtime multiplier m_k = bf16(fl32(1 / lambda_k)) applied to X; the weights absorb
  1 / m_k, so (X diag(m)) (diag(1/m) W) = X W;
* low-rank split of the smoothed weight What = diag(1/m) W [K, N]: the top-r SVD,
  L1 = U_r Sigma_r [K, r] and L2 = V_r^T [r, N], each column of L1 signed so that
  its largest-magnitude entry is positive, then rounded to bf16;
* residual R = What - L1_bf16 @ L2_bf16 (float64, stored as float32), quantized
  per output column in groups along K with the same rule as the activations
  (int4: s = bf16(amax / 7), q = rne(R / s) in [-8, 7]; NVFP4: per-tensor
  g_w = fl32(amax|R| / (6 * 448)), E4M3 block scales, E2M1 codes);
* NVFP4 activation scale g_x = fl32(amax|Xhat_cal| / (6 * 448)), static;
* AWQ W4A16 (no smoothing, no low-rank): per (column, group of 64) asymmetric
  uint4 with s = bf16(fl32((max - min) / 15)), z = clamp(rne(-min / s), 0, 15),
  q = clamp(rne(w / s) + z, 0, 15); the activation-aware scale search needs
  calibration data and is not modelled.
"""

from __future__ import annotations

import dataclasses

import numpy as np

from . import formats as F
from . import quant as Q


@dataclasses.dataclass
class SvdqLayer:
    """A prepared svdq_w4a4 layer in the interchange layout.

    qweight  uint8 [N, K/2]   packed codes (int4 two's complement or E2M1)
    wscales  [N, K/G]         bf16 bits (int4) or E4M3 codes (nvfp4)
    w_global float            NVFP4 per-tensor weight scale (1.0 for int4)
    act_global float          NVFP4 static activation scale (1.0 for int4)
    smooth   uint16 [K]       bf16 multiplier m
    lora_down uint16 [r, K]   bf16 L1^T
    lora_up  uint16 [N, r]    bf16 L2^T
    bias     uint16 [N] | None
    """

    precision: str
    K: int
    N: int
    rank: int
    qweight: np.ndarray
    wscales: np.ndarray
    w_global: float
    act_global: float
    smooth: np.ndarray
    lora_down: np.ndarray
    lora_up: np.ndarray
    bias: np.ndarray | None
    residual: np.ndarray | None = None   # float32 [K, N], kept for checks
    smoothed_w: np.ndarray | None = None  # float64 [K, N], kept for checks


@dataclasses.dataclass
class AwqLayer:
    K: int
    N: int
    group: int
    qweight: np.ndarray   # uint8 [N, K/2] unsigned nibbles
    scales: np.ndarray    # bf16 bits [N, K/64]
    zeros: np.ndarray     # uint8 [N, K/64] in 0..15
    bias: np.ndarray | None


def smoothing_factors(x_cal_bits) -> np.ndarray:
    """m = bf16(fl32(1 / sqrt(max(amax_k, 1e-5)))) per input channel, bf16 bits [K]."""
    amax = np.max(np.abs(F.bf16_to_f64(x_cal_bits)), axis=0)
    lam = np.sqrt(np.maximum(amax, 1e-5))
    return F.bf16_rne((1.0 / lam).astype(np.float32))


def low_rank(w_hat: np.ndarray, rank: int):
    """Top-``rank`` SVD factors of w_hat [K, N]: (L1 [K, r], L2 [r, N]) float64."""
    K, N = w_hat.shape
    if rank == 0:
        return np.zeros((K, 0)), np.zeros((0, N))
    U, S, Vt = np.linalg.svd(w_hat, full_matrices=False)
    L1 = U[:, :rank] * S[None, :rank]
    L2 = Vt[:rank, :].copy()
    for j in range(rank):
        i = int(np.argmax(np.abs(L1[:, j])))
        if L1[i, j] < 0:
            L1[:, j] = -L1[:, j]
            L2[j, :] = -L2[j, :]
    return L1, L2


def residual(w_hat: np.ndarray, l1_bits, l2_bits) -> np.ndarray:
    """R = What - L1_bf16 @ L2_bf16 in float64, stored as float32 [K, N]."""
    R = np.asarray(w_hat, np.float64) - F.bf16_to_f64(l1_bits) @ F.bf16_to_f64(l2_bits)
    return R.astype(np.float32)


def residual_int4(r32: np.ndarray):
    """int4 weight quantization of the residual per output column (rows of R^T) in
    groups of 64 along K: (packed codes [N, K/2], bf16 scale bits [N, K/64])."""
    q, s_bits = Q.int4_scales_codes(np.ascontiguousarray(np.asarray(r32, np.float32).T),
                                    Q.INT4_GROUP)
    return F.pack_nibbles(F.int4_encode(q)), s_bits


def nvfp4_global(amax: float) -> float:
    """Per-tensor NVFP4 scale fl32(amax / (6 * 448))."""
    return float(np.float32(np.float32(amax) / np.float32(6.0 * 448.0)))


def residual_nvfp4(r32: np.ndarray):
    """NVFP4 weight quantization of the residual per output column in blocks of 16:
    (g_w, packed E2M1 codes [N, K/2], E4M3 scale codes [N, K/16])."""
    r32 = np.asarray(r32, np.float32)
    gw = nvfp4_global(float(np.max(np.abs(r32))))
    c, s_codes = Q.nvfp4_scales_codes(np.ascontiguousarray(r32.T), gw, Q.NVFP4_GROUP)
    return gw, F.pack_nibbles(c), s_codes


def nvfp4_act_global(x_cal_bits, m_bits) -> float:
    """Static NVFP4 activation scale g_x from the smoothed calibration activations."""
    xhat = Q.smooth(x_cal_bits, m_bits)
    return nvfp4_global(float(np.max(np.abs(F.bf16_to_f32(xhat)))))


def prepare_svdq(w_f32, x_cal_bits, bias_bits, rank: int = 32, precision: str = "int4",
                 smooth: bool = True) -> SvdqLayer:
    """Full offline preparation of one svdq_w4a4 layer from W [K, N] and X_cal."""
    w = np.asarray(w_f32, dtype=np.float64)
    K, N = w.shape
    m_bits = smoothing_factors(x_cal_bits) if smooth else F.bf16_rne(np.ones(K, np.float32))
    m = F.bf16_to_f64(m_bits)
    w_hat = w / m[:, None]
    L1, L2 = low_rank(w_hat, rank)
    l1_bits = F.bf16_rne(L1.astype(np.float32))          # [K, r]
    l2_bits = F.bf16_rne(L2.astype(np.float32))          # [r, N]
    R32 = residual(w_hat, l1_bits, l2_bits)
    if precision == "int4":
        qweight, wscales = residual_int4(R32)
        gw, gx = 1.0, 1.0
    elif precision == "nvfp4":
        gw, qweight, wscales = residual_nvfp4(R32)
        gx = nvfp4_act_global(x_cal_bits, m_bits)
    else:
        raise ValueError(precision)
    return SvdqLayer(precision=precision, K=K, N=N, rank=rank, qweight=qweight,
                     wscales=wscales, w_global=gw, act_global=gx, smooth=m_bits,
                     lora_down=np.ascontiguousarray(l1_bits.T),
                     lora_up=np.ascontiguousarray(l2_bits.T),
                     bias=None if bias_bits is None else np.asarray(bias_bits, np.uint16),
                     residual=R32, smoothed_w=w_hat)


def prepare_awq(w_f32, bias_bits, group: int = 64) -> AwqLayer:
    """Asymmetric uint4 weight-only quantization of W [K, N], per column and group."""
    w = np.asarray(w_f32, dtype=np.float32)
    K, N = w.shape
    wt = np.ascontiguousarray(w.T).reshape(N, K // group, group)       # [N, G, 64]
    mx = wt.max(axis=2)
    mn = wt.min(axis=2)
    s_bits = F.bf16_rne(((mx - mn) / np.float32(15.0)).astype(np.float32))
    s = F.bf16_to_f64(s_bits)
    with np.errstate(divide="ignore", invalid="ignore"):
        z = np.where(s > 0, np.clip(np.rint(-mn.astype(np.float64) / s), 0, 15), 0)
        q = np.where(s[:, :, None] > 0,
                     np.clip(np.rint(wt.astype(np.float64) / s[:, :, None]) + z[:, :, None], 0, 15),
                     0)
    q = q.reshape(N, K).astype(np.uint8)
    return AwqLayer(K=K, N=N, group=group, qweight=F.pack_nibbles(q), scales=s_bits,
                    zeros=z.astype(np.uint8),
                    bias=None if bias_bits is None else np.asarray(bias_bits, np.uint16))
