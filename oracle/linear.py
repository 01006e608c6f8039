"""The W4A4 linear and the AWQ W4A16 linear (oracle, test infrastructure only).

Diffusers docs "Nunchaku Lite", "Supported quantization types" table: svdq_w4a4
(int4 group 64 / nvfp4 group 16) with the SVDQ low-rank correction, and awq_w4a16
(INT4 weight-only, group 64).  Y = X @ W with W logically [K, N]; weights are stored
per output column (rows of length K), like nn.Linear.

Reference values are formed in float64:

  int4   r[m,n] = sum_g sx[m,g] sw[n,g] P_g[m,n] + sum_j U[m,j] L2[j,n] + b[n],
         P_g = sum_{k in g} qx[m,k] qw[n,k]            (exact integers)
  nvfp4  r[m,n] = gx gw sum_b sx[m,b] sw[n,b] P_b[m,n] + U L2 + b,
         P_b = sum_{k in b} e2m1(x) e2m1(w)             (exact multiples of 1/4)
  awq    r[m,n] = sum_g s[n,g] sum_{k in g} x[m,k] (q[n,k] - z[n,g]) + b[n]

Y = bf16(r), rounded once.  ``lora_up`` is L2^T, shape [N, r].
"""

from __future__ import annotations

import numpy as np

from . import formats as F
from . import quant as Q


def _lowrank_bias(U, lora_up_bits, bias_bits, M, N):
    """U @ L2 + b in float64; U is the unrounded down projection [M, r]."""
    out = np.zeros((M, N), dtype=np.float64)
    if lora_up_bits is not None and np.asarray(U).shape[1] > 0:
        out += np.asarray(U, dtype=np.float64) @ F.bf16_to_f64(lora_up_bits).T
    if bias_bits is not None:
        out += F.bf16_to_f64(bias_bits)[None, :]
    return out


def gemm_int4(x_codes, x_scales, w_codes, w_scales, group: int = Q.INT4_GROUP):
    """sum_g sx sw P_g in float64.  Codes are packed [rows, K/2], scales bf16 bits."""
    # float64 holds these small integers and their 64-term dot products exactly
    qx = F.int4_decode(F.unpack_nibbles(x_codes)).astype(np.float64)
    qw = F.int4_decode(F.unpack_nibbles(w_codes)).astype(np.float64)
    sx = F.bf16_to_f64(x_scales)
    sw = F.bf16_to_f64(w_scales)
    M, K = qx.shape
    N = qw.shape[0]
    assert qw.shape[1] == K and K % group == 0
    acc = np.zeros((M, N), dtype=np.float64)
    for g in range(K // group):
        ks = slice(g * group, (g + 1) * group)
        P = qx[:, ks] @ qw[:, ks].T                      # exact integers
        acc += sx[:, g, None] * sw[None, :, g] * P
    return acc


def gemm_nvfp4(x_codes, x_scales, w_codes, w_scales, gx: float, gw: float,
               group: int = Q.NVFP4_GROUP):
    """gx gw sum_b sx sw P_b in float64.  Codes packed E2M1, scales E4M3 codes."""
    vx = F.e2m1_decode(F.unpack_nibbles(x_codes))
    vw = F.e2m1_decode(F.unpack_nibbles(w_codes))
    sx = F.e4m3_decode(x_scales)
    sw = F.e4m3_decode(w_scales)
    M, K = vx.shape
    N = vw.shape[0]
    assert vw.shape[1] == K and K % group == 0
    acc = np.zeros((M, N), dtype=np.float64)
    for b in range(K // group):
        ks = slice(b * group, (b + 1) * group)
        P = vx[:, ks] @ vw[:, ks].T                      # multiples of 1/4, exact
        acc += sx[:, b, None] * sw[None, :, b] * P
    return float(np.float32(gx)) * float(np.float32(gw)) * acc


def w4a4_linear(precision: str, x_bits, layer, act_global: float | None = None):
    """svdq_w4a4_linear: quantize X, 4-bit GEMM, add U @ L2 and the bias.

    ``layer`` is an ``oracle.prep.SvdqLayer``.  Returns dict(r=float64 [M, N],
    y=bf16 bits [M, N], act=the quantize_act outputs).
    """
    M = np.asarray(x_bits).shape[0]
    N = layer.N
    if precision == "int4":
        act = Q.quantize_act_int4(x_bits, layer.smooth, layer.lora_down)
        main = gemm_int4(act["codes"], act["scales"], layer.qweight, layer.wscales)
    elif precision == "nvfp4":
        g = layer.act_global if act_global is None else act_global
        act = Q.quantize_act_nvfp4(x_bits, layer.smooth, g, layer.lora_down)
        main = gemm_nvfp4(act["codes"], act["scales"], layer.qweight, layer.wscales,
                          g, layer.w_global)
    else:
        raise ValueError(precision)
    r = main + _lowrank_bias(act["lora_act"], layer.lora_up, layer.bias, M, N)
    return dict(r=r, y=F.bf16_rne(r.astype(np.float32)), act=act)


def w4a4_linear_rows(precision: str, x_bits, layer, rows, act_global=None):
    """The same reference value on a subset of rows (rows are independent)."""
    return w4a4_linear(precision, np.asarray(x_bits)[rows], layer, act_global)


def awq_w4a16_linear(x_bits, awq):
    """awq_w4a16_linear reference: ``awq`` is an ``oracle.prep.AwqLayer``."""
    x = F.bf16_to_f64(x_bits)
    q = F.unpack_nibbles(awq.qweight).astype(np.float64)      # unsigned 0..15
    s = F.bf16_to_f64(awq.scales)
    z = awq.zeros.astype(np.float64)
    M, K = x.shape
    N = q.shape[0]
    G = awq.group
    acc = np.zeros((M, N), dtype=np.float64)
    for g in range(K // G):
        ks = slice(g * G, (g + 1) * G)
        acc += s[None, :, g] * (x[:, ks] @ (q[:, ks] - z[:, g, None]).T)
    if awq.bias is not None:
        acc += F.bf16_to_f64(awq.bias)[None, :]
    return dict(r=acc, y=F.bf16_rne(acc.astype(np.float32)))


def brute_force_int4(x_bits, layer):
    """Dequantize-then-matmul: (q_x s_x) @ (q_w s_w)^T + U L2 + b, dense float64.

    Independent of ``gemm_int4``'s group loop; used to pin it.
    """
    act = Q.quantize_act_int4(x_bits, layer.smooth, layer.lora_down)
    qx = F.int4_decode(F.unpack_nibbles(act["codes"])).astype(np.float64)
    qw = F.int4_decode(F.unpack_nibbles(layer.qweight)).astype(np.float64)
    sx = np.repeat(F.bf16_to_f64(act["scales"]), Q.INT4_GROUP, axis=1)
    sw = np.repeat(F.bf16_to_f64(layer.wscales), Q.INT4_GROUP, axis=1)
    M, N = qx.shape[0], qw.shape[0]
    return (qx * sx) @ (qw * sw).T + _lowrank_bias(act["lora_act"], layer.lora_up,
                                                    layer.bias, M, N)


def brute_force_nvfp4(x_bits, layer, act_global=None):
    g = layer.act_global if act_global is None else act_global
    act = Q.quantize_act_nvfp4(x_bits, layer.smooth, g, layer.lora_down)
    vx = F.e2m1_decode(F.unpack_nibbles(act["codes"]))
    vw = F.e2m1_decode(F.unpack_nibbles(layer.qweight))
    sx = np.repeat(F.e4m3_decode(act["scales"]), Q.NVFP4_GROUP, axis=1)
    sw = np.repeat(F.e4m3_decode(layer.wscales), Q.NVFP4_GROUP, axis=1)
    M, N = vx.shape[0], vw.shape[0]
    gg = float(np.float32(g)) * float(np.float32(layer.w_global))
    return gg * ((vx * sx) @ (vw * sw).T) + _lowrank_bias(act["lora_act"], layer.lora_up,
                                                           layer.bias, M, N)
