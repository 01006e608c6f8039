"""Test-side helpers: host <-> device transfer of bit patterns, the Y tolerance check,
and a decoder of the library's kernel layouts (so tests can compare them with the
oracle's interchange codes)."""

from __future__ import annotations

import numpy as np

from oracle import formats as F


def dev_bf16(bits: np.ndarray):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def dev_u8(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def host_bits(t) -> np.ndarray:
    """bf16 / uint8 device tensor -> numpy bit patterns (uint16 / uint8)."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def check_y(y_bits: np.ndarray, r: np.ndarray, max_ulp: int = 2, max_rel: float = 1e-2,
            mean_rel: float = 2e-3, floor_frac: float = 1e-3):
    """The output tolerance: within `max_ulp` bf16 steps of bf16(r) wherever
    |r| >= floor (floor = 1e-3 rms(r)), and relative error e = |y - r| / max(|r|, floor)
    with max(e) <= 1e-2 and mean(e) <= 2e-3."""
    y = F.bf16_to_f64(y_bits)
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    floor = floor_frac * rms if rms > 0 else 1e-30
    big = np.abs(r) >= floor
    ref_bits = F.bf16_rne(r.astype(np.float32))
    ulp = F.bf16_ulp_distance(y_bits, ref_bits)
    worst_ulp = int(ulp[big].max()) if big.any() else 0
    e = np.abs(y - r) / np.maximum(np.abs(r), floor)
    stats = dict(worst_ulp=worst_ulp, max_rel=float(e.max()) if e.size else 0.0,
                 mean_rel=float(e.mean()) if e.size else 0.0)
    assert worst_ulp <= max_ulp, stats
    assert stats["max_rel"] <= max_rel, stats
    assert stats["mean_rel"] <= mean_rel, stats
    return stats


def check_u(u: np.ndarray, ref: dict, lora_down_bits: np.ndarray, chain: int | None = None):
    """The low-rank down projection: fp32 device result u [M, r] against the oracle's
    float64 U, within the rounding bound of an fp32 accumulation whose chain of
    roundings is at most `chain` deep: |u - U| <= chain 2^-24 sum_k |xhat_k L1[k, j]|.
    The default chain = K/8 + 16 is well above the depth of the kernels' sums: the
    fused quantizers sum each 128-wide k-block on the MFMA (four accumulating calls of
    32 products), add the k-blocks of a k-split in a fixed order and hand the GEMM one
    partial per k-split of 1536, which it adds in order; in the interchange quantizer
    each of 8 waves accumulates its k-blocks w, w + 8, ... on the MFMA (at most K/8
    products in one chain) and the 8 partials are then added."""
    if chain is None:
        chain = ref["xhat"].shape[1] // 8 + 16
    xh = np.abs(F.bf16_to_f64(ref["xhat"]))
    ld = np.abs(F.bf16_to_f64(lora_down_bits))
    bound = chain * 2.0 ** -24 * (xh @ ld.T)
    err = np.abs(np.asarray(u, dtype=np.float64) - ref["lora_act"])
    assert np.all(err <= bound), float((err / np.maximum(bound, 1e-300)).max())


def scale_records(buf: np.ndarray, groups: int, rows: int) -> np.ndarray:
    """Activation scale records [groups][rows] of 8 bytes, {s, 0, 0, 0} for an even
    group and {0, s, 0, 0} for an odd one (bf16 positions) -> s bits [groups, rows];
    asserts the zero padding."""
    rec = np.asarray(buf, dtype=np.uint8)[: groups * rows * 8].view(np.uint16).reshape(groups, rows, 4)
    even = np.arange(groups) % 2 == 0
    assert np.all(rec[even][..., 1:] == 0), "nonzero padding in an even-group scale record"
    assert np.all(rec[~even][..., [0, 2, 3]] == 0), "nonzero padding in an odd-group scale record"
    return np.where(even[:, None], rec[..., 0], rec[..., 1])


def pair_scale_records(buf: np.ndarray, groups: int, cols: int) -> np.ndarray:
    """Weight scale records [groups/2][cols] of 8 bytes {s[2p], s[2p+1], 0, 0} -> s bits
    [groups, cols]; asserts the zero padding."""
    assert groups % 2 == 0
    rec = np.asarray(buf, dtype=np.uint8)[: groups // 2 * cols * 8].view(np.uint16).reshape(groups // 2, cols, 4)
    assert np.all(rec[..., 2:] == 0), "nonzero padding in a weight scale record"
    return rec[..., :2].transpose(0, 2, 1).reshape(groups, cols)


def u_partials(buf: np.ndarray, nsplit: int, rows_pad: int, rank: int) -> np.ndarray:
    """Partial low-rank activations in the GEMM's fragment layout
    [split][rows/32][rank/16][2][64 lanes][4] fp32 -> [split, rows, rank]: lane
    l = row % 32 + 32 * ((j % 16) // 8) holds j = 16 c + 8 (l // 32) + [0, 8), the first
    four in the first half, the rest in the second."""
    f = np.asarray(buf, dtype=np.uint8)[: nsplit * rows_pad * rank * 4].view(np.float32)
    f = f.reshape(nsplit, rows_pad // 32, rank // 16, 2, 2, 32, 4)  # .., half, lh, lr, e
    # -> split, row block, lr, slice, lh, half, e
    return f.transpose(0, 1, 5, 2, 4, 3, 6).reshape(nsplit, rows_pad, rank)


def int4_interchange(q: np.ndarray) -> np.ndarray:
    return F.pack_nibbles(F.int4_encode(q))


def decode_fp6_operand(buf: np.ndarray, rows_pad: int, K: int) -> np.ndarray:
    """GEMM A-operand layout (E2M3 lane slots) -> signed int4 codes [rows_pad, K].

    Chunk (row // 32, g) of 1536 B: lane slot h*32 + row%32 holds dwords 0-3 at
    slot*16 and dwords 4-5 at 1024 + slot*8; field f (bits 6f..6f+5 of the six
    dwords) is k = 64 g + 32 h + f, an E2M3 code of value q/8 with sign bit 5: the
    magnitude |q| <= 7 in bits 2:0 (subnormal), or 8 as the normal 1.0 (exponent
    field 1, mantissa 0, i.e. bits 4:0 = 0b01000).
    """
    G = K // 64
    b = np.asarray(buf, dtype=np.uint8)[: rows_pad // 32 * G * 1536].reshape(rows_pad // 32, G, 1536)
    lo = b[:, :, :1024].reshape(rows_pad // 32, G, 64, 16).view(np.uint32)        # [rb, g, slot, 4]
    hi = b[:, :, 1024:].reshape(rows_pad // 32, G, 64, 8).view(np.uint32)         # [rb, g, slot, 2]
    dw = np.concatenate([lo, hi], axis=-1).astype(np.uint64)                       # [rb, g, slot, 6]
    out = np.zeros(dw.shape[:-1] + (32,), dtype=np.int64)
    for f in range(32):
        code = np.zeros(dw.shape[:-1], dtype=np.uint64)
        for bit in range(6):
            p = 6 * f + bit
            code |= ((dw[..., p // 32] >> np.uint64(p % 32)) & np.uint64(1)) << np.uint64(bit)
        mag = (code & np.uint64(0x1F)).astype(np.int64)
        assert np.all(mag <= 8), "an E2M3 field outside the int4 values"
        assert np.all((mag < 8) | ((code & np.uint64(0x20)) > 0)), "+8 is not an int4 code"
        out[..., f] = np.where(code & np.uint64(0x20), -mag, mag)
    # [rb, g, h*32 + r, f] -> row = 32 rb + r, k = 64 g + 32 h + f
    out = out.reshape(rows_pad // 32, G, 2, 32, 32).transpose(0, 3, 1, 2, 4)
    return out.reshape(rows_pad, K)


def _round256(n: int) -> int:
    return -(-n // 256) * 256


def k1_splits(K: int) -> int:
    """k-splits of the layer's quantizer (at most 1536 values each)."""
    return -(-K // 1536)


def int4_workspace(buf: np.ndarray, rows_pad: int, K: int, rank: int):
    """The int4 linear's workspace -> (codes [rows_pad, K], scale bits [K/64, rows_pad],
    partial U [splits, rows_pad, rank] or None): the E2M3 operand, then the scale
    records, then the fp32 partial U, each area starting on a 256-byte boundary."""
    G = K // 64
    w = np.asarray(buf, dtype=np.uint8)
    q = decode_fp6_operand(w, rows_pad, K)
    off_s = _round256(rows_pad * K * 3 // 4)
    s = scale_records(w[off_s:], G, rows_pad)
    off_u = off_s + _round256(G * rows_pad * 8)
    u = u_partials(w[off_u:], k1_splits(K), rows_pad, rank) if rank else None
    return q, s, u


def decode_fp4_operand(buf: np.ndarray, rows_pad: int, K: int, dword_major: bool = False):
    """NVFP4 GEMM operand (FP4 lane slots, then fp16 block scales) -> (E2M1 codes
    [rows_pad, K], block scales as float64 [rows_pad, K/16]).

    Chunk (row // 32, q) of 1 KiB: lane slot 32 h + row % 32 holds in dword j the codes
    of k = 64 q + 16 j + 8 h + [0, 8), element e in bits 4e..4e+3; slot-major (slot l's
    dwords at 16 l, the quantizer's activations) or dword-major (dword j of slot l at
    256 j + 4 l, the packed weights).  The scales follow at the next 256-byte boundary
    as fp16 [K/64][rows_pad][4] (block 4 q + j of a row)."""
    Q = K // 64
    w = np.asarray(buf, dtype=np.uint8)
    if dword_major:
        d = w[: rows_pad * K // 2].view(np.uint32).reshape(rows_pad // 32, Q, 4, 2, 32)  # rb,q,j,h,r
        d = d.transpose(0, 1, 3, 4, 2)                                                 # rb,q,h,r,j
    else:
        d = w[: rows_pad * K // 2].view(np.uint32).reshape(rows_pad // 32, Q, 2, 32, 4)  # rb,q,h,r,j
    nib = np.stack([(d >> np.uint32(4 * e)) & np.uint32(15) for e in range(8)], axis=-1)
    codes = nib.transpose(0, 3, 1, 4, 2, 5).reshape(rows_pad, K).astype(np.uint8)   # rb,r,q,j,h,e
    off = _round256(rows_pad * K // 2)
    s16 = w[off: off + rows_pad * K // 8].view(np.float16).reshape(Q, rows_pad, 4)
    scales = s16.transpose(1, 0, 2).reshape(rows_pad, K // 16).astype(np.float64)
    return codes, scales


def nvfp4_workspace_values(buf: np.ndarray, rows_pad: int, K: int) -> np.ndarray:
    """The NVFP4 linear's staged activations -> float64 values [rows_pad, K]: the exact
    dequantized operand e2m1 * s_b (without the tensor scale)."""
    codes, scales = decode_fp4_operand(buf, rows_pad, K)
    return F.e2m1_decode(codes) * np.repeat(scales, 16, axis=1)
