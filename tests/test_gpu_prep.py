"""GPU weight preparation (svdq_prepare_weight, awq_prepare_weight) against the
oracle's preparation: the smoothing factors bit-exact, the residual within one float32
step of the oracle's formula on the GPU's own bf16 factors, the int4 or NVFP4 codes,
scales and tensor scales bit-exact on the GPU's residual, the factorization's residual
norm within 1 % of the exact top-r SVD's (Eckart-Young), the sign convention, the
prepared layer end to end, and the AWQ weights bit-exact."""

import ctypes

import numpy as np
import pytest
import torch

import w4a4_rank_corrected_linear_amd as svdq
from helpers import check_y, dev_bf16, dev_u8, host_bits
from oracle import formats as F
from oracle import linear as OL
from oracle import prep as P
from synth import inputs as I

pytestmark = pytest.mark.gpu


def gpu_prepare(w, x_cal, rank=32, oversample=16, iters=8, seed=7, precision="int4"):
    K, N = w.shape
    nv = precision == "nvfp4"
    L = svdq.lib()
    dev = torch.device("cuda")
    w_d = torch.from_numpy(np.ascontiguousarray(w, np.float32)).to(dev)
    xc_d = dev_bf16(x_cal)
    om = torch.from_numpy(I.gaussian_test_matrix(N, rank + oversample, seed)).to(dev) if rank else None
    qw = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    ws_ = (torch.empty((N, K // 16), dtype=torch.uint8, device=dev) if nv else
           torch.empty((N, K // 64), dtype=torch.bfloat16, device=dev))
    sm = torch.empty((K,), dtype=torch.bfloat16, device=dev)
    ld = torch.empty((max(rank, 1), K), dtype=torch.bfloat16, device=dev)
    lu = torch.empty((N, max(rank, 1)), dtype=torch.bfloat16, device=dev)
    res = torch.empty((K, N), dtype=torch.float32, device=dev)
    nbytes = L.svdq_prepare_workspace_bytes(K, N, rank, oversample)
    # the workspace as sized, followed by a guard region the call must leave alone
    guard = 1 << 20
    work = torch.full((nbytes + guard,), 0xA5, dtype=torch.uint8, device=dev)
    gw, gx = ctypes.c_float(0.0), ctypes.c_float(0.0)
    cfg = svdq._lib.config(precision, rank)
    st = L.svdq_prepare_weight(ctypes.byref(cfg), K, N, w_d.data_ptr(), xc_d.data_ptr(),
                               x_cal.shape[0], om.data_ptr() if rank else None, oversample, iters,
                               qw.data_ptr(), ws_.data_ptr(), sm.data_ptr(),
                               ld.data_ptr() if rank else None, lu.data_ptr() if rank else None,
                               res.data_ptr(), ctypes.byref(gw), ctypes.byref(gx), work.data_ptr(),
                               nbytes, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    svdq._lib.check(st, "svdq_prepare_weight")
    assert bool((work[nbytes:] == 0xA5).all()), "svdq_prepare_weight wrote past its workspace"
    out = dict(qweight=host_bits(qw), wscales=host_bits(ws_), smooth=host_bits(sm),
               residual=res.cpu().numpy(), w_global=gw.value, act_global=gx.value)
    if rank:
        out["lora_down"] = host_bits(ld)
        out["lora_up"] = host_bits(lu)
    return out


def check_prepared(w, x_cal, g, ref, rank, precision="int4"):
    # smoothing factors: bit-exact
    assert np.array_equal(g["smooth"], ref.smooth)
    m = F.bf16_to_f64(g["smooth"])
    w_hat = np.asarray(w, np.float64) / m[:, None]
    if rank:
        l1 = np.ascontiguousarray(g["lora_down"].T)
        l2 = np.ascontiguousarray(g["lora_up"].T)
        r_ref = P.residual(w_hat, l1, l2)
        # the sign convention: the largest-magnitude entry of each L1 column is positive
        v = F.bf16_to_f64(l1)
        assert np.all(v.max(axis=0) >= -v.min(axis=0))
        # factorization quality against the exact top-r SVD (both with bf16 factors)
        ratio = np.linalg.norm(g["residual"]) / np.linalg.norm(ref.residual)
        assert ratio <= 1.01, ratio
    else:
        r_ref = w_hat.astype(np.float32)
    # the residual within one float32 step (the length-r float64 sums may differ in order)
    r = g["residual"]
    assert np.all(np.abs(r.astype(np.float64) - r_ref) <= np.spacing(np.abs(r_ref))), \
        float(np.max(np.abs(r.astype(np.float64) - r_ref)))
    # the quantization of the GPU's residual: bit-exact
    if precision == "int4":
        qw, s = P.residual_int4(r)
    else:
        gw, qw, s = P.residual_nvfp4(r)
        assert np.float32(g["w_global"]) == np.float32(gw)
        assert np.float32(g["act_global"]) == np.float32(P.nvfp4_act_global(x_cal, g["smooth"]))
    assert np.array_equal(g["qweight"], qw)
    assert np.array_equal(g["wscales"], s)


@pytest.mark.parametrize("rank", [0, 16, 32])
def test_prepare_tiny(rank):
    li = I.layer_inputs(**I.TINY)
    ref = P.prepare_svdq(li.w, li.x_cal, li.bias, rank=rank)
    g = gpu_prepare(li.w, li.x_cal, rank=rank)
    check_prepared(li.w, li.x_cal, g, ref, rank)


@pytest.mark.parametrize("K,N", [(1024, 1536), (1536, 1024)])
def test_prepare_rectangular_with_outliers(K, N):
    """Wide and tall weights (the orthogonalization runs on K and on N rows) with 1 %
    outlier channels x30 in the calibration data."""
    li = I.layer_inputs(config_id=2, M=64, K=K, N=N, cal_rows=512)
    ref = P.prepare_svdq(li.w, li.x_cal, li.bias, rank=32)
    g = gpu_prepare(li.w, li.x_cal, rank=32)
    check_prepared(li.w, li.x_cal, g, ref, 32)


def test_prepared_layer_end_to_end():
    """A layer prepared on the GPU runs through svdq_w4a4_linear within the tolerance of
    the oracle's linear on the same prepared bytes, and its error against the exact
    float64 X W is below that of plain W4A4 (no smoothing, rank 0)."""
    li = I.layer_inputs(**I.TINY)
    g = gpu_prepare(li.w, li.x_cal, rank=32)
    layer = P.SvdqLayer(precision="int4", K=li.K, N=li.N, rank=32, qweight=g["qweight"],
                        wscales=g["wscales"], w_global=1.0, act_global=1.0, smooth=g["smooth"],
                        lora_down=g["lora_down"], lora_up=g["lora_up"], bias=li.bias)
    dev = svdq.SvdqLinear.from_interchange(dev_u8(layer.qweight), dev_bf16(layer.wscales),
                                           dev_bf16(layer.smooth), dev_bf16(layer.lora_down),
                                           dev_bf16(layer.lora_up), dev_bf16(layer.bias))
    y = host_bits(dev(dev_bf16(li.x)))
    check_y(y, OL.w4a4_linear("int4", li.x, layer)["r"])
    exact = F.bf16_to_f64(li.x) @ np.asarray(li.w, np.float64) + F.bf16_to_f64(li.bias)[None, :]
    plain = P.prepare_svdq(li.w, li.x_cal, li.bias, rank=0, smooth=False)
    e_gpu = np.linalg.norm(F.bf16_to_f64(y) - exact)
    e_plain = np.linalg.norm(OL.w4a4_linear("int4", li.x, plain)["r"] - exact)
    assert e_gpu < e_plain, (e_gpu, e_plain)


@pytest.mark.parametrize("rank", [0, 32])
def test_prepare_nvfp4(rank):
    li = I.layer_inputs(**I.TINY)
    ref = P.prepare_svdq(li.w, li.x_cal, li.bias, rank=rank, precision="nvfp4")
    g = gpu_prepare(li.w, li.x_cal, rank=rank, precision="nvfp4")
    check_prepared(li.w, li.x_cal, g, ref, rank, precision="nvfp4")


@pytest.mark.parametrize("K,N", [(512, 512), (1024, 1536)])
def test_prepare_awq(K, N):
    """awq_prepare_weight bit-exact against the oracle, including a constant group
    (s = 0) and a group with only non-negative values (z = 0)."""
    w = I.weights(K, N, 11)
    w[:64, 5] = 0.25                  # constant group: max - min = 0
    w[64:128, 7] = np.abs(w[64:128, 7])
    ref = P.prepare_awq(w, None)
    L = svdq.lib()
    dev = torch.device("cuda")
    w_d = torch.from_numpy(np.ascontiguousarray(w, np.float32)).to(dev)
    qw = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    sc = torch.empty((N, K // 64), dtype=torch.bfloat16, device=dev)
    zs = torch.empty((N, K // 64), dtype=torch.uint8, device=dev)
    st = L.awq_prepare_weight(K, N, w_d.data_ptr(), qw.data_ptr(), sc.data_ptr(), zs.data_ptr(),
                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    svdq._lib.check(st, "awq_prepare_weight")
    assert np.array_equal(host_bits(qw), ref.qweight)
    assert np.array_equal(host_bits(sc), ref.scales)
    assert np.array_equal(host_bits(zs), ref.zeros)


@pytest.mark.parametrize("precision", ["int4", "nvfp4"])
def test_prepare_layer_wrapper(precision):
    """svdq.prepare_layer: prepared and packed on the GPU, its output closer to the exact
    X W than plain W4A4 (no smoothing, rank 0); svdq.prepare_awq_layer within the
    tolerance of the oracle's AWQ linear on the oracle's AWQ weights (bit-exact weights)."""
    li = I.layer_inputs(**I.TINY)
    w = torch.from_numpy(np.ascontiguousarray(li.w, np.float32)).cuda()
    layer = svdq.prepare_layer(w, dev_bf16(li.x_cal), dev_bf16(li.bias), precision=precision)
    y = F.bf16_to_f64(host_bits(layer(dev_bf16(li.x))))
    exact = F.bf16_to_f64(li.x) @ np.asarray(li.w, np.float64) + F.bf16_to_f64(li.bias)[None, :]
    plain = P.prepare_svdq(li.w, li.x_cal, li.bias, rank=0, precision=precision, smooth=False)
    e_plain = np.linalg.norm(OL.w4a4_linear(precision, li.x, plain)["r"] - exact)
    assert np.linalg.norm(y - exact) < e_plain
    awq = svdq.prepare_awq_layer(w, dev_bf16(li.bias))
    ref = P.prepare_awq(li.w, li.bias)
    check_y(host_bits(awq(dev_bf16(li.x))), OL.awq_w4a16_linear(li.x, ref)["r"])
