"""GPU parity of awq_w4a16_linear (INT4 weight-only, group 64) against the oracle:
Y within the stated tolerance; bit-exact on grid-exact inputs."""

import numpy as np
import pytest

import w4a4_rank_corrected_linear_amd as svdq
from helpers import check_y, dev_bf16, dev_u8, host_bits
from oracle import formats as F
from oracle import linear as OL
from oracle import prep as P
from synth import inputs as I

pytestmark = pytest.mark.gpu


def _dev(awq, bias=True):
    return svdq.AwqLinear(dev_u8(awq.qweight), dev_bf16(awq.scales), dev_u8(awq.zeros),
                          dev_bf16(awq.bias) if (bias and awq.bias is not None) else None)


@pytest.fixture(scope="module")
def tiny():
    li = I.layer_inputs(**I.TINY)
    return li, P.prepare_awq(li.w, li.bias)


@pytest.mark.parametrize("M", [256, 1, 17, 129])
def test_awq_tiny(tiny, M):
    li, awq = tiny
    y = _dev(awq)(dev_bf16(li.x[:M]))
    check_y(host_bits(y), OL.awq_w4a16_linear(li.x[:M], awq)["r"])


def test_awq_no_bias_wide_k():
    li = I.layer_inputs(config_id=9, M=96, K=1024, N=384, outlier_count=8, factor=20.0)
    awq = P.prepare_awq(li.w, None)
    y = _dev(awq)(dev_bf16(li.x))
    check_y(host_bits(y), OL.awq_w4a16_linear(li.x, awq)["r"])


@pytest.mark.parametrize("M,N,K", [(300, 640, 640), (1000, 768, 512), (64, 384, 384)])
def test_awq_ragged_tiles(M, N, K):
    """Several 256-row tiles with a partial last one: 128-wide tiles in row-major order
    (M = 300, N = 640) and 192-wide tiles in the XCD-aware order (M = 1000, N = 768);
    K/64 not a multiple of 8 (K = 640, 384) takes the two-group scale loads."""
    li = I.layer_inputs(config_id=9, M=M, K=K, N=N, outlier_count=8, factor=20.0)
    awq = P.prepare_awq(li.w, li.bias)
    y = _dev(awq)(dev_bf16(li.x))
    check_y(host_bits(y), OL.awq_w4a16_linear(li.x, awq)["r"])


def test_awq_grid_exact_is_bit_exact():
    """X = small integers times 2^-3, power-of-two scales in a narrow range: every
    product and partial sum is exact in fp32, so Y equals bf16(r) bit for bit."""
    rng = np.random.default_rng(93)
    M, K, N = 72, 512, 256
    x = F.bf16_rne((rng.integers(-8, 9, size=(M, K)) * 0.125).astype(np.float32))
    q = rng.integers(0, 16, size=(N, K))
    z = rng.integers(0, 16, size=(N, K // 64)).astype(np.uint8)
    s = F.bf16_rne((2.0 ** rng.integers(-6, -3, size=(N, K // 64))).astype(np.float32))
    awq = P.AwqLayer(K=K, N=N, group=64, qweight=F.pack_nibbles(q.astype(np.uint8)), scales=s,
                     zeros=z, bias=None)
    ref = OL.awq_w4a16_linear(x, awq)
    y = _dev(awq)(dev_bf16(x))
    assert np.array_equal(host_bits(y), ref["y"])


@pytest.mark.parametrize("N", [3072, 12288])
def test_awq_full_size_sampled_rows(N):
    """M = 4096, K = 3072 -> N = 3072 and 12288 (the nvfp4 shapes): sampled rows."""
    li = I.layer_inputs(config_id=4, M=4096, K=3072, N=N)
    awq = P.prepare_awq(li.w, li.bias)
    y = host_bits(_dev(awq)(dev_bf16(li.x)))
    rows = np.unique(np.concatenate([np.arange(11, 4096, 173), [0, 4095]]))
    check_y(y[rows], OL.awq_w4a16_linear(li.x[rows], awq)["r"])
