"""The exact GELU kernel (every finite bf16 input) and the W4A4 linears of a DiT block
called in sequence at the block's token counts (M = 4608 for one 1024x1024 image,
18432 for four), each layer checked against the oracle on its own GPU input."""

import numpy as np
import pytest
import torch

import w4a4_rank_corrected_linear_amd as svdq
from helpers import check_y, dev_bf16, dev_u8, host_bits
from oracle import activation as A
from oracle import formats as F
from oracle import linear as OL
from oracle import prep as P
from synth import inputs as I

pytestmark = pytest.mark.gpu


def _finite_bf16_patterns():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    return b[((b >> 7) & 0xFF) != 0xFF]          # exponent all ones: inf / NaN


def test_gelu_every_finite_bf16_input():
    x = _finite_bf16_patterns()
    y = host_bits(svdq.gelu(dev_bf16(x)))
    _, ref = A.gelu_bf16(x)
    d = F.bf16_ulp_distance(y, ref)
    assert int(d.max()) <= 1, int(d.max())
    assert np.mean(d == 0) > 0.999, float(np.mean(d == 0))


@pytest.mark.parametrize("n", [1, 7, 8, 9, 1000, 4103])
def test_gelu_tail_lengths_and_in_place(n):
    rng = np.random.default_rng(n)
    x = F.bf16_rne((rng.standard_normal(n) * 3).astype(np.float32))
    _, ref = A.gelu_bf16(x)
    t = dev_bf16(x)
    svdq.gelu(t, out=t)
    assert int(F.bf16_ulp_distance(host_bits(t), ref).max()) <= 1


def _oracle_layer(pb):
    return P.SvdqLayer(precision="int4", K=pb.K, N=pb.N, rank=pb.rank, qweight=pb.qweight,
                       wscales=pb.wscales, w_global=1.0, act_global=1.0, smooth=pb.smooth,
                       lora_down=pb.lora_down, lora_up=pb.lora_up, bias=pb.bias)


def _dev_layer(pb):
    return svdq.SvdqLinear.from_interchange(dev_u8(pb.qweight), dev_bf16(pb.wscales),
                                            dev_bf16(pb.smooth), dev_bf16(pb.lora_down),
                                            dev_bf16(pb.lora_up), dev_bf16(pb.bias))


@pytest.fixture(scope="module")
def block():
    pbs = I.chain_layer_bytes()
    layers = {k: _oracle_layer(v) for k, v in pbs.items()}
    dev = {k: _dev_layer(v) for k, v in pbs.items()}
    return layers, svdq.DitBlockChain(dev["qkv"], dev["out"], dev["up"], dev["down"]), dev


@pytest.mark.parametrize("M,step", [(4608, 0), (18432, 3)])
def test_block_chain_each_layer_on_its_gpu_input(block, M, step):
    layers, chain, _ = block
    x = I.chain_step_activations(M, step)
    r = chain(dev_bf16(x))
    torch.cuda.synchronize()
    out = {k: host_bits(v) for k, v in r.items()}
    rows = np.unique(np.concatenate([np.arange(11, M, M // 13), [0, M - 1]]))
    inputs = {"qkv": x, "out": x, "up": out["out"], "down": out["act"]}
    for name in ("qkv", "out", "up", "down"):
        ref = OL.w4a4_linear_rows("int4", inputs[name], layers[name], rows)
        check_y(out[name][rows], ref["r"])
    _, act_ref = A.gelu_bf16(out["up"][rows])
    assert int(F.bf16_ulp_distance(out["act"][rows], act_ref).max()) <= 1
    for v in out.values():
        assert np.all(np.isfinite(F.bf16_to_f64(v)))


def test_block_chain_steps_are_deterministic_and_distinct(block):
    _, chain, _ = block
    a = [host_bits(chain(dev_bf16(I.chain_step_activations(4608, s)))["down"]).copy() for s in (0, 1, 0)]
    assert np.array_equal(a[0], a[2])
    assert not np.array_equal(a[0], a[1])


def test_block_chain_with_gelu_fused_into_mlp_up(block):
    """MLP-up with the GELU in its epilogue: gelu of the unrounded result, rounded once,
    against the oracle's gelu(r) on the layer's GPU input; the other layers as before."""
    layers, _, dev = block
    chain = svdq.DitBlockChain(dev["qkv"], dev["out"], dev["up"], dev["down"], fuse_gelu=True)
    M = 4608
    x = I.chain_step_activations(M, 5)
    r = chain(dev_bf16(x))
    torch.cuda.synchronize()
    out = {k: host_bits(v) for k, v in r.items()}
    assert "up" not in out
    rows = np.unique(np.concatenate([np.arange(7, M, M // 11), [0, M - 1]]))
    ref_up = OL.w4a4_linear_rows("int4", out["out"], layers["up"], rows)["r"]
    check_y(out["act"][rows], A.gelu_f64(ref_up))
    ref_down = OL.w4a4_linear_rows("int4", out["act"], layers["down"], rows)["r"]
    check_y(out["down"][rows], ref_down)


def test_block_chain_with_gelu_in_mlp_down_quantizer(block):
    """MLP-down taking the GELU of MLP-up's bf16 output in its quantizer: no hidden
    activation is written; MLP-down against the oracle on bf16(gelu(up)) formed by the
    GELU kernel (the same values the quantizer forms), the other layers as before."""
    layers, _, dev = block
    chain = svdq.DitBlockChain(dev["qkv"], dev["out"], dev["up"], dev["down"], fuse_gelu="down")
    M = 4608
    x = I.chain_step_activations(M, 6)
    r = chain(dev_bf16(x))
    torch.cuda.synchronize()
    out = {k: host_bits(v) for k, v in r.items()}
    assert "act" not in out and set(out) == set(chain.results())
    rows = np.unique(np.concatenate([np.arange(5, M, M // 12), [0, M - 1]]))
    check_y(out["up"][rows], OL.w4a4_linear_rows("int4", out["out"], layers["up"], rows)["r"])
    h = host_bits(svdq.gelu(dev_bf16(out["up"])))
    check_y(out["down"][rows], OL.w4a4_linear_rows("int4", h, layers["down"], rows)["r"])
    with pytest.raises(ValueError):
        svdq.DitBlockChain(dev["qkv"], dev["out"], dev["up"], dev["down"], fuse_gelu="both")


@pytest.mark.parametrize("fuse", [False, True, "down"])
def test_block_chain_graph_replays_match_eager(block, fuse):
    """Three denoise steps recorded into one HIP graph (svdq_capture_begin/end): every
    replay, with eager calls and synchronizations between replays, leaves exactly the
    eager results of the last step; the eager calls in between see their own results."""
    layers, _, dev = block
    chain = svdq.DitBlockChain(dev["qkv"], dev["out"], dev["up"], dev["down"], fuse_gelu=fuse)
    M = 4608
    steps = (2, 6, 7)
    xs = [dev_bf16(I.chain_step_activations(M, s)) for s in steps]
    x_other = dev_bf16(I.chain_step_activations(M, 4))

    def snapshot():
        torch.cuda.synchronize()
        return {k: host_bits(v).copy() for k, v in chain.results().items()}

    chain(x_other)
    other = snapshot()
    chain(xs[-1])
    ref = snapshot()
    assert not np.array_equal(ref["down"], other["down"])
    graph = chain.capture(xs)
    for rep in range(3):
        graph.launch()
        got = snapshot()
        assert got.keys() == ref.keys()
        for k in ref:
            assert np.array_equal(got[k], ref[k]), f"replay {rep}: {k} differs from the eager result"
        chain(x_other)
        got = snapshot()
        for k in other:
            assert np.array_equal(got[k], other[k]), f"eager call after replay {rep}: {k}"
    graph.destroy()
    # the replayed last step against the oracle on sampled rows
    rows = np.array([0, 1234, M - 1])
    act = ref["act"] if "act" in ref else host_bits(svdq.gelu(dev_bf16(ref["up"])))
    ref_down = OL.w4a4_linear_rows("int4", act, layers["down"], rows)["r"]
    check_y(ref["down"][rows], ref_down)


def test_capture_rejects_the_null_stream_and_timing():
    """The null stream cannot be captured, and capture is refused while the per-kernel
    timing hook is on; nothing is left capturing after either error."""
    lib = svdq.lib()
    assert lib.svdq_capture_begin(None) != 0
    svdq.timing_start(4)
    try:
        s = torch.cuda.Stream()
        assert lib.svdq_capture_begin(s.cuda_stream) != 0
        assert "timing" in svdq._lib.last_error()
    finally:
        svdq.timing_stop()
    x = dev_bf16(np.zeros(64, np.uint16))
    y = svdq.gelu(x)
    torch.cuda.synchronize()
    assert not host_bits(y).any()


def test_block_chain_fully_fused_with_graph(block):
    """The chain with the Q/K norm + rotary fused into QKV and the GELU into MLP-up,
    recorded into a graph over two steps: the replay equals the eager calls, and the
    QKV and MLP-down outputs of the last step match the oracle on sampled rows."""
    from oracle import attention as AT
    layers, _, dev = block
    M = 4608
    nq, nk = I.qk_norm_weights()
    rope_np = I.rope_table(M)
    rope = torch.from_numpy(rope_np).cuda()
    chain = svdq.DitBlockChain(dev["qkv"], dev["out"], dev["up"], dev["down"], fuse_gelu=True,
                               qk_norm=(dev_bf16(nq), dev_bf16(nk), I.QK_NORM_EPS))
    x_np = [I.chain_step_activations(M, s) for s in (1, 3)]
    xs = [dev_bf16(v) for v in x_np]
    chain(xs[-1], rope)
    torch.cuda.synchronize()
    ref = {k: host_bits(v).copy() for k, v in chain.results().items()}
    assert set(ref) == {"qkv", "out", "act", "down"}
    g = chain.capture(xs, rope)
    g.launch()
    torch.cuda.synchronize()
    for k, v in chain.results().items():
        assert np.array_equal(host_bits(v), ref[k]), k
    g.destroy()
    rows = np.array([0, 511, 512, 2049, M - 1])
    r = OL.w4a4_linear_rows("int4", x_np[-1], layers["qkv"], rows)["r"]
    check_y(ref["qkv"][rows], AT.qkv_norm_rope_f64(r, nq, nk, I.QK_NORM_EPS, rope_np[rows]))
    check_y(ref["down"][rows], OL.w4a4_linear_rows("int4", ref["act"], layers["down"], rows)["r"])


def test_block_chain_with_separate_qk_pass(block):
    """fuse_qk=False: the plain QKV projection, then the separate Q/K norm + rotary pass
    on its bf16 output (in place); checked against the oracle on that bf16 output."""
    from oracle import attention as AT
    _, _, dev = block
    M = 1000
    nq, nk = I.qk_norm_weights()
    rope_np = I.rope_table(M)
    x = dev_bf16(I.chain_step_activations(M, 2))
    plain = host_bits(dev["qkv"](x)).copy()
    chain = svdq.DitBlockChain(dev["qkv"], dev["out"], dev["up"], dev["down"], fuse_gelu=True,
                               qk_norm=(dev_bf16(nq), dev_bf16(nk), I.QK_NORM_EPS), fuse_qk=False)
    got = host_bits(chain(x, torch.from_numpy(rope_np).cuda())["qkv"])
    check_y(got, AT.qkv_norm_rope_f64(F.bf16_to_f64(plain), nq, nk, I.QK_NORM_EPS, rope_np))
    assert np.array_equal(got[:, 6144:], plain[:, 6144:])
