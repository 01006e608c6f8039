"""The W4A4 linears of one DiT transformer block, called in sequence.

A block of the 1024x1024 DiT (3072 hidden, 4096 image + 512 text tokens) runs four
svdq_w4a4 linears: the fused QKV projection 3072 -> 9216, the attention output
projection 3072 -> 3072, and the MLP pair 3072 -> 12288 -> 3072 with an exact GELU
between (Diffusers docs "Nunchaku Lite", "Fused kernels": the block's projections and
its GELU MLP).  Attention itself, the norms and the residual adds are not part of the
layer: the QKV output is produced for the attention that would consume it, and the
output projection reads the block's input activations in place of the attention
output.  The GELU runs as its own kernel, fused into the MLP-up GEMM's epilogue (on
the fp32 result, before the bf16 rounding), or fused into MLP-down's quantizer (on the
bf16 MLP-up output as the quantizer loads it, the same values the separate kernel
writes).  Several denoise steps can be
recorded into one HIP graph and replayed with one launch (the launch overhead that the
tutorial's torch.compile section recovers).  Every step runs in the library's kernels;
this module only orders the calls.
"""

from __future__ import annotations

import torch

from .api import Graph, SvdqLinear, capture, gelu, qk_norm_rope


class DitBlockChain:
    """qkv, out, up, down: SvdqLinear layers of shapes 3072->9216, 3072->3072,
    3072->12288 and 12288->3072 (any K/N that chain the same way)."""

    def __init__(self, qkv: SvdqLinear, out: SvdqLinear, up: SvdqLinear, down: SvdqLinear,
                 fuse_gelu: bool | str = False, qk_norm=None, fuse_qk: bool = True):
        """fuse_gelu: False (the GELU as its own kernel), True or "up" (in MLP-up's
        epilogue) or "down" (in MLP-down's quantizer).  qk_norm: None, or (norm_q, norm_k, eps) to apply the per-head Q/K RMSNorm and
        rotary embedding to the QKV output, fused into the projection's epilogue
        (fuse_qk) or as a separate pass over its bf16 output; forward then takes the
        rotary table (float32 [M, 64, 2])."""
        if out.N != up.K or up.N != down.K or qkv.K != out.K:
            raise ValueError("layer shapes do not chain: "
                             f"qkv {qkv.K}->{qkv.N}, out {out.K}->{out.N}, up {up.K}->{up.N}, "
                             f"down {down.K}->{down.N}")
        self.qkv, self.out, self.up, self.down = qkv, out, up, down
        if fuse_gelu not in (False, True, "up", "down"):
            raise ValueError(f"fuse_gelu = {fuse_gelu!r}: False, True, 'up' or 'down'")
        self.gelu_mode = "up" if fuse_gelu is True else (fuse_gelu or "separate")
        self.fuse_gelu = fuse_gelu
        self.qk_norm = qk_norm
        self.fuse_qk = fuse_qk
        self._buf = {}

    def _tensor(self, name: str, shape, device, dtype=torch.bfloat16) -> torch.Tensor:
        t = self._buf.get(name)
        if t is None or tuple(t.shape) != tuple(shape) or t.device != device:
            t = torch.empty(shape, dtype=dtype, device=device)
            self._buf[name] = t
        return t

    def forward(self, x: torch.Tensor, rope: torch.Tensor | None = None) -> dict:
        """x [M, K] bf16 -> {"qkv", "out", "up", "act", "down"} ("up" absent when the GELU
        is fused into MLP-up's epilogue, "act" when it is fused into MLP-down); the buffers are reused by the next call of the
        same M (copy what must outlive it).  rope: the rotary table, needed when the
        chain fuses the Q/K norm and rotary embedding into the QKV projection."""
        M, dev = x.shape[0], x.device
        need = max(layer.workspace_bytes(M) for layer in (self.qkv, self.out, self.up, self.down))
        ws = self._tensor("ws", (need,), dev, torch.uint8)   # one workspace, calls run in order
        r = {}
        if self.qk_norm is not None:
            if rope is None:
                raise ValueError("this chain fuses the Q/K norm and rotary embedding: pass rope")
            nq, nk, eps = self.qk_norm
            qkv = self._tensor("qkv", (M, self.qkv.N), dev)
            if self.fuse_qk:
                r["qkv"] = self.qkv.qkv_norm_rope(x, nq, nk, eps, rope, out=qkv, workspace=ws)
            else:
                self.qkv(x, out=qkv, workspace=ws)
                r["qkv"] = qk_norm_rope(qkv, nq, nk, eps, rope, out=qkv)
        else:
            r["qkv"] = self.qkv(x, out=self._tensor("qkv", (M, self.qkv.N), dev), workspace=ws)
        r["out"] = self.out(x, out=self._tensor("out", (M, self.out.N), dev), workspace=ws)
        if self.gelu_mode == "up":
            r["act"] = self.up(r["out"], out=self._tensor("act", (M, self.up.N), dev), workspace=ws,
                               gelu=True)
        else:
            r["up"] = self.up(r["out"], out=self._tensor("up", (M, self.up.N), dev), workspace=ws)
        if self.gelu_mode == "down":
            r["down"] = self.down(r["up"], out=self._tensor("down", (M, self.down.N), dev),
                                  workspace=ws, gelu_in=True)
            return r
        if self.gelu_mode == "separate":
            r["act"] = gelu(r["up"], out=self._tensor("act", (M, self.up.N), dev))
        r["down"] = self.down(r["act"], out=self._tensor("down", (M, self.down.N), dev), workspace=ws)
        return r

    __call__ = forward

    def results(self) -> dict:
        """The result buffers of the last call or replay, by name (see forward)."""
        names = {"up": ("qkv", "out", "act", "down"), "down": ("qkv", "out", "up", "down"),
                 "separate": ("qkv", "out", "up", "act", "down")}[self.gelu_mode]
        return {n: self._buf[n] for n in names if n in self._buf}

    def capture(self, xs, rope: torch.Tensor | None = None) -> "Graph":
        """One HIP graph of len(xs) consecutive steps, step i on input xs[i] (all of one
        M): 4 or 5 kernels' worth of calls per step, replayed with one launch
        (Graph.launch).  After a replay the buffers hold the last step's results, as
        after the same eager calls.  The inputs and this chain's buffers must stay alive
        and in place while the graph may run; the graph keeps references to them."""
        xs = list(xs)
        if not xs or any(x.shape != xs[0].shape for x in xs):
            raise ValueError("capture needs one or more step inputs of one shape")
        self.forward(xs[0], rope)    # creates the buffers outside the capture
        torch.cuda.current_stream().synchronize()

        def steps():
            for x in xs:
                self.forward(x, rope)

        return capture(steps, keep=(tuple(xs), rope, dict(self._buf)))
