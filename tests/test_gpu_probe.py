"""The dense MFMA rate probe (svdq_mfma_probe) runs every instruction type on the GPU,
leaves finite values in its sink, and measures a rate within reach of the published
dense peak of its type (a sanity range: the probe's own figure is what the bench
reports)."""

import math

import pytest
import torch

import w4a4_rank_corrected_linear_amd as svdq

pytestmark = pytest.mark.gpu

PUBLISHED = {"fp6": 10100.0, "fp4": 10100.0, "fp8": 5000.0, "int8": 5000.0, "fp16": 2500.0,
             "bf16": 2500.0, "bf16_k8": 2500.0}


@pytest.mark.parametrize("op", sorted(svdq.MFMA_OPS))
def test_mfma_probe_runs_at_a_plausible_rate(op):
    sink, ops = svdq.mfma_probe(op, 64)
    torch.cuda.synchronize()
    assert torch.isfinite(sink).all()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    _, ops = svdq.mfma_probe(op, 1024, sink)
    e1.record()
    e1.synchronize()
    rate = ops / (e0.elapsed_time(e1) * 1e-3) / 1e12
    assert math.isfinite(rate) and 0.1 * PUBLISHED[op] < rate < 1.15 * PUBLISHED[op], rate
