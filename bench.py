"""Throughput of the svdq_w4a4 int4 linear on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload attn_proj]
                    [--no-cpu-baseline] [--copy-probe]

One step is one svdq_w4a4_linear call (quantize kernel + GEMM kernel) on a resident
batch: X bf16 [M, K] -> Y bf16 [M, N].  The default workload is the DiT attention
projection of a 1024x1024 image: M = 4096 tokens, K = N = 3072, int4 group 64,
rank 32.  Inputs are seeded synthetic data; the layer's weights are seeded bytes in
the prepared int4 layout (codes in -7..7, bf16 scales, smoothing, low-rank factors,
bias), since weight preparation is an offline step outside the timed call.

Prints one JSON line:
  value        effective TOPS = 2 M N K / (wall time per call), from W untimed and
               K timed calls bracketed by device synchronizations
  roofline     for the GEMM kernel: 2 M N K / its mean duration, from HIP events
               recorded on the launch stream during the timed calls, against the
               dense peak of the MFMA data type it issues (FP6, 10.1 PFLOP/s);
               `traffic` is the HBM bytes per launch from the FETCH_SIZE / WRITE_SIZE
               counter runs recorded under profiles/, or null if the GEMM source has
               changed since they were taken
  cpu_baseline the CPU oracle on the same inputs (full call, repeated for about
               10-30 s), on the host's cores
  clock_settle before the W warmup steps, the same step runs untimed for --settle-ms
               (200 ms by default): from an idle GPU the clocks take about 20-25 ms
               of sustained load to ramp up, and the first calls run up to 25 %
               slower; the first and last batches' times are reported
"""

from __future__ import annotations

import argparse
import hashlib
import itertools
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A4 linear effective TOPS at M=4096,K=N=3072 (+% MFMA peak)"
PEAK_FP6_TFLOPS = 10100.0   # MI355X dense FP6/FP4 MFMA
PEAK_INT8_TOPS = 5000.0     # MI355X dense int8 MFMA
PEAK_HBM_GBS = 8000.0
COLD_SETS = 5                # rotating operand sets of the cold-cache pass (> 256 MB in all)
WEIGHTS_COLD_BYTES = 320e6   # layer weights rotated by the weights-cold pass (> 256 MB)
SETTLE_MS = 200.0            # untimed sustained load before the warmup steps (clock ramp)

WORKLOADS = {
    # name: (method, config id, M, K, N, rank)
    "attn_proj": ("int4", 2, 4096, 3072, 3072, 32),
    "qkv": ("int4", 3, 4608, 3072, 9216, 32),
    "mlp_up": ("int4", 3, 4608, 3072, 12288, 32),
    "mlp_down": ("int4", 3, 4608, 12288, 3072, 32),
    "out_proj": ("int4", 3, 4608, 3072, 3072, 32),   # the block's attention output projection
    "nvfp4_sq": ("nvfp4", 4, 4096, 3072, 3072, 32),
    "nvfp4_up": ("nvfp4", 4, 4096, 3072, 12288, 32),
    "awq_sq": ("awq", 4, 4096, 3072, 3072, 0),
    "awq_up": ("awq", 4, 4096, 3072, 12288, 0),
}
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA

# Workloads with committed counter summaries: (K1 kernel, GEMM kernel, GEMM sources whose
# hash stamps the summary, the summaries' base names)
PROFILED = {
    "attn_proj": ("k1_int4_fused", "k2_gemm_int4",
                  ["w4a4_rank_corrected_linear_amd/csrc/k2_gemm_int4.hip",
                   "w4a4_rank_corrected_linear_amd/csrc/common.h"],
                  "svdq_w4a4_int4_attn_proj", "k2_gemm_int4_attn_proj"),
    "nvfp4_sq": ("k1_nvfp4_fused", "k2_gemm_fp4",
                 ["w4a4_rank_corrected_linear_amd/csrc/k2_gemm_fp4.hip",
                  "w4a4_rank_corrected_linear_amd/csrc/k2_common.h",
                  "w4a4_rank_corrected_linear_amd/csrc/common.h"],
                 "svdq_w4a4_nvfp4_sq", "k2_gemm_fp4_nvfp4_sq"),
    # the AWQ W4A16 layer is one kernel (no quantizer)
    "awq_sq": (None, "k4_gemm_awq",
               ["w4a4_rank_corrected_linear_amd/csrc/k4_gemm_awq.hip",
                "w4a4_rank_corrected_linear_amd/csrc/k2_common.h",
                "w4a4_rank_corrected_linear_amd/csrc/common.h"],
               "awq_w4a16_sq", "k4_gemm_awq_awq_sq"),
}


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"{PROFILED[workload][4]}_traffic.txt")


def gemm_source_hash(workload: str = "attn_proj") -> str:
    h = hashlib.sha256()
    for p in PROFILED[workload][2]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str):
    """HBM bytes per GEMM launch from the committed counter summary, or None."""
    if workload not in PROFILED or not os.path.exists(traffic_file(workload)):
        return None
    kv = {}
    with open(traffic_file(workload)) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("gemm_source_sha256_16") != gemm_source_hash(workload):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def make_inputs(workload: str):
    from synth import inputs as I
    method, cid, M, K, N, rank = WORKLOADS[workload]
    sd = I.seeds(cid)
    idx = I.outlier_channels(K, I.default_outlier_count(K), sd.outliers)
    x = I.activations(M, K, sd.x, idx, 30.0)
    if method == "int4":
        pb = I.prepared_int4_bytes(cid, K, N, rank)
    elif method == "nvfp4":
        pb = I.prepared_nvfp4_bytes(cid, K, N, rank)
    else:
        pb = I.prepared_awq_bytes(cid, K, N)
    return dict(method=method, M=M, K=K, N=N, rank=rank, x=x, pb=pb,
                seeds=dict(x=sd.x, w=sd.w, bias=sd.bias, outliers=sd.outliers))


def _threads() -> int:
    """BLAS threads the oracle runs with (the CPU baseline's core count)."""
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:
        return int(os.cpu_count() or 1)


def cpu_baseline(inp, min_seconds: float = 10.0, max_reps: int = 8):
    """The oracle on the same inputs, timed on the host (test infrastructure)."""
    from oracle import linear as OL
    from oracle import prep as P
    pb, method = inp["pb"], inp["method"]
    if method == "awq":
        layer = P.AwqLayer(K=pb.K, N=pb.N, group=64, qweight=pb.qweight, scales=pb.scales,
                           zeros=pb.zeros, bias=pb.bias)
        run = lambda: OL.awq_w4a16_linear(inp["x"], layer)  # noqa: E731
    else:
        wg = getattr(pb, "w_global", 1.0)
        ag = getattr(pb, "act_global", 1.0)
        layer = P.SvdqLayer(precision=method, K=pb.K, N=pb.N, rank=pb.rank, qweight=pb.qweight,
                            wscales=pb.wscales, w_global=wg, act_global=ag, smooth=pb.smooth,
                            lora_down=pb.lora_down, lora_up=pb.lora_up, bias=pb.bias)
        run = lambda: OL.w4a4_linear(method, inp["x"], layer)  # noqa: E731
    M, K, N = inp["M"], inp["K"], inp["N"]
    times = []
    t_all = time.perf_counter()
    while len(times) < 2 or (time.perf_counter() - t_all < min_seconds and len(times) < max_reps):
        t0 = time.perf_counter()
        run()
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    return {"value": round(2.0 * M * N * K / t / 1e12, 6), "unit": "TOPS", "cores": _threads(),
            "kind": "oracle",
            "sample": f"full {M}x{K}x{N} call on the same inputs, {len(times)} runs, median "
                      f"{t:.3f} s (float64 numpy/BLAS)"}


def clock_settle(step, ms: float, per_batch: int) -> dict | None:
    """Runs `step` untimed in batches of `per_batch` (synchronized) until `ms` of wall
    time have passed, so that the timed steps start at the clocks sustained load runs
    at; returns the settle time, the step count and the first and last batches' times
    per step, or None when ms <= 0."""
    import torch
    if ms <= 0:
        return None
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    n, batches = 0, []
    while True:
        t0 = time.perf_counter()
        for _ in range(per_batch):
            step()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        n += per_batch
        batches.append((t1 - t0) * 1e3 / per_batch)
        if (t1 - t_start) * 1e3 >= ms:
            break
    out = {"ms": round((t1 - t_start) * 1e3, 1), "steps": n,
           "ms_per_step_first_batch": round(batches[0], 6),
           "ms_per_step_last_batch": round(batches[-1], 6)}
    print(f"[bench] clock settle: {n} untimed steps in {out['ms']} ms, "
          f"{out['ms_per_step_first_batch']} ms per step in the first batch, "
          f"{out['ms_per_step_last_batch']} in the last", file=sys.stderr, flush=True)
    return out


def run_chain(args) -> int:
    """One DiT block's four W4A4 linears and the GELU per denoise step (config 5): the
    steps cycle through 8 fresh seeded inputs resident in HBM; K timed steps, then an
    instrumented pass with an event pair around every call for the per-layer times."""
    import numpy as np
    import torch
    import w4a4_rank_corrected_linear_amd as svdq
    from synth import inputs as I

    dev = torch.device("cuda:0")
    M = 4608 * args.batch

    def bf16(bits):
        t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
        return t.view(torch.bfloat16).to(dev)

    def u8(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(dev)

    pbs = I.chain_layer_bytes()
    lay = {k: svdq.SvdqLinear.from_interchange(u8(pb.qweight), bf16(pb.wscales), bf16(pb.smooth),
                                               bf16(pb.lora_down), bf16(pb.lora_up), bf16(pb.bias))
           for k, pb in pbs.items()}
    qk_norm, rope = None, None
    if args.qkv_norm_rope:
        nq, nk = (bf16(b) for b in I.qk_norm_weights())
        qk_norm = (nq, nk, I.QK_NORM_EPS)
        rope = torch.from_numpy(I.rope_table(M)).to(dev)
    chain = svdq.DitBlockChain(lay["qkv"], lay["out"], lay["up"], lay["down"],
                               fuse_gelu="down" if args.gelu_down else args.fuse_gelu, qk_norm=qk_norm,
                               fuse_qk=not args.qk_separate)
    xs = [bf16(I.chain_step_activations(M, s)) for s in range(8)]
    print(f"[bench] workload chain: DiT block (QKV, out, MLP-up, GELU, MLP-down), M={M}, 8 fresh "
          f"step inputs; warmup {args.warmup}, steps {args.steps}", file=sys.stderr, flush=True)
    settle_i = itertools.count()
    settle = clock_settle(lambda: chain(xs[next(settle_i) % 8], rope), args.settle_ms, 2)
    for i in range(args.warmup):
        chain(xs[i % 8], rope)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        chain(xs[i % 8], rope)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    eager_ms = wall * 1e3 / args.steps
    graph_info = None
    if args.graph:
        # the 8 steps recorded once into one HIP graph, replayed ceil(K/8) times
        g = chain.capture(xs, rope)
        reps = -(-args.steps // 8)
        for _ in range(-(-args.warmup // 8)):
            g.launch()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            g.launch()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * args.steps / (8 * reps)
        # host time to enqueue 8 steps: the calls one by one against one graph launch
        # (median of 5, from an idle queue)
        host_e, host_g = [], []
        for _ in range(5):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for x in xs:
                chain(x, rope)
            host_e.append(time.perf_counter() - t0)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            g.launch()
            host_g.append(time.perf_counter() - t0)
        torch.cuda.synchronize()
        g.destroy()
        graph_info = {"replays": reps, "steps_per_replay": 8, "eager_ms_per_step": round(eager_ms, 6),
                      "host_enqueue_us_per_step": {
                          "eager": round(sorted(host_e)[2] * 1e6 / 8, 1),
                          "graph": round(sorted(host_g)[2] * 1e6 / 8, 1)}}

    # per-layer times: events around each call on the current stream (they include the
    # dispatch of the call's kernels)
    names = ["qkv"] + (["qk_norm_rope"] if args.qkv_norm_rope and args.qk_separate else []) + (
        ["out", "up", "down"] if (args.fuse_gelu or args.gelu_down) else ["out", "up", "gelu", "down"])
    n_inst = min(args.steps, 200)
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in names] for _ in range(n_inst)]
    ws = torch.empty(max(l.workspace_bytes(M) for l in lay.values()), dtype=torch.uint8, device=dev)
    bufs = {"qkv": torch.empty((M, lay["qkv"].N), dtype=torch.bfloat16, device=dev),
            "out": torch.empty((M, lay["out"].N), dtype=torch.bfloat16, device=dev),
            "up": torch.empty((M, lay["up"].N), dtype=torch.bfloat16, device=dev),
            "act": torch.empty((M, lay["up"].N), dtype=torch.bfloat16, device=dev),
            "down": torch.empty((M, lay["down"].N), dtype=torch.bfloat16, device=dev)}
    sep = bool(qk_norm) and args.qk_separate
    calls = [(lambda x: lay["qkv"].qkv_norm_rope(x, *qk_norm[:2], qk_norm[2], rope, out=bufs["qkv"],
                                                 workspace=ws)) if qk_norm and not sep else
             (lambda x: lay["qkv"](x, out=bufs["qkv"], workspace=ws))]
    if sep:
        calls.append(lambda x: svdq.qk_norm_rope(bufs["qkv"], *qk_norm[:2], qk_norm[2], rope,
                                                 out=bufs["qkv"]))
    calls += [
             lambda x: lay["out"](x, out=bufs["out"], workspace=ws)]
    if args.fuse_gelu:
        calls.append(lambda x: lay["up"](bufs["out"], out=bufs["act"], workspace=ws, gelu=True))
    elif args.gelu_down:
        calls.append(lambda x: lay["up"](bufs["out"], out=bufs["up"], workspace=ws))
    else:
        calls += [lambda x: lay["up"](bufs["out"], out=bufs["up"], workspace=ws),
                  lambda x: svdq.gelu(bufs["up"], out=bufs["act"])]
    if args.gelu_down:
        calls.append(lambda x: lay["down"](bufs["up"], out=bufs["down"], workspace=ws, gelu_in=True))
    else:
        calls.append(lambda x: lay["down"](bufs["act"], out=bufs["down"], workspace=ws))
    for i in range(n_inst):
        for j, c in enumerate(calls):
            ev[i][j][0].record()
            c(xs[i % 8])
            ev[i][j][1].record()
    torch.cuda.synchronize()
    per = {n: sum(ev[i][j][0].elapsed_time(ev[i][j][1]) for i in range(n_inst)) / n_inst
           for j, n in enumerate(names)}

    shapes = {n: (K, N) for n, K, N in I.CHAIN_LAYERS}
    ops_step = sum(2.0 * M * K * N for K, N in shapes.values())
    ms_per_step = wall * 1e3 / args.steps
    value = ops_step / (ms_per_step * 1e-3) / 1e12
    layers = {n: {"ms": round(per[n], 6),
                  **({"TOPS": round(2.0 * M * shapes[n][0] * shapes[n][1] / (per[n] * 1e-3) / 1e12, 3)}
                     if n in shapes else {"GBps": round(
                         (4.0 * M * shapes["up"][1] if n == "gelu" else
                          4.0 * M * shapes["qkv"][1] * 2 / 3 + M * 512) / (per[n] * 1e-3) / 1e9, 1)})}
              for n in names}
    out = {
        "metric": f"DiT block chain of svdq_w4a4 int4 linears (QKV, out, MLP-up, GELU, MLP-down) "
                  f"effective TOPS at M={M}" + (", GELU fused into MLP-up" if args.fuse_gelu else "")
                  + (", GELU fused into MLP-down's quantizer" if args.gelu_down else "")
                  + ((", Q/K norm + rotary as a separate pass" if args.qk_separate else
                      ", Q/K norm + rotary fused into QKV") if args.qkv_norm_rope else "")
                  + (", 8 steps per HIP graph" if args.graph else ""),
        "value": round(value, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle": settle,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4",
        "data": "synthetic",
        "config": {"workload": f"chain: DiT block, batch {args.batch} (M={M}), 8 fresh step inputs "
                               "cycled, int4 g64 rank 32" + (", GELU in the MLP-up epilogue"
                                                             if args.fuse_gelu else "")
                               + (", GELU in MLP-down's quantizer" if args.gelu_down else "")
                               + (", 8 steps per HIP graph replay" if args.graph else "")
                               + (", Q/K RMSNorm + rotary in the QKV epilogue"
                                  if args.qkv_norm_rope else ""),
                   "M": M, "layers": {n: {"K": K, "N": N} for n, (K, N) in shapes.items()},
                   "seeds": {"steps": [I.seeds(I.CHAIN_CONFIG).step(s) for s in range(8)]}},
        "chain_8_steps_ms": round(8 * ms_per_step, 6),
        "layers": layers,
        "sum_of_call_ms": round(sum(per.values()), 6),
        **({"graph": graph_info} if graph_info else {}),
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)
    return 0


def run_prep(args) -> int:
    """Offline int4 weight preparation on the GPU (svdq_prepare_weight) of the attention
    projection's weight (K = N = 3072, rank 32, 16 oversampling columns, 8 power
    iterations, 4096 calibration rows), timed per call; with the CPU baseline, the
    oracle's preparation (exact float64 SVD) on the same inputs, and the ratio of the
    two residual norms."""
    import ctypes
    import numpy as np
    import torch
    import w4a4_rank_corrected_linear_amd as svdq
    from synth import inputs as I

    K = N = 3072
    rank, over, iters = 32, 16, 8
    li = I.layer_inputs(config_id=2, M=16, K=K, N=N, cal_rows=4096)
    dev = torch.device("cuda:0")
    L = svdq.lib()
    w = torch.from_numpy(np.ascontiguousarray(li.w, np.float32)).to(dev)
    xc = torch.from_numpy(li.x_cal.view(np.int16)).view(torch.bfloat16).to(dev)
    om = torch.from_numpy(I.gaussian_test_matrix(N, rank + over, 7)).to(dev)
    qw = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    sc = torch.empty((N, K // 64), dtype=torch.bfloat16, device=dev)
    sm = torch.empty((K,), dtype=torch.bfloat16, device=dev)
    ld = torch.empty((rank, K), dtype=torch.bfloat16, device=dev)
    lu = torch.empty((N, rank), dtype=torch.bfloat16, device=dev)
    res = torch.empty((K, N), dtype=torch.float32, device=dev)
    nbytes = L.svdq_prepare_workspace_bytes(K, N, rank, over)
    work = torch.empty((nbytes,), dtype=torch.uint8, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    cfg = svdq._lib.config("int4", rank)

    def call():
        svdq._lib.check(L.svdq_prepare_weight(ctypes.byref(cfg), K, N, w.data_ptr(), xc.data_ptr(),
                                              4096, om.data_ptr(), over, iters, qw.data_ptr(),
                                              sc.data_ptr(), sm.data_ptr(), ld.data_ptr(),
                                              lu.data_ptr(), res.data_ptr(), None, None,
                                              work.data_ptr(), nbytes, stream),
                        "svdq_prepare_weight")

    steps, warmup = min(args.steps, 20), min(args.warmup, 3)
    print(f"[bench] workload prep: K=N={K}, rank {rank}, oversample {over}, {iters} power "
          f"iterations; warmup {warmup}, steps {steps}", file=sys.stderr, flush=True)
    settle = clock_settle(call, args.settle_ms, 1)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    ell = rank + over
    # float64 work of the factorization: 2 K N l per product with What, (2 iters + 2) of them
    flops = 2.0 * K * N * ell * (2 * iters + 2)
    out = {
        "metric": f"GPU int4 weight preparation (smoothing, rank-{rank} factorization, residual "
                  f"quantization) time at K=N={K}",
        "value": round(ms, 3),
        "unit": "ms",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "clock_settle": settle,
        "ms_per_step": round(ms, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": f"prep: W [{K}, {N}] ~ N(0, 0.02), X_cal [4096, {K}] with 1 % "
                               f"outlier channels x30, rank {rank}, l = {ell}, {iters} power "
                               "iterations", "K": K, "N": N, "rank": rank, "oversample": over,
                   "power_iters": iters},
        "factorization_f64_GFLOPs": round(flops / (ms * 1e-3) / 1e9, 1),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from oracle import prep as P
        t0 = time.perf_counter()
        ref = P.prepare_svdq(li.w, li.x_cal, li.bias, rank=rank)
        cpu_s = time.perf_counter() - t0
        ratio = float(np.linalg.norm(res.cpu().numpy()) / np.linalg.norm(ref.residual))
        out["residual_norm_ratio_vs_exact_svd"] = round(ratio, 6)
        out["cpu_baseline"] = {"value": round(cpu_s * 1e3, 1), "unit": "ms", "cores": _threads(),
                               "kind": "oracle",
                               "sample": "one oracle preparation (float64 numpy SVD) of the same "
                                         "weight"}
    print(json.dumps(out), flush=True)
    return 0


PROFILE_CMDS = {
    "stats": "cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -d <out>/prof_stats "
             "-o run --output-format csv -- python3 <repo>/bench.py --workload {w} --no-cpu-baseline "
             "--no-cold",
    "fetch": "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc FETCH_SIZE -d <out>/pmc_fetch -o run "
             "--output-format csv -- python3 <repo>/bench.py --workload {w} --no-cpu-baseline "
             "--no-cold --steps 20 --warmup 5 --copy-probe",
    "write": "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc WRITE_SIZE -d <out>/pmc_write -o run "
             "--output-format csv -- python3 <repo>/bench.py --workload {w} --no-cpu-baseline "
             "--no-cold --steps 20 --warmup 5 --copy-probe",
}


# published dense peaks (TFLOP/s or TOP/s) of the probe's instruction types
MFMA_PUBLISHED = {"fp6": 10100.0, "fp4": 10100.0, "fp8": 5000.0, "int8": 5000.0, "fp16": 2500.0,
                  "bf16": 2500.0, "bf16_k8": 2500.0}


def mfma_achievable(iters: int = 2048, reps: int = 3) -> dict:
    """The dense rate the matrix cores sustain per instruction type (svdq_mfma_probe:
    every CU, two waves per SIMD, four independent MFMAs per round), timed with HIP
    events on the launching stream: the median of `reps` launches after one warm-up."""
    import torch

    import w4a4_rank_corrected_linear_amd as svdq
    out = {}
    sink = None
    for op in svdq.MFMA_OPS:
        sink, ops = svdq.mfma_probe(op, iters, sink)
        ms = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            svdq.mfma_probe(op, iters, sink)
            e1.record()
            e1.synchronize()
            ms.append(e0.elapsed_time(e1))
        t = sorted(ms)[len(ms) // 2]
        rate = ops / (t * 1e-3) / 1e12
        out[op] = {"tflops": round(rate, 1), "published": MFMA_PUBLISHED[op],
                   "frac_of_published": round(rate / MFMA_PUBLISHED[op], 4)}
    return out


def summarize_stats(csv_dir: str, name: str, command: str, what: str) -> None:
    """One rocprofv3 --kernel-trace --stats run (CSV under csv_dir) as a text summary
    profiles/<name>_kernel_stats.txt: the kernel table with the command that made it
    (host only, no GPU)."""
    import csv
    import glob
    files = glob.glob(os.path.join(csv_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(os.path.join(csv_dir, "**/*kernel_stats.csv"))
    lines = [f"# rocprofv3 kernel statistics: {what}",
             f"# command: {command}",
             "# kernel                                        calls     avg_us     min_us     max_us   share_%"]
    for r in csv.DictReader(open(files[0])):
        nm = r["Name"].replace("(anonymous namespace)::", "")
        nm = nm[: nm.index("(")] if "(" in nm else nm
        lines.append(f"{nm[:46]:46s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.3f} "
                     f"{float(r['MinNs']) / 1e3:10.3f} {float(r['MaxNs']) / 1e3:10.3f} "
                     f"{float(r['Percentage']):8.2f}")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"{name}_kernel_stats.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def svdq_mfma_ops():
    """Names of the probe's instruction types in op order (host only: no GPU)."""
    return {"fp6": 0, "fp4": 1, "fp8": 2, "int8": 3, "fp16": 4, "bf16": 5, "bf16_k8": 6}


def summarize_profiles(out_dir: str, workload: str = "attn_proj") -> None:
    """Turn the CSV output of the three rocprofv3 runs in PROFILE_CMDS (under
    out_dir) into the text summaries kept under profiles/ (host only, no GPU)."""
    import csv
    import glob

    k1_name, k2_name, _, stats_base, _ = PROFILED[workload]

    def one(pattern):
        files = glob.glob(os.path.join(out_dir, pattern), recursive=True)
        if not files:
            raise FileNotFoundError(os.path.join(out_dir, pattern))
        return files[0]

    def short(name):
        for key in (k1_name, k2_name, "MulFunctor", "FillFunctor", "k_pack_int4", "k_pack_nvfp4",
                    "k_pack_lora_down", "k_pair_scales", "k_zero_flag", "copyBuffer"):
            if key and key in name:
                return key
        if "k_mfma_probe<" in name:   # the achievable-rate probe, by instruction type
            op = int(name.split("k_mfma_probe<")[1].split(">")[0])
            return "k_mfma_probe " + list(svdq_mfma_ops())[op]
        return name[:40]

    method, cid, M, K, N, rank = WORKLOADS[workload]
    desc = {"int4": "int4 g64", "nvfp4": "nvfp4 g16", "awq": "awq_w4a16 int4 g64"}[method]
    cmds = {k: v.format(w=workload) for k, v in PROFILE_CMDS.items()}
    lines = [f"# rocprofv3 kernel statistics: bench.py, workload {workload} "
             f"(M={M} K={K} N={N} rank {rank}, {desc}), 200 ms untimed clock settle, 50 warmup + "
             f"500 timed + 500 event-timed calls",
             f"# command: {cmds['stats']}",
             "# kernel                      calls     avg_us     min_us     max_us   share_%"]
    for r in csv.DictReader(open(one("prof_stats/**/*kernel_stats.csv"))):
        lines.append(f"{short(r['Name']):28s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.3f} "
                     f"{float(r['MinNs']) / 1e3:10.3f} {float(r['MaxNs']) / 1e3:10.3f} "
                     f"{float(r['Percentage']):8.2f}")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"{stats_base}_kernel_stats.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")

    per = {}
    for tag, counter in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        acc = {}
        for r in csv.DictReader(open(one(f"pmc_{tag}/**/*counter_collection.csv"))):
            if r["Counter_Name"] != counter:
                continue
            acc.setdefault(short(r["Kernel_Name"]), {}).setdefault(r["Dispatch_Id"], 0.0)
            acc[short(r["Kernel_Name"])][r["Dispatch_Id"]] += float(r["Counter_Value"])
        per[tag] = {k: sum(v.values()) / len(v) for k, v in acc.items()}   # KiB per dispatch
    copy_bytes = 256.0 * 1024 * 1024
    f_fetch = per["fetch"]["MulFunctor"] * 1024 / copy_bytes
    f_write = per["write"]["MulFunctor"] * 1024 / copy_bytes
    k2_traffic = per["fetch"][k2_name] * 1024 / f_fetch + per["write"][k2_name] * 1024 / f_write
    k1_traffic = (per["fetch"][k1_name] * 1024 / f_fetch + per["write"][k1_name] * 1024 / f_write
                  if k1_name else None)
    t = [f"# HBM traffic per dispatch from rocprofv3 counters, workload {workload} "
         f"(M={M} K={K} N={N} rank {rank}, {desc})",
         f"# fetch command: {cmds['fetch']}",
         f"# write command: {cmds['write']}",
         "# scale: the copy probe (elementwise multiply, float32, 256 MiB read + 256 MiB write)",
         "# reads FETCH_SIZE = copy_fetch_KiB and WRITE_SIZE = copy_write_KiB; bytes = counter KiB",
         "# * 1024 / factor, factor = counter bytes of the probe / 256 MiB",
         f"copy_fetch_KiB = {per['fetch']['MulFunctor']:.1f}",
         f"copy_write_KiB = {per['write']['MulFunctor']:.1f}",
         f"fetch_factor = {f_fetch:.4f}",
         f"write_factor = {f_write:.4f}"]
    for k in (k1_name, k2_name):
        if k:
            t.append(f"{k}_fetch_KiB = {per['fetch'][k]:.1f}")
            t.append(f"{k}_write_KiB = {per['write'][k]:.1f}")
    if k1_traffic is not None:
        t.append(f"k1_traffic_bytes_per_launch = {k1_traffic:.0f}")
    t += [f"traffic_bytes_per_launch = {k2_traffic:.0f}",
          f"gemm_source_sha256_16 = {gemm_source_hash(workload)}"]
    with open(traffic_file(workload), "w") as f:
        f.write("\n".join(t) + "\n")
    print("\n".join(lines + t))


def summarize_counters(name: str, what: str, *runs: str) -> None:
    """rocprofv3 --pmc runs (each given as "<csv_dir>=<command>") as one text summary
    profiles/<name>_counters.txt: per kernel, the mean of every counter per dispatch,
    and derived figures (host only, no GPU).  SQ_BUSY_CYCLES is summed over the chip's
    32 shader engines, so SQ_BUSY_CYCLES / 32 is the kernel's duration in cycles
    (GRBM_GUI_ACTIVE spans the profiler's serialized dispatch, not the kernel alone);
    SQ_VALU_MFMA_BUSY_CYCLES and SQ_VALU_MFMA_COEXEC_CYCLES are per-SIMD counts summed
    over the 1024 SIMDs, so the MFMA-busy fraction is busy / 1024 / kernel cycles, and
    the co-exec share is the part of the MFMA-busy cycles in which the SIMD also
    executed VALU work."""
    import csv
    import glob
    simds, engines = 1024, 32
    per = {}      # kernel -> counter -> [values per dispatch]
    cmds = []
    for run in runs:
        d, cmd = run.split("=", 1)
        cmds.append(cmd)
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise FileNotFoundError(os.path.join(d, "**/*counter_collection.csv"))
        acc = {}
        for r in csv.DictReader(open(files[0])):
            nm = r["Kernel_Name"].replace("(anonymous namespace)::", "")
            nm = nm[: nm.index("(")] if "(" in nm else nm
            nm = nm.replace("void ", "").replace("svdq::", "")
            key = (nm, r["Counter_Name"], r["Dispatch_Id"])
            acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
        for (nm, c, _), v in acc.items():
            per.setdefault(nm, {}).setdefault(c, []).append(v)
    lines = [f"# rocprofv3 hardware counters: {what}"]
    lines += [f"# command: {c}" for c in cmds]
    lines.append(f"# summary: python bench.py --summarize-counters {name} <what> <csv_dir>=<command> ...")
    wl = next((w for w, v in PROFILED.items() if v[4] == name), "attn_proj")
    lines.append(f"# gemm_source_sha256_16 = {gemm_source_hash(wl)}")
    for nm in sorted(per, key=lambda k: -max(len(v) for v in per[k].values())):
        cs = per[nm]
        n = max(len(v) for v in cs.values())
        if n < 5:
            continue
        lines.append(f"[{nm}]  dispatches {n}")
        mean = {c: sum(v) / len(v) for c, v in cs.items()}
        for c in sorted(mean):
            lines.append(f"  {c} = {mean[c]:.1f}")
        kc = mean.get("SQ_BUSY_CYCLES", 0.0) / engines
        if kc > 0:
            lines.append(f"  kernel_cycles = {kc:.0f}")
        if kc > 0 and "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
            busy = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / simds
            lines.append(f"  mfma_busy_cycles_per_simd = {busy:.0f}")
            lines.append(f"  mfma_busy_fraction = {busy / kc:.3f}")
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in mean and mean.get("SQ_VALU_MFMA_BUSY_CYCLES"):
            lines.append(f"  coexec_share_of_mfma_busy = "
                         f"{mean['SQ_VALU_MFMA_COEXEC_CYCLES'] / mean['SQ_VALU_MFMA_BUSY_CYCLES']:.3f}")
        if mean.get("SQ_INSTS_LDS") and "SQ_LDS_BANK_CONFLICT" in mean:
            lines.append(f"  lds_bank_conflict_cycles_per_lds_inst = "
                         f"{mean['SQ_LDS_BANK_CONFLICT'] / mean['SQ_INSTS_LDS']:.3f}")
        if mean.get("SQ_INSTS_VALU"):
            lines.append(f"  valu_insts_per_simd = {mean['SQ_INSTS_VALU'] / simds:.0f}")
            if mean.get("SQ_INSTS_MFMA"):
                lines.append(f"  valu_insts_per_mfma = {mean['SQ_INSTS_VALU'] / mean['SQ_INSTS_MFMA']:.2f}")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"{name}_counters.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))

def cold_cache_pass(args, inp, layer_args, M: int, N: int, K: int, dev) -> dict:
    """The same call over COLD_SETS rotating sets of layer weights, X, Y and workspace
    (more bytes in total than the 256 MB Infinity Cache, so each call finds its
    operands in HBM, not in a cache), timed like the headline."""
    import torch
    import w4a4_rank_corrected_linear_amd as svdq

    sets = []
    for _ in range(COLD_SETS):
        la, kw = layer_args()
        lay = svdq.SvdqLinear.from_interchange(*la, **kw)
        x = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        x.view(torch.int16).copy_(torch.from_numpy(inp["x"].view("int16")).to(dev))
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(lay.workspace_bytes(M), dtype=torch.uint8, device=dev)
        sets.append((lay, x, y, ws))
    per_set = sum(t.numel() * t.element_size() for t in
                  (sets[0][0].qweight, sets[0][0].wscales, sets[0][0].smooth, sets[0][0].lora_down,
                   sets[0][0].lora_up, sets[0][0].bias, sets[0][1], sets[0][2], sets[0][3]))
    steps = min(args.steps, 200)
    for i in range(2 * COLD_SETS):
        lay, x, y, ws = sets[i % COLD_SETS]
        lay(x, out=y, workspace=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        lay, x, y, ws = sets[i % COLD_SETS]
        lay(x, out=y, workspace=ws)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = wall * 1e3 / steps
    print(f"[bench] cold-cache pass: {steps} calls over {COLD_SETS} sets of {per_set / 1e6:.1f} MB",
          file=sys.stderr, flush=True)
    # the same rotation once more with per-kernel events (quantizer, GEMM)
    svdq.timing_start(steps)
    for i in range(steps):
        lay, x, y, ws = sets[i % COLD_SETS]
        lay(x, out=y, workspace=ws)
    torch.cuda.synchronize()
    _, kms = svdq.timing_stop(4)
    x0, y0, ws0 = sets[0][1], sets[0][2], sets[0][3]
    del sets
    out = {"ms_per_step": round(ms, 6), "TOPS": round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 3),
           "sets": COLD_SETS, "bytes_per_set": per_set, "steps": steps,
           "kernels_ms": {"quantize": round(kms[0], 6), "gemm": round(kms[1], 6)} if len(kms) >= 2 else None}

    # Weights cold, activations warm (a layer inside a model: its input was just
    # written, its weights were last read a whole forward pass ago): one X, Y and
    # workspace, the call rotating over enough copies of the layer that their weights
    # exceed the Infinity Cache.
    layers = []
    w_bytes = 0
    while w_bytes < WEIGHTS_COLD_BYTES:
        la, kw = layer_args()
        lay = svdq.SvdqLinear.from_interchange(*la, **kw)
        layers.append(lay)
        w_bytes += sum(t.numel() * t.element_size() for t in
                       (lay.qweight, lay.wscales, lay.smooth, lay.lora_down, lay.lora_up, lay.bias)
                       if t is not None)
    for i in range(len(layers)):
        layers[i](x0, out=y0, workspace=ws0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        layers[i % len(layers)](x0, out=y0, workspace=ws0)
    torch.cuda.synchronize()
    wms = (time.perf_counter() - t0) * 1e3 / steps
    svdq.timing_start(steps)
    for i in range(steps):
        layers[i % len(layers)](x0, out=y0, workspace=ws0)
    torch.cuda.synchronize()
    _, wkms = svdq.timing_stop(4)
    print(f"[bench] weights-cold pass: {steps} calls over {len(layers)} layers "
          f"({w_bytes / 1e6:.0f} MB of weights), one X", file=sys.stderr, flush=True)
    n_layers = len(layers)
    del layers
    out["weights_cold"] = {
        "ms_per_step": round(wms, 6), "TOPS": round(2.0 * M * N * K / (wms * 1e-3) / 1e12, 3),
        "layers": n_layers, "weight_bytes_rotated": w_bytes, "steps": steps,
        "kernels_ms": {"quantize": round(wkms[0], 6), "gemm": round(wkms[1], 6)} if len(wkms) >= 2 else None}
    return out


def main() -> int:
    if len(sys.argv) in (3, 4) and sys.argv[1] == "--summarize-profiles":
        summarize_profiles(*sys.argv[2:4])
        return 0
    if len(sys.argv) == 6 and sys.argv[1] == "--summarize-stats":
        summarize_stats(*sys.argv[2:6])
        return 0
    if len(sys.argv) >= 5 and sys.argv[1] == "--summarize-counters":
        summarize_counters(*sys.argv[2:])
        return 0
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="untimed sustained load before the warmup steps (0: none)")
    ap.add_argument("--workload", default="attn_proj", choices=sorted(WORKLOADS) + ["chain", "prep"])
    ap.add_argument("--batch", type=int, default=1, choices=[1, 4],
                    help="chain workload: images per step (M = 4608 per image)")
    ap.add_argument("--fuse-gelu", action="store_true",
                    help="chain workload: GELU in the MLP-up GEMM's epilogue")
    ap.add_argument("--gelu-down", action="store_true",
                    help="chain workload: GELU in MLP-down's quantizer, applied to MLP-up's bf16 "
                         "output as it is loaded (svdq_w4a4_linear_gelu_in)")
    ap.add_argument("--graph", action="store_true",
                    help="chain: record the 8 steps into one HIP graph and time its replays")
    ap.add_argument("--qkv-norm-rope", action="store_true",
                    help="qkv and chain workloads: the fused QKV epilogue with per-head Q/K RMSNorm and the "
                         "rotary embedding (1024x1024 DiT table)")
    ap.add_argument("--qk-separate", action="store_true",
                    help="chain with --qkv-norm-rope: the Q/K norm + rotary as a separate pass "
                         "over the bf16 QKV output instead of the fused epilogue")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache pass (rotating sets larger than the Infinity Cache)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 256 MiB device copy (scale reference for HBM counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the layer shards by tokens with no exchange, run one process per GPU instead",
              file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2
    if args.fuse_gelu and args.gelu_down:
        print("--fuse-gelu and --gelu-down place the one GELU in two layers: pick one", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import w4a4_rank_corrected_linear_amd as svdq

    if not torch.cuda.is_available():
        print("no GPU visible: bench.py needs a gfx950 device", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    svdq.check_device(0)
    if args.workload == "chain":
        return run_chain(args)
    if args.workload == "prep":
        return run_prep(args)
    if args.qkv_norm_rope and args.workload != "qkv":
        print("--qkv-norm-rope applies to the qkv and chain workloads only", file=sys.stderr)
        return 2

    inp = make_inputs(args.workload)
    method = inp["method"]
    M, K, N, rank = inp["M"], inp["K"], inp["N"], inp["rank"]
    pb = inp["pb"]

    def bf16(bits):
        t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
        return t.view(torch.bfloat16).to(dev)

    def u8(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(dev)

    x = bf16(inp["x"])
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    if method == "awq":
        layer = svdq.AwqLinear(u8(pb.qweight), bf16(pb.scales), u8(pb.zeros), bf16(pb.bias))
        call = lambda: layer(x, out=y)  # noqa: E731
        n_kernels = 1
    else:
        def layer_args():
            scales = bf16(pb.wscales) if method == "int4" else u8(pb.wscales)
            return ((u8(pb.qweight), scales, bf16(pb.smooth), bf16(pb.lora_down),
                     bf16(pb.lora_up), bf16(pb.bias)),
                    dict(precision=method, w_global=getattr(pb, "w_global", 1.0),
                         act_global=getattr(pb, "act_global", 1.0)))
        la, kw = layer_args()
        layer = svdq.SvdqLinear.from_interchange(*la, **kw)
        ws = layer.workspace(M, dev)
        call = lambda: layer(x, out=y, workspace=ws)  # noqa: E731
        if args.qkv_norm_rope:
            from synth import inputs as I
            nq, nk = (bf16(b) for b in I.qk_norm_weights())
            rope = torch.from_numpy(I.rope_table(M)).to(dev)
            call = lambda: layer.qkv_norm_rope(x, nq, nk, I.QK_NORM_EPS, rope, out=y,  # noqa: E731
                                               workspace=ws)
        n_kernels = 2
    print(f"[bench] workload {args.workload} ({method}) M={M} K={K} N={N} rank={rank}; warmup "
          f"{args.warmup}, steps {args.steps}", file=sys.stderr, flush=True)

    settle = clock_settle(call, args.settle_ms, 20)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()

    # The timed region: K calls, nothing else on the stream.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(f"[bench] timed {args.steps} calls in {wall:.4f} s", file=sys.stderr, flush=True)

    # Per-kernel durations: the same K calls again with the library's timing hook, which
    # launches each kernel with a start/end event pair on the kernel's own stream.  The
    # event timestamps add about 8 us per call of dispatch overhead between the kernels,
    # so this pass is kept out of the whole-call figure; the durations agree with
    # rocprofv3's kernel trace.
    svdq.timing_start(args.steps)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    wall_events = time.perf_counter() - t1
    calls, kern_ms = svdq.timing_stop()
    # an int4 GEMM whose last round of tiles is split along K adds a third kernel that
    # finishes the split tiles
    if calls != args.steps or len(kern_ms) not in (n_kernels, n_kernels + (method == "int4")):
        raise RuntimeError(f"kernel timing recorded {calls} calls / {len(kern_ms)} kernels")
    print(f"[bench] instrumented pass: {args.steps} calls in {wall_events:.4f} s", file=sys.stderr,
          flush=True)

    if args.copy_probe:
        n = 64 << 20
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        print("[bench] copy probe: 3 x elementwise 256 MiB read + 256 MiB write", file=sys.stderr,
              flush=True)

    ops = 2.0 * M * N * K
    ms_per_step = wall * 1e3 / args.steps
    value = ops / (ms_per_step * 1e-3) / 1e12
    gemm_ms = sum(kern_ms[n_kernels - 1:])     # the GEMM (and its tail kernel)
    achieved = ops / (gemm_ms * 1e-3) / 1e12
    peak = PEAK_FP6_TFLOPS if method == "int4" else PEAK_BF16_TFLOPS
    kernels = {"gemm_ms": round(gemm_ms, 6), "gemm_TOPS": round(achieved, 3),
               **({"gemm_tail_ms": round(kern_ms[-1], 6)} if len(kern_ms) > n_kernels else {}),
               "ms_per_call_with_event_timing": round(wall_events * 1e3 / args.steps, 6)}
    if n_kernels == 2:
        # X read; A operand (E2M3 lane slots + 8-byte scale records, or E2M1 codes + fp16
        # block scales) and the fp32 partial U of each K-split of at most 1536 values
        # written
        act_bytes = (M * K * 3 // 4 + (K // 64) * M * 8 if method == "int4"
                     else M * K // 2 + M * K // 8)
        k1_bytes = M * K * 2 + act_bytes + M * rank * 4 * (-(-K // 1536))
        k1_gbps = k1_bytes / (kern_ms[0] * 1e-3) / 1e9
        kernels = {"quantize_ms": round(kern_ms[0], 6),
                   "quantize_GBps_algorithmic": round(k1_gbps, 1),
                   "quantize_frac_hbm": round(k1_gbps / PEAK_HBM_GBS, 4),
                   **kernels}
    desc = {"int4": "svdq_w4a4 int4 g64", "nvfp4": "svdq_w4a4 nvfp4 g16",
            "awq": "awq_w4a16 int4 g64"}[method]
    metric = METRIC if args.workload == "attn_proj" else (
        f"{desc} linear effective TOPS at M={M},K={K},N={N}")
    if args.qkv_norm_rope:
        metric += ", Q/K RMSNorm + rotary fused in the epilogue"
        desc += ", Q/K RMSNorm + rotary epilogue"

    out = {
        "metric": metric,
        "value": round(value, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle": settle,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"int4": "int4", "nvfp4": "nvfp4", "awq": "int4-weight/bf16-act"}[method],
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {desc}" + (f" rank {rank}" if rank else "") +
                               f", M={M} K={K} N={N}",
                   "M": M, "K": K, "N": N, "rank": rank, "method": method,
                   "compute_dtype": "bf16", "seeds": inp["seeds"]},
        "pct_int8_peak": round(100.0 * value / PEAK_INT8_TOPS, 2),
        "pct_fp4_peak": round(100.0 * value / PEAK_FP6_TFLOPS, 2),
        "kernels": kernels,
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": recorded_traffic(args.workload),
        },
        "cpu_baseline": None,
    }
    # the achievable dense rate of the matrix instructions, beside the published peaks
    out["mfma_achievable"] = mfma_achievable()
    ach = out["mfma_achievable"][{"int4": "fp6", "nvfp4": "fp16", "awq": "bf16"}[method]]["tflops"]
    out["roofline"]["achievable_peak"] = ach
    out["roofline"]["frac_of_achievable"] = round(achieved / ach, 4)
    if method != "awq":
        # device bytes the layer keeps resident: packed codes and scales, smoothing,
        # lora_down, lora_up, bias
        wbytes = layer.qweight.numel() * layer.qweight.element_size() + \
            layer.wscales.numel() * layer.wscales.element_size()
        rest = sum(t.numel() * t.element_size() for t in
                   (layer.smooth, layer.lora_down, layer.lora_up, layer.bias) if t is not None)
        out["resident"] = {"weight_bytes": wbytes, "bits_per_weight": round(8.0 * wbytes / (N * K), 4),
                           "layer_bytes": wbytes + rest}
        if not args.no_cold:
            out["cold_cache"] = cold_cache_pass(args, inp, layer_args, M, N, K, dev)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on the same inputs", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
