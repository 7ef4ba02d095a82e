"""Benchmark of the quantized GEMM path on one MI355X.

One step = one pass of the dense W4A16 decode-to-prefill sweep: uint4 codes
with a zero point and bf16 scales per group of 128, N = K = 8192, one
hum_linear call at each M in {1, 4, 16, 64, 256, 1024, 4096} (tile / split-K
chosen by the selector per M).  `value` is that sweep's aggregate TFLOP/s.
The same run also measures the other workloads (dense W4A16 tiny, dense W8A8
FP8, MoE W4A16 MXFP4, MoE W4A8 MXFP4 x MXFP8 with Zipf-skewed routing) and
reports each against the MI355X roofline.

Measurement follows the protocol of "Announcing Humming: Fast, Flexible
Kernels for Quantized Inference", section "Performance": warmed kernels, cold
caches between samples -- here R rotating copies of the weights (> 1 GiB in
total) defeat the 4 MB L2 per XCD and the 256 MB Infinity Cache; MoE time is
the whole layer (align, gate_up, down, reduce).  Times come from HIP events
recorded around HIP-graph replays of the calls (so host-side launch cost is
excluded), on the stream the kernels run on.

The CPU baseline is the oracle (NumPy float64) timed on the host on a
bounded sample of the same sweep.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12            # B/s
BF16_PEAK = 2.5e15           # FLOP/s dense
FP8_PEAK = 5.0e15
FP4_PEAK = 10.1e15


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--suite", choices=["dense", "all"], default="all")
    ap.add_argument("--iters", type=int, default=50, help="launches per timing sample")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--eager", action="store_true",
                    help="launch every timed call directly instead of replaying a HIP graph (for counter runs)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run 5 plain device copies of BYTES bytes (calibrates HBM byte counters) and exit")
    return ap.parse_args()


def _dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


class Timer:
    """Device time per call: `iters` calls are captured into one HIP graph
    (the library launches kernels only, on torch's current stream, and
    allocates nothing when given its output and workspace), and the graph's
    replay is bracketed by HIP events on the replay stream -- so host-side
    call overhead does not enter the figure."""

    def __init__(self, eager=False):
        import torch
        self.torch = torch
        self.eager = eager

    def run(self, fn, iters):
        torch = self.torch
        if self.eager:
            s = torch.cuda.current_stream()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(s)
            for i in range(iters):
                fn(i)
            e1.record(s)
            e1.synchronize()
            return e0.elapsed_time(e1) * 1e-3 / iters
        fn(0)                       # first-call setup (kernel attributes) outside the capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(iters):
                fn(i)
        g.replay()                  # warm replay
        torch.cuda.synchronize()
        s = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        g.replay()
        e1.record(s)
        e1.synchronize()
        del g
        return e0.elapsed_time(e1) * 1e-3 / iters   # seconds per call


def rotate_copies(packed, nbytes_total_min=1 << 30):
    reps = max(2, int(np.ceil(nbytes_total_min / packed.numel())))
    return [packed] + [packed.clone() for _ in range(reps - 1)]


def dense_w4a16_sweep(hum, timer, iters):
    import synth
    n = k = 8192
    case = synth.dense_w4a16(synth.seed_for(2), 1, n, k, group=128, asym=True)
    desc = hum.make_desc("uint4", "group", 128, "bf16", n, k, has_zero=True)
    packed = hum.prepare_weight(desc, _dev(case["codes"]), _dev(case["scales"]), _dev(case["zeros"]))
    copies = rotate_copies(packed)
    g = synth.rng(synth.seed_for(2, 1))
    wbytes = n * k // 2 + n * (k // 128) * 2 + n * (k // 128) // 2
    xs, outs, res = {}, {}, []
    import torch
    for m in synth.DENSE_SWEEP_M:
        xs[m] = _dev(synth.bf16_normal(g, (m, k)))
        outs[m] = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    ws = hum.Workspace("cuda").get(max(hum.linear_workspace_bytes(desc, m) for m in synth.DENSE_SWEEP_M))
    for m in synth.DENSE_SWEEP_M:
        fn = lambda i, m=m: hum.linear(desc, copies[i % len(copies)], xs[m], out=outs[m], workspace=ws)
        timer.run(fn, 3)
        t = timer.run(fn, iters)
        flops = 2.0 * m * n * k
        c = hum.select_config(desc, m)
        bound = "hbm" if m <= 64 else "mfma"
        res.append({
            "m": m, "us": t * 1e6, "tflops": flops / t / 1e12, "weight_gbs": wbytes / t / 1e9,
            "bound": bound,
            "frac": (wbytes / t / HBM_PEAK) if bound == "hbm" else (flops / t / BF16_PEAK),
            "tile": list(c.as_tuple()),
        })
    step = lambda i: [hum.linear(desc, copies[(i * 7 + j) % len(copies)], xs[m], out=outs[m], workspace=ws)
                      for j, m in enumerate(synth.DENSE_SWEEP_M)]
    flops_step = sum(2.0 * m * n * k for m in synth.DENSE_SWEEP_M)
    return {"desc": desc, "copies": copies, "xs": xs, "outs": outs, "ws": ws, "res": res,
            "step": step, "flops_step": flops_step, "wbytes": wbytes, "case": case}


def dense_w4a16_fp4(hum, timer, iters, scale):
    """4-bit weights x bf16 at N = K = 8192, the W4A16 sweep's shape: MXFP4
    (E8M0 per 32), NVFP4 (E4M3 per 16 + an f32 tensor scale) or MXINT4 (INT4
    codes, E8M0 per 32)."""
    import synth
    import torch
    n = k = 8192
    if scale in ("e8m0", "mxint4"):
        wd = "e2m1" if scale == "e8m0" else "int4"
        w = synth.quant_weights(synth.seed_for(11, 3 if scale == "mxint4" else 0), wd, "group", 32, "e8m0", 1, n, k)
        desc = hum.make_desc(wd, "group", 32, "e8m0", n, k)
        packed = hum.prepare_weight(desc, _dev(w["codes"]), _dev(w["scales"]))
        wbytes = n * k // 2 + n * (k // 32)
    else:
        w = synth.quant_weights(synth.seed_for(11, 1), "e2m1", "group", 16, "e4m3", 1, n, k, global_scale=True)
        desc = hum.make_desc("e2m1", "group", 16, "e4m3", n, k, has_global=True)
        packed = hum.prepare_weight(desc, _dev(w["codes"]), _dev(w["scales"]), None, _dev(w["global_scale"]))
        wbytes = n * k // 2 + n * (k // 16)
    copies = rotate_copies(packed)
    g = synth.rng(synth.seed_for(11, 2))
    out = []
    for m in synth.DENSE_SWEEP_M:
        x = _dev(synth.bf16_normal(g, (m, k)))
        o = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        ws = hum.Workspace("cuda").get(hum.linear_workspace_bytes(desc, m))
        fn = lambda i: hum.linear(desc, copies[i % len(copies)], x, out=o, workspace=ws)
        timer.run(fn, 3)
        t = timer.run(fn, iters)
        flops = 2.0 * m * n * k
        bound = "hbm" if m <= 64 else "mfma"
        out.append({"m": m, "us": t * 1e6, "tflops": flops / t / 1e12, "weight_gbs": wbytes / t / 1e9,
                    "bound": bound, "frac": (wbytes / t / HBM_PEAK) if bound == "hbm" else flops / t / BF16_PEAK,
                    "tile": list(hum.select_config(desc, m).as_tuple())})
    return out


def dense_tiny(hum, timer, iters):
    import synth
    case = synth.dense_w4a16(synth.seed_for(1), 16, 512, 1024, group=128)
    desc = hum.make_desc("int4", "group", 128, "bf16", 512, 1024)
    packed = hum.prepare_weight(desc, _dev(case["codes"]), _dev(case["scales"]))
    x = _dev(case["x"])
    import torch
    o = torch.empty((16, 512), dtype=torch.bfloat16, device="cuda")
    ws = hum.Workspace("cuda").get(hum.linear_workspace_bytes(desc, 16))
    t = timer.run(lambda i: hum.linear(desc, packed, x, out=o, workspace=ws), iters)
    wbytes = 512 * 1024 // 2 + 512 * 8 * 2
    return [{"m": 16, "us": t * 1e6, "tflops": 2 * 16 * 512 * 1024 / t / 1e12, "weight_gbs": wbytes / t / 1e9,
             "bound": "latency", "frac": wbytes / t / HBM_PEAK}]


def dense_w8a8(hum, timer, iters):
    import synth
    import torch
    n, k = 7168, 2048
    case = synth.dense_w8a8(synth.seed_for(3), 1, n, k)
    desc = hum.make_desc("e4m3", "channel", 0, "f32", n, k, act_fmt="fp8_token")
    packed = hum.prepare_weight(desc, _dev(case["codes"]), _dev(case["scales"]))
    copies = rotate_copies(packed)
    g = synth.rng(synth.seed_for(3, 1))
    wbytes = n * k + n * 4
    out = []
    for m in synth.FP8_SWEEP_M:
        x = _dev(synth.bf16_normal(g, (m, k)))
        o = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        ws = hum.Workspace("cuda").get(hum.linear_workspace_bytes(desc, m))
        fn = lambda i: hum.linear(desc, copies[i % len(copies)], x, out=o, workspace=ws)
        timer.run(fn, 3)
        t = timer.run(fn, iters)
        flops = 2.0 * m * n * k
        bound = "hbm" if m <= 128 else "mfma"
        out.append({"m": m, "us": t * 1e6, "tflops": flops / t / 1e12, "weight_gbs": wbytes / t / 1e9,
                    "bound": bound, "frac": (wbytes / t / HBM_PEAK) if bound == "hbm" else flops / t / FP8_PEAK,
                    "tile": list(hum.select_config(desc, m).as_tuple())})
    return out


def dense_w8a16(hum, timer, iters, weight_dtype):
    """8-bit weights (E4M3 or INT8, per-channel f32 scales) x bf16
    activations, at the W8A8 layer's shape N = 7168, K = 2048."""
    import synth
    import torch
    n, k = 7168, 2048
    if weight_dtype == "e4m3":
        case = synth.dense_w8a8(synth.seed_for(8), 1, n, k)
    else:
        case = synth.quant_weights(synth.seed_for(8, 2), "int8", "channel", 0, "f32", 1, n, k,
                                   scale_lo=0.0002, scale_hi=0.001)
    desc = hum.make_desc(weight_dtype, "channel", 0, "f32", n, k, act_fmt="bf16")
    packed = hum.prepare_weight(desc, _dev(case["codes"]), _dev(case["scales"]))
    copies = rotate_copies(packed)
    g = synth.rng(synth.seed_for(8, 1))
    wbytes = n * k + n * 4
    out = []
    for m in synth.FP8_SWEEP_M:
        x = _dev(synth.bf16_normal(g, (m, k)))
        o = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        ws = hum.Workspace("cuda").get(hum.linear_workspace_bytes(desc, m))
        fn = lambda i: hum.linear(desc, copies[i % len(copies)], x, out=o, workspace=ws)
        timer.run(fn, 3)
        t = timer.run(fn, iters)
        flops = 2.0 * m * n * k
        bound = "hbm" if m <= 128 else "mfma"
        out.append({"m": m, "us": t * 1e6, "tflops": flops / t / 1e12, "weight_gbs": wbytes / t / 1e9,
                    "bound": bound, "frac": (wbytes / t / HBM_PEAK) if bound == "hbm" else flops / t / BF16_PEAK,
                    "tile": list(hum.select_config(desc, m).as_tuple())})
    return out


def dense_w8a8_block(hum, timer, iters):
    """Block-scaled FP8 W8A8 (128 x 128 weight-block scales, per-row groups of
    128 activations quantized in the call), at the W8A8 layer's shape."""
    import synth
    import torch
    n, k = 7168, 2048
    w = synth.quant_weights(synth.seed_for(7), "e4m3", "block", 128, "f32", 1, n, k,
                            scale_lo=0.0005, scale_hi=0.002)
    desc = hum.make_desc("e4m3", "block", 128, "f32", n, k, act_fmt="fp8_group")
    packed = hum.prepare_weight(desc, _dev(w["codes"]), _dev(w["scales"]))
    copies = rotate_copies(packed)
    g = synth.rng(synth.seed_for(7, 1))
    wbytes = n * k + (n // 128) * (k // 128) * 4
    out = []
    for m in synth.FP8_SWEEP_M:
        x = _dev(synth.bf16_normal(g, (m, k)))
        o = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        ws = hum.Workspace("cuda").get(hum.linear_workspace_bytes(desc, m))
        fn = lambda i: hum.linear(desc, copies[i % len(copies)], x, out=o, workspace=ws)
        timer.run(fn, 3)
        t = timer.run(fn, iters)
        flops = 2.0 * m * n * k
        bound = "hbm" if m <= 128 else "mfma"
        out.append({"m": m, "us": t * 1e6, "tflops": flops / t / 1e12, "weight_gbs": wbytes / t / 1e9,
                    "bound": bound, "frac": (wbytes / t / HBM_PEAK) if bound == "hbm" else flops / t / FP8_PEAK,
                    "tile": list(hum.select_config(desc, m).as_tuple())})
    return out


def dense_w4a4(hum, timer, iters):
    """Dense W4A4 (MXFP4 weights x MXFP4 activations quantized in the call),
    at the W8A8 layer's shape N = 7168, K = 2048."""
    import synth
    import torch
    n, k = 7168, 2048
    w = synth.moe_weights_mxfp4(synth.seed_for(6), 1, n, k)
    desc = hum.make_desc("e2m1", "group", 32, "e8m0", n, k, act_fmt="mxfp4")
    packed = hum.prepare_weight(desc, _dev(w["codes"]), _dev(w["scales"]))
    copies = rotate_copies(packed)
    g = synth.rng(synth.seed_for(6, 1))
    wbytes = n * k // 2 + n * k // 32
    out = []
    for m in synth.FP8_SWEEP_M:
        x = _dev(synth.bf16_normal(g, (m, k)))
        o = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        ws = hum.Workspace("cuda").get(hum.linear_workspace_bytes(desc, m))
        fn = lambda i: hum.linear(desc, copies[i % len(copies)], x, out=o, workspace=ws)
        timer.run(fn, 3)
        t = timer.run(fn, iters)
        flops = 2.0 * m * n * k
        bound = "hbm" if m <= 128 else "mfma"
        out.append({"m": m, "us": t * 1e6, "tflops": flops / t / 1e12, "weight_gbs": wbytes / t / 1e9,
                    "bound": bound, "frac": (wbytes / t / HBM_PEAK) if bound == "hbm" else flops / t / FP4_PEAK,
                    "tile": list(hum.select_config(desc, m).as_tuple())})
    return out


def moe(hum, timer, iters, act):
    import synth
    import torch
    e, h, inter, topk = 128, 4096, 1024, 8
    w13 = synth.moe_weights_mxfp4(synth.seed_for(4), e, 2 * inter, h)
    w2 = synth.moe_weights_mxfp4(synth.seed_for(4, 1), e, h, inter)
    d13 = hum.make_desc("e2m1", "group", 32, "e8m0", 2 * inter, h, num_experts=e, act_fmt=act)
    d2 = hum.make_desc("e2m1", "group", 32, "e8m0", h, inter, num_experts=e, act_fmt=act)
    p13 = [hum.prepare_weight(d13, _dev(w13["codes"]), _dev(w13["scales"]))]
    p2 = [hum.prepare_weight(d2, _dev(w2["codes"]), _dev(w2["scales"]))]
    del w13, w2
    p13.append(p13[0].clone())
    p2.append(p2[0].clone())
    per_expert = (2 * inter * h // 2 + 2 * inter * h // 32) + (h * inter // 2 + h * inter // 32)
    ts = synth.MOE_W4A16_T if act == "bf16" else synth.MOE_W4A8_T
    cfgno = 4 if act == "bf16" else 5
    out = []
    for i, t in enumerate(ts):
        ids, wts = synth.routing(synth.seed_for(cfgno, i), t, e, topk, zipf_s=(None if act == "bf16" else 1.1))
        touched = int(len(np.unique(ids)))
        x = _dev(synth.bf16_normal(synth.rng(synth.seed_for(cfgno, 100 + i)), (t, h)))
        di, dw = _dev(ids), _dev(wts)
        o = torch.empty((t, h), dtype=torch.bfloat16, device="cuda")
        ws = hum.Workspace("cuda").get(hum.moe_workspace_bytes(d13, d2, t, topk))
        fn = lambda j: hum.moe_gemm(d13, p13[j % 2], d2, p2[j % 2], x, di, dw, out=o, workspace=ws)
        timer.run(fn, 2)
        tt = timer.run(fn, max(5, iters // 2))
        flops = 2.0 * t * topk * (2 * inter * h + h * inter)
        wb = touched * per_expert
        bound = "hbm" if t * topk < 8 * 1024 else "mfma"
        peak = {"bf16": BF16_PEAK, "mxfp8": FP8_PEAK, "mxfp4": FP4_PEAK}[act]
        cnt = np.bincount(ids.reshape(-1), minlength=e)
        out.append({"tokens": t, "us": tt * 1e6, "tflops": flops / tt / 1e12, "weight_gbs": wb / tt / 1e9,
                    "experts_touched": touched, "max_rows": int(cnt.max()), "bound": bound,
                    "frac": (wb / tt / HBM_PEAK) if bound == "hbm" else flops / tt / peak})
    del p13, p2
    torch.cuda.empty_cache()
    return out


def moe_masked(hum, timer, iters, act):
    """The W4A8 expert layer on the grouped_masked layout (per-expert padded
    buffers [E][max_m][H] with device-side row counts, no top-k combine), the
    same 128 experts as the indexed sweep; counts from Zipf-skewed routing of
    T tokens, clamped to max_m."""
    import synth
    import torch
    e, h, inter, topk, max_m = 128, 4096, 1024, 8, 256
    w13 = synth.moe_weights_mxfp4(synth.seed_for(4), e, 2 * inter, h)
    w2 = synth.moe_weights_mxfp4(synth.seed_for(4, 1), e, h, inter)
    d13 = hum.make_desc("e2m1", "group", 32, "e8m0", 2 * inter, h, num_experts=e, act_fmt=act)
    d2 = hum.make_desc("e2m1", "group", 32, "e8m0", h, inter, num_experts=e, act_fmt=act)
    p13 = [hum.prepare_weight(d13, _dev(w13["codes"]), _dev(w13["scales"]))]
    p2 = [hum.prepare_weight(d2, _dev(w2["codes"]), _dev(w2["scales"]))]
    del w13, w2
    p13.append(p13[0].clone())
    p2.append(p2[0].clone())
    per_expert = (2 * inter * h // 2 + 2 * inter * h // 32) + (h * inter // 2 + h * inter // 32)
    x = _dev(synth.bf16_normal(synth.rng(synth.seed_for(6, 100)), (e, max_m, h)))
    o = torch.empty((e, max_m, h), dtype=torch.bfloat16, device="cuda")
    out = []
    for i, t in enumerate((16, 128, 1024)):
        ids, _ = synth.routing(synth.seed_for(6, i), t, e, topk, zipf_s=1.1)
        cnt = np.minimum(np.bincount(ids.reshape(-1), minlength=e), max_m).astype(np.int32)
        expected = -(-t * topk // e)
        dc = _dev(cnt)
        ws = hum.Workspace("cuda").get(hum.moe_masked_workspace_bytes(d13, d2, max_m, expected))
        fn = lambda j: hum.moe_gemm_masked(d13, p13[j % 2], d2, p2[j % 2], x, dc, expected, out=o, workspace=ws)
        timer.run(fn, 2)
        tt = timer.run(fn, max(5, iters // 2))
        rows = int(cnt.sum())
        flops = 2.0 * rows * (2 * inter * h + h * inter)
        touched = int((cnt > 0).sum())
        wb = touched * per_expert
        bound = "hbm" if rows < 8 * 1024 else "mfma"
        peak = {"bf16": BF16_PEAK, "mxfp8": FP8_PEAK, "mxfp4": FP4_PEAK}[act]
        out.append({"tokens": t, "max_m": max_m, "expected_m": expected, "rows": rows, "us": tt * 1e6,
                    "tflops": flops / tt / 1e12, "weight_gbs": wb / tt / 1e9, "experts_touched": touched,
                    "bound": bound, "frac": (wb / tt / HBM_PEAK) if bound == "hbm" else flops / tt / peak})
    del p13, p2
    torch.cuda.empty_cache()
    return out


def cpu_baseline(case, budget_s=30.0):
    """Oracle (NumPy float64) on the host: the same M sweep restricted to a
    column sample of the weights."""
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    n, k = 8192, 8192
    od = oracle.gemm.WeightDesc("uint4", "group", 128, "bf16", True, False, 1, n, k)
    g = synth.rng(synth.seed_for(2, 2))
    cols = 256
    flops = 0.0
    t0 = time.perf_counter()
    while True:
        sub = oracle.gemm.WeightDesc("uint4", "group", 128, "bf16", True, False, 1, cols, k)
        w = {"codes": case["codes"][:, :cols], "scales": case["scales"][:, :cols], "zeros": case["zeros"][:, :cols]}
        for m in synth.DENSE_SWEEP_M:
            a = oracle.formats.decode_bf16(synth.bf16_normal(g, (m, k)))
            oracle.gemm.linear(sub, a, w["codes"], w["scales"], w["zeros"])
            flops += 2.0 * m * cols * k
        el = time.perf_counter() - t0
        if el > budget_s / 3 or cols >= n:
            break
        cols = min(n, cols * 2)
    el = time.perf_counter() - t0
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"dense W4A16 uint4+zp G128 K=8192, M sweep 1..4096 on weight columns "
                      f"(256 doubling to {cols}) of N=8192; {flops / 1e9:.1f} GFLOP in {el:.1f} s"}


def traffic_for(kernel_src_hash):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic_dense_w4a16_m4096.json")
    try:
        d = json.load(open(path))
    except Exception:
        return None
    if d.get("kernel_src_sha256") != kernel_src_hash:
        return None
    return d.get("bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1"}))
        sys.exit(2)
    import torch
    if args.copy_probe:
        torch.cuda.set_device(0)
        src = torch.ones(args.copy_probe // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": src.numel() * 4, "launches": 5}))
        return
    import quantized_gemm_packed_amd as hum
    hum.load_library()
    torch.cuda.set_device(0)
    timer = Timer(eager=args.eager)
    iters = args.iters
    d = dense_w4a16_sweep(hum, timer, iters)
    # timed steps
    for i in range(args.warmup):
        d["step"](i)
    torch.cuda.synchronize()
    t_step = timer.run(lambda i: d["step"](i), args.steps)
    value = d["flops_step"] / t_step / 1e12
    # dominant kernel: the M=4096 GEMM (largest share of the step)
    dom = max(d["res"], key=lambda r: r["us"])
    src = open(os.path.join(ROOT, "quantized_gemm_packed_amd", "csrc", "gemm.hip"), "rb").read()
    src_hash = hashlib.sha256(src).hexdigest()
    dom_flops = 2.0 * dom["m"] * 8192 * 8192
    roofline = {
        "bound": "mfma", "achieved": dom["tflops"], "peak": BF16_PEAK / 1e12, "unit": "TFLOP/s",
        "frac": dom["tflops"] * 1e12 / BF16_PEAK, "traffic": traffic_for(src_hash),
        "kernel": f"tile_kernel F_INT m={dom['m']} tile={dom['tile']} (+ rowsum_kernel)", "flops_per_launch": dom_flops,
        "us_per_launch": dom["us"],
    }
    sweep = {"dense_w4a16_uint4_zp_g128_n8192_k8192": d["res"]}
    if args.suite == "all":
        sweep["dense_w4a16_int4_g128_m16_n512_k1024"] = dense_tiny(hum, timer, iters)
        sweep["dense_w8a8_fp8_n7168_k2048"] = dense_w8a8(hum, timer, iters)
        sweep["dense_w8a8_fp8_block128_n7168_k2048"] = dense_w8a8_block(hum, timer, iters)
        sweep["dense_w8a16_fp8_n7168_k2048"] = dense_w8a16(hum, timer, iters, "e4m3")
        sweep["dense_w8a16_int8_n7168_k2048"] = dense_w8a16(hum, timer, iters, "int8")
        sweep["dense_w4a16_mxfp4_n8192_k8192"] = dense_w4a16_fp4(hum, timer, iters, "e8m0")
        sweep["dense_w4a16_nvfp4_n8192_k8192"] = dense_w4a16_fp4(hum, timer, iters, "e4m3")
        sweep["dense_w4a16_mxint4_n8192_k8192"] = dense_w4a16_fp4(hum, timer, iters, "mxint4")
        sweep["dense_w4a4_mxfp4_n7168_k2048"] = dense_w4a4(hum, timer, iters)
        del d["copies"]
        torch.cuda.empty_cache()
        sweep["moe_w4a16_mxfp4_e128_top8_h4096_i1024"] = moe(hum, timer, iters, "bf16")
        sweep["moe_w4a8_mxfp4_mxfp8_zipf1.1_e128_top8_h4096_i1024"] = moe(hum, timer, iters, "mxfp8")
        sweep["moe_w4a4_mxfp4_mxfp4_zipf1.1_e128_top8_h4096_i1024"] = moe(hum, timer, iters, "mxfp4")
        sweep["moe_masked_w4a8_mxfp4_mxfp8_e128_maxm256_h4096_i1024"] = moe_masked(hum, timer, iters, "mxfp8")
    cpu = None if args.no_cpu else cpu_baseline(d["case"])
    line = {
        "metric": "quant GEMM TFLOP/s + weight HBM GB/s vs roofline, dense & MoE, M=1..4096",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": t_step * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "dense W4A16 uint4+zero-point G128 bf16-scale, N=K=8192, "
                               "M sweep {1,4,16,64,256,1024,4096} (one hum_linear per M = one step)",
                   "weights_bytes": d["wbytes"], "seed": 2000, "rotating_weight_copies": True},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "sweep": sweep,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
