"""Benchmark of the quantized GEMM path on one MI355X.

One step = one pass of the dense W4A16 decode-to-prefill sweep: uint4 codes
with a zero point and bf16 scales per group of 128, N = K = 8192, one
hum_linear call at each M in {1, 4, 16, 64, 256, 1024, 4096} (tile / split-K
chosen by the selector per M).  `value` is that sweep's aggregate TFLOP/s.
The same run also measures the other workloads (dense W4A16 tiny, dense W8A8
FP8, MoE W4A16 MXFP4, MoE W4A8 MXFP4 x MXFP8 with Zipf-skewed routing, and
the other formats of the description) and reports each against the MI355X
roofline, next to this box's own re-measured peaks.

Measurement follows the protocol of "Announcing Humming: Fast, Flexible
Kernels for Quantized Inference", section "Performance": warmed kernels, cold
caches between samples -- here R rotating copies of the weights (> 1 GiB in
total) defeat the 4 MB L2 per XCD and the 256 MB Infinity Cache; MoE time is
the whole layer (align, gate_up, down, reduce).  Times come from HIP events
recorded around HIP-graph replays of the calls (so host-side launch cost is
excluded), on the stream the kernels run on.  Every shape also gets one
single-launch sample after a 512 MB write flushes the caches (`us_flush`).

The CPU baseline is the oracle (NumPy float64) timed on the host on a
bounded sample of the same sweep.

Options for single-shape runs (counter collection):
  --only SUITE[,SUITE]  run only these suites (names below), no timed step
  --sizes N[,N]         only these M / token counts
  --eager               launch every timed call directly (no graph)
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

SUITES = ("dense_w4a16", "tiny", "w8a8", "w8a8_block", "w8a16_fp8", "w8a16_int8", "w4a16_mxfp4",
          "w4a16_nvfp4", "w4a16_mxint4", "w3a16", "w2a16", "w6a16", "w4a4", "moe_w4a16", "moe_w4a8", "moe_w4a4", "moe_masked",
          "moe_w8a8_block", "peaks")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--suite", choices=["dense", "all"], default="all")
    ap.add_argument("--only", default="", help="comma-separated suites: " + ",".join(SUITES))
    ap.add_argument("--sizes", default="", help="comma-separated M / token counts to run")
    ap.add_argument("--iters", type=int, default=50, help="launches per timing sample")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-flush", action="store_true", help="skip the single-launch-after-flush samples")
    ap.add_argument("--eager", action="store_true",
                    help="launch every timed call directly instead of replaying a HIP graph (for counter runs)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run 5 plain device copies of BYTES bytes (calibrates HBM byte counters) and exit")
    return ap.parse_args()


ARGS = None


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def sizes(default):
    if not ARGS.sizes:
        return tuple(default)
    want = {int(s) for s in ARGS.sizes.split(",") if s}
    return tuple(s for s in default if s in want)


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
        self.flush_buf = None

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

    def flushed(self, fn, reps=3):
        """One call after a 512 MB write (larger than the 256 MB Infinity
        Cache and the L2s), timed alone; the median of `reps` samples.  The
        write runs long enough on the device that the call is queued behind
        the first event before the device reaches it."""
        torch = self.torch
        if ARGS.no_flush:
            return None
        if self.flush_buf is None:
            self.flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        s = torch.cuda.current_stream()
        out = []
        for r in range(reps):
            self.flush_buf.fill_(r + 1)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(s)
            fn(r)
            e1.record(s)
            e1.synchronize()
            out.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(out))


def rotate_copies(packed, nbytes_total_min=1 << 30):
    reps = max(2, int(np.ceil(nbytes_total_min / packed.numel())))
    return [packed] + [packed.clone() for _ in range(reps - 1)]


def _row(m, t, flops, wbytes, bound, peak, tile, t_flush):
    r = {"m": m, "us": t * 1e6, "tflops": flops / t / 1e12, "weight_gbs": wbytes / t / 1e9, "bound": bound,
         "frac": (wbytes / t / HBM_PEAK) if bound == "hbm" else (flops / t / peak), "tile": tile}
    if t_flush is not None:
        r["us_flush"] = t_flush * 1e6
    return r


def dense_sweep(hum, timer, iters, name, desc, packed, wbytes, ms, hbm_max_m, peak, x_seed):
    """One hum_linear per M over rotating weight copies."""
    import synth
    import torch
    n, k = desc.n, desc.k
    copies = rotate_copies(packed)
    g = synth.rng(x_seed)
    out = []
    for m in ms:
        x = _dev(synth.bf16_normal(g, (m, k)))
        o = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        ws = hum.Workspace("cuda").get(hum.linear_workspace_bytes(desc, m))
        fn = lambda i: hum.linear(desc, copies[i % len(copies)], x, out=o, workspace=ws)
        timer.run(fn, 3)
        t = timer.run(fn, iters)
        tf = timer.flushed(fn)
        bound = "hbm" if m <= hbm_max_m else "mfma"
        out.append(_row(m, t, 2.0 * m * n * k, wbytes, bound, peak, list(hum.select_config(desc, m).as_tuple()), tf))
        log(f"{name} m={m}: {t * 1e6:.1f} us ({out[-1]['frac']:.3f} of {bound})")
    del copies
    torch.cuda.empty_cache()
    return out


def dense_w4a16_sweep(hum, timer, iters):
    import synth
    import torch
    n = k = 8192
    case = synth.dense_w4a16(synth.seed_for(2), 1, n, k, group=128, asym=True)
    desc = hum.make_desc("uint4", "group", 128, "bf16", n, k, has_zero=True)
    packed = hum.prepare_weight(desc, _dev(case["codes"]), _dev(case["scales"]), _dev(case["zeros"]))
    copies = rotate_copies(packed)
    g = synth.rng(synth.seed_for(2, 1))
    wbytes = n * k // 2 + n * (k // 128) * 2 + n * (k // 128) // 2
    xs, outs, res = {}, {}, []
    ms = sizes(synth.DENSE_SWEEP_M)
    for m in synth.DENSE_SWEEP_M:
        xs[m] = _dev(synth.bf16_normal(g, (m, k)))
        outs[m] = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    ws = hum.Workspace("cuda").get(max(hum.linear_workspace_bytes(desc, m) for m in synth.DENSE_SWEEP_M))
    for m in ms:
        fn = lambda i, m=m: hum.linear(desc, copies[i % len(copies)], xs[m], out=outs[m], workspace=ws)
        timer.run(fn, 3)
        t = timer.run(fn, iters)
        tf = timer.flushed(fn)
        bound = "hbm" if m <= 64 else "mfma"
        res.append(_row(m, t, 2.0 * m * n * k, wbytes, bound, BF16_PEAK, list(hum.select_config(desc, m).as_tuple()),
                        tf))
        log(f"dense_w4a16 m={m}: {t * 1e6:.1f} us ({res[-1]['frac']:.3f} of {bound})")
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
    name = {"e8m0": "w4a16_mxfp4", "mxint4": "w4a16_mxint4"}.get(scale, "w4a16_nvfp4")
    return dense_sweep(hum, timer, iters, name, desc, packed, wbytes, sizes(synth.DENSE_SWEEP_M), 64, BF16_PEAK,
                       synth.seed_for(11, 2))


def dense_lowbit(hum, timer, iters, wd):
    """b-bit integer weights (INT3 / INT2, G = 128, bf16 scales, no zero
    point) x bf16 at N = K = 8192, the W4A16 sweep's shape."""
    import synth
    n = k = 8192
    bits = synth.INT_BITS[wd]
    w = synth.quant_weights(synth.seed_for(12, bits), wd, "group", 128, "bf16", 1, n, k)
    desc = hum.make_desc(wd, "group", 128, "bf16", n, k)
    packed = hum.prepare_weight(desc, _dev(w["codes"]), _dev(w["scales"]))
    wbytes = n * k * bits // 8 + n * (k // 128) * 2
    return dense_sweep(hum, timer, iters, f"w{bits}a16_{wd}", desc, packed, wbytes, sizes(synth.DENSE_SWEEP_M), 64,
                       BF16_PEAK, synth.seed_for(12, 9))


def dense_mxfp6(hum, timer, iters):
    """MXFP6 E2M3 weights (E8M0 per 32) x bf16 at N = K = 8192."""
    import synth
    n = k = 8192
    w = synth.quant_weights(synth.seed_for(13), "e2m3", "group", 32, "e8m0", 1, n, k)
    desc = hum.make_desc("e2m3", "group", 32, "e8m0", n, k)
    packed = hum.prepare_weight(desc, _dev(w["codes"]), _dev(w["scales"]))
    wbytes = n * k * 6 // 8 + n * (k // 32)
    return dense_sweep(hum, timer, iters, "w6a16_mxfp6", desc, packed, wbytes, sizes(synth.DENSE_SWEEP_M), 64,
                       BF16_PEAK, synth.seed_for(13, 1))


def dense_tiny(hum, timer, iters):
    import synth
    import torch
    case = synth.dense_w4a16(synth.seed_for(1), 16, 512, 1024, group=128)
    desc = hum.make_desc("int4", "group", 128, "bf16", 512, 1024)
    packed = hum.prepare_weight(desc, _dev(case["codes"]), _dev(case["scales"]))
    x = _dev(case["x"])
    o = torch.empty((16, 512), dtype=torch.bfloat16, device="cuda")
    ws = hum.Workspace("cuda").get(hum.linear_workspace_bytes(desc, 16))
    fn = lambda i: hum.linear(desc, packed, x, out=o, workspace=ws)
    t = timer.run(fn, iters)
    tf = timer.flushed(fn)
    wbytes = 512 * 1024 // 2 + 512 * 8 * 2
    r = _row(16, t, 2 * 16 * 512 * 1024, wbytes, "latency", BF16_PEAK, list(hum.select_config(desc, 16).as_tuple()),
             tf)
    r["frac"] = wbytes / t / HBM_PEAK
    log(f"tiny: {t * 1e6:.1f} us")
    return [r]


def dense_w8a8(hum, timer, iters):
    import synth
    n, k = 7168, 2048
    case = synth.dense_w8a8(synth.seed_for(3), 1, n, k)
    desc = hum.make_desc("e4m3", "channel", 0, "f32", n, k, act_fmt="fp8_token")
    packed = hum.prepare_weight(desc, _dev(case["codes"]), _dev(case["scales"]))
    return dense_sweep(hum, timer, iters, "w8a8", desc, packed, n * k + n * 4, sizes(synth.FP8_SWEEP_M), 128,
                       FP8_PEAK, synth.seed_for(3, 1))


def dense_w8a16(hum, timer, iters, weight_dtype):
    """8-bit weights (E4M3 or INT8, per-channel f32 scales) x bf16
    activations, at the W8A8 layer's shape N = 7168, K = 2048."""
    import synth
    n, k = 7168, 2048
    if weight_dtype == "e4m3":
        case = synth.dense_w8a8(synth.seed_for(8), 1, n, k)
    else:
        case = synth.quant_weights(synth.seed_for(8, 2), "int8", "channel", 0, "f32", 1, n, k,
                                   scale_lo=0.0002, scale_hi=0.001)
    desc = hum.make_desc(weight_dtype, "channel", 0, "f32", n, k, act_fmt="bf16")
    packed = hum.prepare_weight(desc, _dev(case["codes"]), _dev(case["scales"]))
    return dense_sweep(hum, timer, iters, f"w8a16_{weight_dtype}", desc, packed, n * k + n * 4,
                       sizes(synth.FP8_SWEEP_M), 128, BF16_PEAK, synth.seed_for(8, 1))


def dense_w8a8_block(hum, timer, iters):
    """Block-scaled FP8 W8A8 (128 x 128 weight-block scales, per-row groups of
    128 activations quantized in the call), at the W8A8 layer's shape."""
    import synth
    n, k = 7168, 2048
    w = synth.quant_weights(synth.seed_for(7), "e4m3", "block", 128, "f32", 1, n, k,
                            scale_lo=0.0005, scale_hi=0.002)
    desc = hum.make_desc("e4m3", "block", 128, "f32", n, k, act_fmt="fp8_group")
    packed = hum.prepare_weight(desc, _dev(w["codes"]), _dev(w["scales"]))
    return dense_sweep(hum, timer, iters, "w8a8_block", desc, packed, n * k + (n // 128) * (k // 128) * 4,
                       sizes(synth.FP8_SWEEP_M), 128, FP8_PEAK, synth.seed_for(7, 1))


def dense_w4a4(hum, timer, iters):
    """Dense W4A4 (MXFP4 weights x MXFP4 activations quantized in the call),
    at the W8A8 layer's shape N = 7168, K = 2048."""
    import synth
    n, k = 7168, 2048
    w = synth.moe_weights_mxfp4(synth.seed_for(6), 1, n, k)
    desc = hum.make_desc("e2m1", "group", 32, "e8m0", n, k, act_fmt="mxfp4")
    packed = hum.prepare_weight(desc, _dev(w["codes"]), _dev(w["scales"]))
    return dense_sweep(hum, timer, iters, "w4a4", desc, packed, n * k // 2 + n * k // 32, sizes(synth.FP8_SWEEP_M),
                       128, FP4_PEAK, synth.seed_for(6, 1))


def moe(hum, timer, iters, act, peaks):
    """The MoE layer over the bench token counts (MXFP4 experts, or with
    act = "fp8_group" the same shapes with 128 x 128 block-scaled FP8
    experts).  Bound: HBM while the batch is small (T <= 512 for W4A16,
    T <= 1024 otherwise), the matrix instruction's rate above."""
    import synth
    import torch
    e, h, inter, topk = 128, 4096, 1024, 8
    if act == "fp8_group":
        w13 = synth.quant_weights(synth.seed_for(9), "e4m3", "block", 128, "f32", e, 2 * inter, h,
                                  scale_lo=0.0005, scale_hi=0.002)
        w2 = synth.quant_weights(synth.seed_for(9, 1), "e4m3", "block", 128, "f32", e, h, inter,
                                 scale_lo=0.0005, scale_hi=0.002)
        desc = ("e4m3", "block", 128, "f32")
        per_expert = (2 * inter * h + (2 * inter // 128) * (h // 128) * 4) + (h * inter + (h // 128) * (inter // 128) * 4)
    else:
        w13 = synth.moe_weights_mxfp4(synth.seed_for(4), e, 2 * inter, h)
        w2 = synth.moe_weights_mxfp4(synth.seed_for(4, 1), e, h, inter)
        desc = ("e2m1", "group", 32, "e8m0")
        per_expert = (2 * inter * h // 2 + 2 * inter * h // 32) + (h * inter // 2 + h * inter // 32)
    d13 = hum.make_desc(*desc, 2 * inter, h, num_experts=e, act_fmt=act)
    d2 = hum.make_desc(*desc, h, inter, num_experts=e, act_fmt=act)
    p13 = [hum.prepare_weight(d13, _dev(w13["codes"]), _dev(w13["scales"]))]
    p2 = [hum.prepare_weight(d2, _dev(w2["codes"]), _dev(w2["scales"]))]
    del w13, w2
    p13.append(p13[0].clone())
    p2.append(p2[0].clone())
    ts = synth.MOE_W4A16_T if act == "bf16" else synth.MOE_W4A8_T
    cfgno = 4 if act == "bf16" else 5
    hbm_max_t = 512 if act == "bf16" else 1024
    peak = {"bf16": BF16_PEAK, "mxfp8": peaks.get("mfma_fp8_fp4_flops", FP8_PEAK), "mxfp4": FP4_PEAK,
            "fp8_group": FP8_PEAK}[act]
    out = []
    for i, t in enumerate(ts):
        if t not in sizes(ts):
            continue
        ids, wts = synth.routing(synth.seed_for(cfgno, i), t, e, topk, zipf_s=(None if act == "bf16" else 1.1))
        touched = int(len(np.unique(ids)))
        x = _dev(synth.bf16_normal(synth.rng(synth.seed_for(cfgno, 100 + i)), (t, h)))
        di, dw = _dev(ids), _dev(wts)
        o = torch.empty((t, h), dtype=torch.bfloat16, device="cuda")
        ws = hum.Workspace("cuda").get(hum.moe_workspace_bytes(d13, d2, t, topk))
        fn = lambda j: hum.moe_gemm(d13, p13[j % 2], d2, p2[j % 2], x, di, dw, out=o, workspace=ws)
        timer.run(fn, 2)
        tt = timer.run(fn, max(5, iters // 2))
        tf = timer.flushed(fn)
        flops = 2.0 * t * topk * (2 * inter * h + h * inter)
        wb = touched * per_expert
        bound = "hbm" if t <= hbm_max_t else "mfma"
        cnt = np.bincount(ids.reshape(-1), minlength=e)
        r = {"tokens": t, "us": tt * 1e6, "tflops": flops / tt / 1e12, "weight_gbs": wb / tt / 1e9,
             "experts_touched": touched, "max_rows": int(cnt.max()), "bound": bound,
             "frac": (wb / tt / HBM_PEAK) if bound == "hbm" else flops / tt / peak,
             "tile_up": list(hum.moe_select_config(d13, d2, t, topk, gate_up=True).as_tuple()),
             "tile_down": list(hum.moe_select_config(d13, d2, t, topk).as_tuple())}
        if tf is not None:
            r["us_flush"] = tf * 1e6
        out.append(r)
        log(f"moe {act} t={t}: {tt * 1e6:.1f} us ({r['frac']:.3f} of {bound})")
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
        if t not in sizes((16, 128, 1024)):
            continue
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
        log(f"moe masked t={t}: {tt * 1e6:.1f} us")
    del p13, p2
    torch.cuda.empty_cache()
    return out


def measure_peaks(hum):
    """This box's sustained rates: a stream read of a 1 GiB buffer, and of the
    dense W4A16 sweep's weight size (35 MB) over rotating copies; the
    matrix-instruction issue loops (flops per second) for the 16x16 shapes
    the kernels issue and the 32x32 shapes (on gfx950 the 16x16 bf16 and
    FP4 shapes run at about half the rate of their 32x32 forms)."""
    import torch
    res = {}
    s = torch.cuda.current_stream()

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(reps):
            fn()
        e1.record(s)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    sink = torch.empty(2048 * 256, dtype=torch.float32, device="cuda")
    big = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(3)
    work = [0.0]

    def rd():
        work[0] = hum.peak_probe(hum.PEAK_HBM_READ, big.numel(), big, sink)[1]
    t = timed(rd)
    res["hbm_read_1GiB_GBs"] = work[0] / t / 1e9
    # 35 MB reads, rotating through the 1 GiB buffer (cold in the caches)
    chunk = 34865152 // 16 * 16
    nchunks = big.numel() // chunk
    idx = [0]

    def rd35():
        i = idx[0] % nchunks
        idx[0] += 1
        hum.peak_probe(hum.PEAK_HBM_READ, chunk, big[i * chunk:(i + 1) * chunk], sink)
    t = timed(rd35, reps=20)
    res["hbm_read_35MB_us"] = t * 1e6
    res["hbm_read_35MB_GBs"] = chunk / t / 1e9
    del big
    for name, kind in (("mfma_bf16_flops", hum.PEAK_MFMA_BF16), ("mfma_fp8_flops", hum.PEAK_MFMA_FP8),
                       ("mfma_fp4_flops", hum.PEAK_MFMA_FP4), ("mfma_fp8_fp4_flops", hum.PEAK_MFMA_FP8_FP4),
                       ("mfma32_bf16_flops", hum.PEAK_MFMA32_BF16), ("mfma32_fp8_flops", hum.PEAK_MFMA32_FP8),
                       ("mfma32_fp4_flops", hum.PEAK_MFMA32_FP4), ("mfma32_fp8_fp4_flops", hum.PEAK_MFMA32_FP8_FP4)):
        def mf(kind=kind):
            work[0] = hum.peak_probe(kind, 2000, None, sink)[1]
        t = timed(mf, reps=3)
        res[name] = work[0] / t
    torch.cuda.empty_cache()
    log("peaks: " + ", ".join(f"{k}={v:.4g}" for k, v in res.items()))
    return res


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
        log(f"cpu baseline: {cols} columns, {el:.1f} s")
        if el > budget_s / 3 or cols >= n:
            break
        cols = min(n, cols * 2)
    el = time.perf_counter() - t0
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"dense W4A16 uint4+zp G128 K=8192, M sweep 1..4096 on weight columns "
                      f"(256 doubling to {cols}) of N=8192; {flops / 1e9:.1f} GFLOP in {el:.1f} s"}


KERNEL_SOURCES = ("gemm_kernels.h", "inst_dense_a.hip", "gemm.hip", "hum_internal.h", "dev_common.h")


def kernel_src_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, "quantized_gemm_packed_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def traffic_for(src_hash):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic_dense_w4a16_m4096.json")
    try:
        d = json.load(open(path))
    except Exception:
        return None
    if d.get("kernel_src_sha256") != src_hash:
        return None
    return d.get("bytes_per_launch")


def run_suites(hum, timer, iters, want, peaks, d=None):
    sweep = {}
    if d is not None:
        sweep["dense_w4a16_uint4_zp_g128_n8192_k8192"] = d["res"]
    elif "dense_w4a16" in want:
        sweep["dense_w4a16_uint4_zp_g128_n8192_k8192"] = dense_w4a16_sweep(hum, timer, iters)["res"]
    table = [
        ("tiny", "dense_w4a16_int4_g128_m16_n512_k1024", lambda: dense_tiny(hum, timer, iters)),
        ("w8a8", "dense_w8a8_fp8_n7168_k2048", lambda: dense_w8a8(hum, timer, iters)),
        ("w8a8_block", "dense_w8a8_fp8_block128_n7168_k2048", lambda: dense_w8a8_block(hum, timer, iters)),
        ("w8a16_fp8", "dense_w8a16_fp8_n7168_k2048", lambda: dense_w8a16(hum, timer, iters, "e4m3")),
        ("w8a16_int8", "dense_w8a16_int8_n7168_k2048", lambda: dense_w8a16(hum, timer, iters, "int8")),
        ("w4a16_mxfp4", "dense_w4a16_mxfp4_n8192_k8192", lambda: dense_w4a16_fp4(hum, timer, iters, "e8m0")),
        ("w4a16_nvfp4", "dense_w4a16_nvfp4_n8192_k8192", lambda: dense_w4a16_fp4(hum, timer, iters, "e4m3")),
        ("w4a16_mxint4", "dense_w4a16_mxint4_n8192_k8192", lambda: dense_w4a16_fp4(hum, timer, iters, "mxint4")),
        ("w3a16", "dense_w3a16_int3_g128_n8192_k8192", lambda: dense_lowbit(hum, timer, iters, "int3")),
        ("w2a16", "dense_w2a16_int2_g128_n8192_k8192", lambda: dense_lowbit(hum, timer, iters, "int2")),
        ("w6a16", "dense_w6a16_mxfp6_e2m3_n8192_k8192", lambda: dense_mxfp6(hum, timer, iters)),
        ("w4a4", "dense_w4a4_mxfp4_n7168_k2048", lambda: dense_w4a4(hum, timer, iters)),
        ("moe_w4a16", "moe_w4a16_mxfp4_e128_top8_h4096_i1024", lambda: moe(hum, timer, iters, "bf16", peaks)),
        ("moe_w4a8", "moe_w4a8_mxfp4_mxfp8_zipf1.1_e128_top8_h4096_i1024",
         lambda: moe(hum, timer, iters, "mxfp8", peaks)),
        ("moe_w4a4", "moe_w4a4_mxfp4_mxfp4_zipf1.1_e128_top8_h4096_i1024",
         lambda: moe(hum, timer, iters, "mxfp4", peaks)),
        ("moe_masked", "moe_masked_w4a8_mxfp4_mxfp8_e128_maxm256_h4096_i1024",
         lambda: moe_masked(hum, timer, iters, "mxfp8")),
        ("moe_w8a8_block", "moe_w8a8_fp8_block128_zipf1.1_e128_top8_h4096_i1024",
         lambda: moe(hum, timer, iters, "fp8_group", peaks)),
    ]
    for key, name, fn in table:
        if key in want:
            sweep[name] = fn()
    return sweep


def main():
    global ARGS
    args = parse()
    ARGS = args
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
    if args.only:
        want = {w for w in args.only.split(",") if w}
        bad = want - set(SUITES)
        if bad:
            print(json.dumps({"error": f"unknown suites {sorted(bad)}"}))
            sys.exit(2)
        peaks = measure_peaks(hum) if "peaks" in want else {}
        sweep = run_suites(hum, timer, iters, want, peaks)
        print(json.dumps({"sweep": sweep, "peaks_measured": peaks}))
        return
    want = set(SUITES) if args.suite == "all" else {"dense_w4a16"}
    peaks = measure_peaks(hum) if "peaks" in want else {}
    d = dense_w4a16_sweep(hum, timer, iters)
    # timed steps
    for i in range(args.warmup):
        d["step"](i)
    torch.cuda.synchronize()
    t_step = timer.run(lambda i: d["step"](i), args.steps)
    value = d["flops_step"] / t_step / 1e12
    log(f"step: {t_step * 1e3:.3f} ms, {value:.1f} TFLOP/s")
    # dominant kernel: the M=4096 GEMM (largest share of the step)
    dom = max(d["res"], key=lambda r: r["us"])
    dom_flops = 2.0 * dom["m"] * 8192 * 8192
    roofline = {
        "bound": "mfma", "achieved": dom["tflops"], "peak": BF16_PEAK / 1e12, "unit": "TFLOP/s",
        "frac": dom["tflops"] * 1e12 / BF16_PEAK, "traffic": traffic_for(kernel_src_hash()),
        "kernel": f"tile_kernel F_INT m={dom['m']} tile={dom['tile']} (+ rowsum_kernel)", "flops_per_launch": dom_flops,
        "us_per_launch": dom["us"],
    }
    # the measured rate of the instruction shape the kernel issues (32x32x16
    # for the 32x32-block tiles, 16x16x32 otherwise)
    pk = "mfma32_bf16_flops" if dom["tile"][0] == 2 else "mfma_bf16_flops"
    if pk in peaks:
        roofline["frac_of_measured_peak"] = dom["tflops"] * 1e12 / peaks[pk]
        roofline["measured_peak_key"] = pk
    del d["copies"]
    torch.cuda.empty_cache()
    sweep = run_suites(hum, timer, iters, want - {"dense_w4a16"}, peaks, d=d)
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
        "peaks_measured": peaks,
        "sweep": sweep,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
