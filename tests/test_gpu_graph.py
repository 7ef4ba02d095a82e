"""GPU: the library's calls replay correctly from a captured HIP graph.

Each case captures a call sequence once, then replays the graph several
times with eager work (other library calls, a host synchronization,
clobbered outputs) between the replays, and checks every replay bit for bit
against the eager result of the same calls."""
import numpy as np
import pytest
import torch

import quantized_gemm_packed_amd as hum
import synth
from gpu_util import descs, dev, prepare

pytestmark = pytest.mark.gpu


def _replays_match(calls, outs, eager_noise):
    for c in calls:            # eager reference (also first-call setup)
        c()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        eager_noise()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o, r), f"replay {rep} differs from the eager result"


@pytest.mark.parametrize("m", [1, 4, 16, 64, 300])
def test_linear_uint4_graph_replay(m):
    n, k = 640, 2048
    case = synth.dense_w4a16(synth.seed_for(9, m), m, n, k, group=128, asym=True)
    hd, _ = descs("uint4", "group", 128, "bf16", 1, n, k, zero=True)
    packed = prepare(hd, case, "bf16")
    x = dev(case["x"])
    out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    ws = hum.Workspace("cuda").get(hum.linear_workspace_bytes(hd, m))
    # eager noise: the same layer at another M, on other buffers
    x2 = dev(synth.bf16_normal(synth.rng(5), (7, k)))
    print(f"case graph linear uint4 m={m}", flush=True)
    _replays_match([lambda: hum.linear(hd, packed, x, out=out, workspace=ws)], [out],
                   lambda: hum.linear(hd, packed, x2))


@pytest.mark.parametrize("m", [1, 128])
def test_linear_fp8_graph_replay(m):
    n, k = 512, 1024
    case = synth.dense_w8a8(synth.seed_for(9, 100 + m), m, n, k)
    hd, _ = descs("e4m3", "channel", 0, "f32", 1, n, k, act="fp8_token")
    packed = prepare(hd, case, "f32")
    x = dev(case["x"])
    out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    ws = hum.Workspace("cuda").get(hum.linear_workspace_bytes(hd, m))
    print(f"case graph linear fp8 m={m}", flush=True)
    _replays_match([lambda: hum.linear(hd, packed, x, out=out, workspace=ws)], [out],
                   lambda: hum.linear(hd, packed, x[:1].contiguous()))


@pytest.mark.parametrize("fmt", ["w4a4", "fp8_block"])
@pytest.mark.parametrize("m", [1, 5])
def test_linear_decode_quantizing_formats_graph_replay(fmt, m):
    """The decode kernels that quantize their activations themselves (W4A4 as
    E4M3 x E2M1, block-scaled FP8) and the quantizer launch they need, from
    a captured graph."""
    n, k = 512, 1024
    if fmt == "w4a4":
        w = synth.moe_weights_mxfp4(synth.seed_for(9, 200 + m), 1, n, k)
        hd, _ = descs("e2m1", "group", 32, "e8m0", 1, n, k, act="mxfp4")
        packed = prepare(hd, w, "e8m0")
    else:
        w = synth.quant_weights(synth.seed_for(9, 300 + m), "e4m3", "block", 128, "f32", 1, n, k,
                                scale_lo=0.0005, scale_hi=0.002)
        hd, _ = descs("e4m3", "block", 128, "f32", 1, n, k, act="fp8_group")
        packed = prepare(hd, w, "f32")
    assert hum.select_config(hd, m).kind == hum.KERNEL_STREAM
    x = dev(synth.bf16_normal(synth.rng(synth.seed_for(9, 400 + m)), (m, k)))
    out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    ws = hum.Workspace("cuda").get(hum.linear_workspace_bytes(hd, m))
    print(f"case graph linear {fmt} m={m}", flush=True)
    _replays_match([lambda: hum.linear(hd, packed, x, out=out, workspace=ws)], [out],
                   lambda: hum.linear(hd, packed, x[:1].contiguous()))


@pytest.mark.parametrize("act", ["bf16", "mxfp8", "mxfp4"])
@pytest.mark.parametrize("t", [1, 40])
def test_moe_graph_replay(act, t):
    e, h, inter, topk = 8, 256, 128, 2
    w13 = synth.moe_weights_mxfp4(740, e, 2 * inter, h)
    w2 = synth.moe_weights_mxfp4(741, e, h, inter)
    d13, _ = descs("e2m1", "group", 32, "e8m0", e, 2 * inter, h, act=act)
    d2, _ = descs("e2m1", "group", 32, "e8m0", e, h, inter, act=act)
    p13, p2 = prepare(d13, w13, "e8m0"), prepare(d2, w2, "e8m0")
    ids, wts = synth.routing(742 + t, t, e, topk)
    x = dev(synth.bf16_normal(synth.rng(743 + t), (t, h)))
    di, dw = dev(ids), dev(wts)
    out = torch.empty((t, h), dtype=torch.bfloat16, device="cuda")
    ws = hum.Workspace("cuda").get(hum.moe_workspace_bytes(d13, d2, t, topk))
    ids2, wts2 = synth.routing(744, 3, e, topk)
    x2 = dev(synth.bf16_normal(synth.rng(745), (3, h)))
    print(f"case graph moe act={act} t={t}", flush=True)
    _replays_match([lambda: hum.moe_gemm(d13, p13, d2, p2, x, di, dw, out=out, workspace=ws)], [out],
                   lambda: hum.moe_gemm(d13, p13, d2, p2, x2, dev(ids2), dev(wts2)))
