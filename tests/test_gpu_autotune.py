"""GPU: on-device autotune (hum_autotune_linear).

The returned configuration must be one the library runs, `out` must hold
exactly what hum_linear_ex gives with it, and that result must meet the
oracle's tolerance; the batch-invariant flag and the workspace bound must
restrict the candidates."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_packed_amd as hum
import synth
from gpu_util import assert_tol, descs, dev, prepare

pytestmark = pytest.mark.gpu


def _int_layer(n=1024, k=2048):
    w = synth.quant_weights(synth.seed_for(13), "uint4", "group", 128, "bf16", 1, n, k, zero=True)
    hd, od = descs("uint4", "group", 128, "bf16", 1, n, k, zero=True)
    return w, hd, od, prepare(hd, w, "bf16")


@pytest.mark.parametrize("m", [1, 64, 700])
def test_autotune_result_matches_its_config(m):
    w, hd, od, packed = _int_layer()
    xb = synth.bf16_normal(synth.rng(synth.seed_for(13, m)), (m, hd.k))
    xd = dev(xb)
    out = torch.empty((m, hd.n), dtype=torch.bfloat16, device="cuda")
    print(f"case autotune m={m}", flush=True)
    best, us = hum.autotune_linear(hd, packed, xd, out=out, iters=3)
    assert us > 0
    again = hum.linear(hd, packed, xd, cfg=best)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), again.view(torch.int16)), best
    ref = oracle.gemm.linear(od, oracle.formats.decode_bf16(xb), w["codes"], w["scales"], w["zeros"])
    assert_tol(out, ref, f"autotune m={m} cfg={best}")
    if m > 16:
        assert best.kind in (hum.KERNEL_TILE, hum.KERNEL_TILE32)   # the decode kernel takes at most 16 rows


def test_autotune_batch_invariant_candidates_only():
    w, hd, od, packed = _int_layer()
    xd = dev(synth.bf16_normal(synth.rng(synth.seed_for(13, 2)), (8, hd.k)))
    best, _ = hum.autotune_linear(hd, packed, xd, iters=2, batch_invariant=True)
    assert best.kind == hum.KERNEL_TILE and best.split_k == 1


def test_autotune_respects_workspace():
    n, k, m = 512, 1024, 40
    w = synth.dense_w8a8(synth.seed_for(13, 3), 1, n, k)
    hd, od = descs("e4m3", "channel", 0, "f32", 1, n, k, act="bf16")
    packed = prepare(hd, w, "f32")
    xb = synth.bf16_normal(synth.rng(synth.seed_for(13, 4)), (m, k))
    empty = torch.empty(0, dtype=torch.uint8, device="cuda")
    out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    best, _ = hum.autotune_linear(hd, packed, dev(xb), out=out, workspace=empty, iters=2)
    assert best.split_k == 1
    torch.cuda.synchronize()
    assert_tol(out, oracle.gemm.linear(od, oracle.formats.decode_bf16(xb), w["codes"], w["scales"]), "ws=0")
    # the integer tile kernel needs row sums in the workspace, and M = 40 is
    # beyond the decode kernel: nothing fits
    _, hdi, _, pi = _int_layer(256, 1024)
    with pytest.raises(hum.HumError, match="no compiled configuration"):
        hum.autotune_linear(hdi, pi, dev(xb), workspace=empty, iters=1)


@pytest.mark.parametrize("act", ["bf16", "mxfp8"])
def test_autotune_moe(act):
    """The MoE autotune's winner reproduces `out` bitwise and meets the
    oracle's tolerance; the invariant flag keeps it on tile kernels."""
    e, h, inter, t, topk = 8, 256, 128, 20, 2
    w13 = synth.moe_weights_mxfp4(synth.seed_for(14), e, 2 * inter, h)
    w2 = synth.moe_weights_mxfp4(synth.seed_for(14, 1), e, h, inter)
    d13, o13 = descs("e2m1", "group", 32, "e8m0", e, 2 * inter, h, act=act)
    d2, o2 = descs("e2m1", "group", 32, "e8m0", e, h, inter, act=act)
    p13, p2 = prepare(d13, w13, "e8m0"), prepare(d2, w2, "e8m0")
    ids, wts = synth.routing(synth.seed_for(14, 2), t, e, topk)
    xb = synth.bf16_normal(synth.rng(synth.seed_for(14, 3)), (t, h))
    out = torch.empty((t, h), dtype=torch.bfloat16, device="cuda")
    print(f"case autotune moe act={act}", flush=True)
    best, us = hum.autotune_moe(d13, p13, d2, p2, dev(xb), dev(ids), dev(wts), out=out, iters=2)
    assert us > 0
    again = hum.moe_gemm(d13, p13, d2, p2, dev(xb), dev(ids), dev(wts), cfg=best)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), again.view(torch.int16)), best
    assert_tol(out, oracle.moe.moe_forward(o13, w13, o2, w2, xb, ids, wts, act), f"autotune moe {act} {best}")
    inv, _ = hum.autotune_moe(d13, p13, d2, p2, dev(xb), dev(ids), dev(wts), iters=1, batch_invariant=True)
    assert inv.kind == hum.KERNEL_TILE
