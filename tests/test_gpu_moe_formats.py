"""GPU: the MoE layer (hum_moe_gemm) with every expert format of the common
description that has a MoE path -- NVFP4 and MXINT4 experts with bf16
activations, FP8 and INT8 experts with bf16 activations (W8A16), FP8
per-channel experts with per-token FP8 activations (W8A8) and 128 x 128
block-scaled FP8 experts with per-group FP8 activations -- against the
oracle at the bf16-output tolerance, on every compiled MoE tile and on the
selector's own choices.  Hidden 1024 and intermediate 512, so both GEMMs
run several K-blocks through the pipelined loops."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_packed_amd as hum
import synth
from gpu_util import (MAX_REL, MAX_REL_FP8_REQUANT_LAYER, REL_FRO, REL_FRO_FP8_REQUANT_LAYER, assert_tol, bf16_bits_of,
                      descs, dev, prepare)

pytestmark = pytest.mark.gpu

MOE_TILES = [(1, 1, 4, 1, 8), (1, 1, 4, 1, 15), (0, 1, 4, 4, 1), (0, 2, 4, 4, 1), (0, 4, 4, 4, 1), (0, 8, 4, 4, 1)]

# (name, weight dtype, granularity, group, scale dtype, global scale, activation format, scale range)
FORMATS = [
    ("nvfp4", "e2m1", "group", 16, "e4m3", True, "bf16", None),
    ("mxint4", "int4", "group", 32, "e8m0", False, "bf16", None),
    ("w8a16_fp8", "e4m3", "channel", 0, "f32", False, "bf16", (0.0005, 0.002)),
    ("w8a16_int8", "int8", "channel", 0, "f32", False, "bf16", (0.0002, 0.001)),
    ("w8a8_fp8_token", "e4m3", "channel", 0, "f32", False, "fp8_token", (0.0005, 0.002)),
    ("w8a8_fp8_block", "e4m3", "block", 128, "f32", False, "fp8_group", (0.0005, 0.002)),
]


def layer_tol(fmt):
    """The layer's bounds: FP8 activation formats requantize the SwiGLU
    output between the GEMMs (see gpu_util)."""
    if fmt.startswith("w8a8"):
        return dict(max_rel=MAX_REL_FP8_REQUANT_LAYER, rel_fro=REL_FRO_FP8_REQUANT_LAYER)
    return dict(max_rel=MAX_REL, rel_fro=REL_FRO)


def cfg(t):
    c = hum.TileConfig()
    c.kind, c.wave_m, c.wave_n, c.waves_n, c.waves_k = t
    c.split_k = 1
    c.block_m = 16 * t[1]
    return c


_CACHE = {}


def layer(fmt, e=8, h=1024, inter=512):
    key = (fmt, e, h, inter)
    if key in _CACHE:
        return _CACHE[key]
    name, wd, gr, gs, sd, glob, act, rng_ = next(f for f in FORMATS if f[0] == fmt)
    kw = {} if rng_ is None else dict(scale_lo=rng_[0], scale_hi=rng_[1])
    # (seeds fixed per format and shape, whatever order the tests run in)
    idx = synth.seed_of("moe-format", fmt, e, h, inter)
    w13 = synth.quant_weights(synth.seed_for(20, idx), wd, gr, gs, sd, e, 2 * inter, h, global_scale=glob, **kw)
    w2 = synth.quant_weights(synth.seed_for(21, idx), wd, gr, gs, sd, e, h, inter, global_scale=glob, **kw)
    d13, o13 = descs(wd, gr, gs, sd, e, 2 * inter, h, glob=glob, act=act)
    d2, o2 = descs(wd, gr, gs, sd, e, h, inter, glob=glob, act=act)
    _CACHE[key] = (w13, w2, d13, o13, d2, o2, prepare(d13, w13, sd), prepare(d2, w2, sd), act)
    return _CACHE[key]


@pytest.mark.parametrize("fmt", [f[0] for f in FORMATS])
@pytest.mark.parametrize("tile", MOE_TILES, ids=lambda t: "t" + "".join(map(str, t)))
@pytest.mark.parametrize("t", [1, 9, 70])
def test_moe_format_every_tile(fmt, tile, t):
    w13, w2, d13, o13, d2, o2, p13, p2, act = layer(fmt)
    e, k = 8, 2
    ids, wts = synth.routing(800 + t, t, e, k)
    xb = synth.bf16_normal(synth.rng(801 + t), (t, d13.k))
    print(f"case moe format={fmt} tile={tile} t={t}", flush=True)
    if fmt == "w8a8_fp8_block" and tile[0] == 1:
        with pytest.raises(hum.HumError, match="tile config not available"):
            hum.moe_gemm(d13, p13, d2, p2, dev(xb), dev(ids), dev(wts), cfg=cfg(tile))
        return
    out = hum.moe_gemm(d13, p13, d2, p2, dev(xb), dev(ids), dev(wts), cfg=cfg(tile))
    torch.cuda.synchronize()
    ref = oracle.moe.moe_forward(o13, w13, o2, w2, xb, ids, wts, act)
    assert_tol(out, ref, f"format={fmt} tile={tile} t={t}", **layer_tol(fmt))


@pytest.mark.parametrize("fmt", [f[0] for f in FORMATS])
@pytest.mark.parametrize("t", [1, 16, 100, 500])
def test_moe_format_default_selection(fmt, t):
    w13, w2, d13, o13, d2, o2, p13, p2, act = layer(fmt)
    e, k = 8, 2
    ids, wts = synth.routing(820 + t, t, e, k, zipf_s=1.2)
    xb = synth.bf16_normal(synth.rng(821 + t), (t, d13.k))
    print(f"case moe format default={fmt} t={t}", flush=True)
    out = hum.moe_gemm(d13, p13, d2, p2, dev(xb), dev(ids), dev(wts))
    torch.cuda.synchronize()
    ref = oracle.moe.moe_forward(o13, w13, o2, w2, xb, ids, wts, act)
    assert_tol(out, ref, f"default format={fmt} t={t}", **layer_tol(fmt))


@pytest.mark.parametrize("fmt", ["w8a8_fp8_token", "w8a8_fp8_block", "nvfp4"])
def test_moe_format_split_k(fmt):
    w13, w2, d13, o13, d2, o2, p13, p2, act = layer(fmt)
    e, k, t = 8, 2, 5
    ids, wts = synth.routing(840, t, e, k)
    xb = synth.bf16_normal(synth.rng(841), (t, d13.k))
    c = cfg((0, 1, 4, 4, 1))
    c.split_k = 2
    out = hum.moe_gemm(d13, p13, d2, p2, dev(xb), dev(ids), dev(wts), cfg=c)
    torch.cuda.synchronize()
    ref = oracle.moe.moe_forward(o13, w13, o2, w2, xb, ids, wts, act)
    assert_tol(out, ref, f"split-K format={fmt}", **layer_tol(fmt))


@pytest.mark.parametrize("fmt", ["w8a8_fp8_token", "w8a8_fp8_block", "mxint4"])
def test_moe_format_masked_layout(fmt):
    w13, w2, d13, o13, d2, o2, p13, p2, act = layer(fmt)
    e, max_m = 8, 64
    cnt = np.array([64, 0, 3, 17, 1, 40, 0, 9], np.int32)
    xb = synth.bf16_normal(synth.rng(850), (e, max_m, d13.k))
    out = hum.moe_gemm_masked(d13, p13, d2, p2, dev(xb), dev(cnt), 16)
    torch.cuda.synchronize()
    ref, valid = oracle.moe.moe_masked(o13, w13, o2, w2, xb, cnt, act)
    assert_tol(out[torch.from_numpy(valid).cuda()], ref[valid], f"masked format={fmt}", **layer_tol(fmt))


@pytest.mark.parametrize("fmt", [f[0] for f in FORMATS])
@pytest.mark.parametrize("tile", [(1, 1, 4, 1, 8), (0, 1, 4, 4, 1), (0, 4, 4, 4, 1)],
                         ids=lambda t: "t" + "".join(map(str, t)))
def test_moe_format_stages_at_gemm_tolerance(fmt, tile):
    """Each GEMM of the layer alone, at the bf16-output GEMM bound: gate_up
    with the bf16 SwiGLU epilogue on the layer input in its activation
    format, then down on the oracle's own intermediate (rounded to bf16 and,
    for FP8 activations, quantized with the format's rule)."""
    w13, w2, d13, o13, d2, o2, p13, p2, act = layer(fmt)
    if fmt == "w8a8_fp8_block" and tile[0] == 1:
        pytest.skip("block-scaled FP8 runs on the tile kernel only")
    e, k, t = 8, 2, 60
    bm = 16 * tile[1]
    ids, _ = synth.routing(860, t, e, k, zipf_s=1.2)
    srt, off, cnt = oracle.moe.align(ids, e, bm)
    xb = synth.bf16_normal(synth.rng(861), (t, d13.k))
    x64 = oracle.formats.decode_bf16(xb)
    if act == "bf16":
        a, a_s = dev(xb), None
    else:
        qf = {"fp8_token": oracle.quant.quant_fp8_per_token, "fp8_group": oracle.quant.quant_fp8_group}[act]
        q, s_ = qf(x64.astype(np.float32))
        a, a_s = dev(q), dev(s_)
    c = cfg(tile)
    print(f"case moe stages format={fmt} tile={tile}", flush=True)
    inter_gpu = hum.moe_grouped_gemm(d13, p13, a, dev(srt), dev(off), bm, t, k, a_mode="gather",
                                     epilogue="swiglu_bf16", a_scales=a_s, cfg=c)
    a_in = oracle.moe.quant_input(x64, act)
    inter = d2.k
    a_mid = np.zeros((len(srt), inter))
    for ex in range(e):
        seg = srt[off[ex]:off[ex] + cnt[ex]]
        if len(seg):
            hh = oracle.gemm.linear(o13, a_in[seg // k], w13["codes"], w13["scales"], w13.get("zeros"),
                                    w13.get("global_scale"), expert=ex)
            a_mid[off[ex]:off[ex] + cnt[ex]] = oracle.moe.swiglu(hh, inter)
    valid = srt < t * k
    torch.cuda.synchronize()
    assert_tol(inter_gpu[torch.from_numpy(valid).cuda()], a_mid[valid], f"gate_up format={fmt} tile={tile}")
    # down on the oracle's intermediate
    mid_b = oracle.moe.round_bf16(a_mid)
    if act == "bf16":
        a2, a2_s, a2v = dev(oracle.formats.encode_bf16(mid_b)), None, mid_b
    else:
        qf = {"fp8_token": oracle.quant.quant_fp8_per_token, "fp8_group": oracle.quant.quant_fp8_group}[act]
        q2, s2 = qf(mid_b.astype(np.float32))
        a2, a2_s, a2v = dev(q2), dev(s2), oracle.gemm.activations(act, q=q2, scales=s2)
    y = hum.moe_grouped_gemm(d2, p2, a2, dev(srt), dev(off), bm, t, k, a_mode="sorted", epilogue="scatter",
                             a_scales=a2_s, cfg=c)
    yref = np.zeros((t * k, d2.n))
    for ex in range(e):
        rows = np.arange(off[ex], off[ex] + cnt[ex])
        if len(rows):
            yref[srt[rows]] = oracle.gemm.linear(o2, a2v[rows], w2["codes"], w2["scales"], w2.get("zeros"),
                                                 w2.get("global_scale"), expert=ex)
    torch.cuda.synchronize()
    assert_tol(y, yref, f"down format={fmt} tile={tile}")


def test_fp8_mfma_accumulation_error():
    """The gfx950 FP8 x FP8 matrix instruction sums its 128-deep dot product
    below fp32 precision (bf16 x bf16 sums are fp32-exact to rounding): the
    gate_up GEMM's fp32 SwiGLU values, whose gate is at least 17 (so that
    silu(gate) is gate in fp32 and the SwiGLU is gate * up up to one fp32
    rounding), are compared with the oracle's exact gate * up.  Bound: 5e-4 of each row's largest value (measured 2.2e-4),
    against 2e-6 on the bf16 path with the same E4M3 weights."""
    e, h, inter, k, t = 4, 1024, 256, 2, 64
    g = synth.rng(880)
    res = {}
    for act in ("fp8_token", "bf16"):
        codes = np.zeros((e, 2 * inter, h), np.uint8)
        codes[:, :inter] = g.integers(0x30, 0x50, size=(e, inter, h)).astype(np.uint8)   # gate > 0: +0.5 .. +8
        cu = g.integers(0, 256, size=(e, inter, h)).astype(np.uint8)
        codes[:, inter:] = np.where((cu & 0x7F) == 0x7F, 0x7E, cu)
        w13 = {"codes": codes, "scales": np.full((e, 2 * inter, 1), 1.0, np.float32)}
        d13, o13 = descs("e4m3", "channel", 0, "f32", e, 2 * inter, h, act=act)
        p13 = prepare(d13, w13, "f32")
        ids, _ = synth.routing(881, t, e, k)
        srt, off, cnt = oracle.moe.align(ids, e, 16)
        x = np.abs(g.standard_normal((t, h))).astype(np.float32) + 0.25
        xb = synth.bf16_bits(x)
        x64 = oracle.formats.decode_bf16(xb)
        if act == "bf16":
            a, a_s, a_in = dev(xb), None, x64
        else:
            q, s_ = oracle.quant.quant_fp8_per_token(x64.astype(np.float32))
            a, a_s, a_in = dev(q), dev(s_), oracle.quant.dequant_fp8_per_token(q, s_)
        _, f32 = hum.moe_grouped_gemm(d13, p13, a, dev(srt), dev(off), 16, t, k, a_mode="gather",
                                      epilogue="swiglu_bf16", a_scales=a_s, keep_swiglu_f32=True)
        torch.cuda.synchronize()
        f32 = f32.cpu().numpy().astype(np.float64)
        worst = 0.0
        for ex in range(e):
            seg = srt[off[ex]:off[ex] + cnt[ex]]
            if len(seg) == 0:
                continue
            hh = oracle.gemm.linear(o13, a_in[seg // k], w13["codes"], w13["scales"], expert=ex)
            gate, up = hh[:, :inter], hh[:, inter:]
            assert gate.min() >= 17.0
            ex_a = gate * up
            rows = np.arange(off[ex], off[ex] + cnt[ex])
            worst = max(worst, float((np.abs(f32[rows] - ex_a) / np.abs(ex_a).max(axis=1, keepdims=True)).max()))
        res[act] = worst
    print("FP8 x FP8 / bf16 path error (of the row max):", res, flush=True)
    assert res["fp8_token"] <= 5e-4 and res["bf16"] <= 2e-6, res
