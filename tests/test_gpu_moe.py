"""GPU: MoE pieces against the oracle -- align (bit exact), weighted reduce,
and the full layer (hum_moe_gemm) for MXFP4 W4A16, W4A8 and W4A4 on every
compiled tile shape, with skewed / empty / single-expert routings."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_packed_amd as hum
import synth
from gpu_util import assert_tol, descs, dev, prepare

pytestmark = pytest.mark.gpu

# (kind, wave_m, wave_n, waves_n, waves_k): every compiled MoE instance
MOE_TILES = [(1, 1, 4, 1, 8), (1, 1, 4, 1, 15), (0, 1, 4, 4, 1), (0, 2, 4, 4, 1), (0, 4, 4, 4, 1), (0, 8, 4, 4, 1)]


def cfg(t, split=1):
    c = hum.TileConfig()
    c.kind, c.wave_m, c.wave_n, c.waves_n, c.waves_k = t
    c.split_k = split
    c.block_m = 16 * t[1]
    return c


@pytest.mark.parametrize("multi", [False, True], ids=["one-wg", "multi-wg"])
@pytest.mark.parametrize("t,k,e,bm,zipf", [(1, 8, 128, 16, None), (37, 8, 16, 32, None), (300, 4, 64, 64, None),
                                           (4096, 8, 128, 128, 1.1), (8192, 8, 128, 16, 1.1), (5, 3, 7, 1, None),
                                           (1025, 8, 128, 64, None), (3000, 7, 512, 16, 1.1), (2049, 4, 3, 128, None),
                                           (8, 8, 128, 16, None), (21, 3, 512, 128, None), (2, 8, 3, 32, None),
                                           (13, 5, 16, 16, None)])
def test_align_bit_exact(t, k, e, bm, zipf, multi):
    """The stable sort bit for bit, by one workgroup and by the multi-
    workgroup path (chunks of 4096 slots: ragged last chunk, 512 experts,
    three experts); tables of at most 64 slots take the one-wave sort (64
    slots exactly, 512 experts with 128-row blocks, three experts; 65 slots
    is the first table past it)."""
    ids, _ = synth.routing(500 + t, t, e, k, zipf_s=zipf)
    print(f"case align t={t} k={k} e={e} bm={bm} multi={multi}", flush=True)
    srt, off, cnt = hum.moe_align(dev(ids), e, bm, multi_workgroup=multi)
    torch.cuda.synchronize()
    rs, ro, rc = oracle.moe.align(ids, e, bm)
    assert np.array_equal(cnt.cpu().numpy(), rc)
    assert np.array_equal(off.cpu().numpy(), ro)
    assert np.array_equal(srt.cpu().numpy(), rs)


def test_align_all_to_one_expert():
    t, k, e = 300, 2, 16
    ids = np.full((t, k), 5, np.int32)
    ids[:, 1] = 9
    srt, off, cnt = hum.moe_align(dev(ids), e, 64)
    torch.cuda.synchronize()
    rs, ro, rc = oracle.moe.align(ids, e, 64)
    assert np.array_equal(srt.cpu().numpy(), rs) and np.array_equal(off.cpu().numpy(), ro)


@pytest.mark.parametrize("t,k,h", [(1, 8, 4096), (33, 8, 256), (7, 1, 64)])
def test_reduce_vs_oracle(t, k, h):
    g = synth.rng(600 + t)
    y = synth.bf16_normal(g, (t * k, h))
    _, w = synth.routing(601 + t, t, 16, k)
    out = hum.moe_reduce(dev(y), dev(w))
    torch.cuda.synchronize()
    ref = oracle.moe.reduce(oracle.formats.decode_bf16(y), w, k)
    got = out.float().cpu().numpy().astype(np.float64)
    # one bf16 rounding of an fp32 sum: within 2^-8 relative per element
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)


def _layer(seed, e, h, inter, act):
    w13 = synth.moe_weights_mxfp4(seed, e, 2 * inter, h)
    w2 = synth.moe_weights_mxfp4(seed + 1, e, h, inter)
    d13, o13 = descs("e2m1", "group", 32, "e8m0", e, 2 * inter, h, act=act)
    d2, o2 = descs("e2m1", "group", 32, "e8m0", e, h, inter, act=act)
    return w13, w2, d13, o13, d2, o2, prepare(d13, w13, "e8m0"), prepare(d2, w2, "e8m0")


@pytest.mark.parametrize("act", ["bf16", "mxfp8", "mxfp4"])
@pytest.mark.parametrize("tile", MOE_TILES, ids=lambda t: "t" + "".join(map(str, t)))
@pytest.mark.parametrize("t", [1, 9, 70])
def test_moe_layer_every_tile(act, tile, t):
    e, h, inter, k = 8, 1024, 512, 2
    w13, w2, d13, o13, d2, o2, p13, p2 = _layer(700, e, h, inter, act)
    ids, wts = synth.routing(701 + t, t, e, k)
    xb = synth.bf16_normal(synth.rng(702 + t), (t, h))
    print(f"case moe act={act} tile={tile} t={t}", flush=True)
    if act == "mxfp4" and tile[0] == 1:
        # W4A4 has no decode-kernel instances
        with pytest.raises(hum.HumError, match="tile config not available"):
            hum.moe_gemm(d13, p13, d2, p2, dev(xb), dev(ids), dev(wts), cfg=cfg(tile))
        return
    out = hum.moe_gemm(d13, p13, d2, p2, dev(xb), dev(ids), dev(wts), cfg=cfg(tile))
    torch.cuda.synchronize()
    ref = oracle.moe.moe_forward(o13, w13, o2, w2, xb, ids, wts, act)
    assert_tol(out, ref, f"act={act} tile={tile} t={t}")


@pytest.mark.parametrize("act", ["bf16", "mxfp8"])
@pytest.mark.parametrize("wm", [2, 4])
@pytest.mark.parametrize("t,inter", [(9, 512), (300, 512), (40, 256)])
def test_moe_layer_three_stages(act, wm, t, inter):
    """The three-stage MoE tiles (gathered gate_up with the SwiGLU epilogue,
    sorted down with the staged scatter), including a down GEMM of two
    K-blocks, fewer than the stages."""
    e, h, k = 8, 1024, 2
    w13, w2, d13, o13, d2, o2, p13, p2 = _layer(720, e, h, inter, act)
    ids, wts = synth.routing(721 + t, t, e, k)
    xb = synth.bf16_normal(synth.rng(722 + t), (t, h))
    c = cfg((0, wm, 4, 4, 1))
    c.stages = 3
    print(f"case moe three stages act={act} wm={wm} t={t} inter={inter}", flush=True)
    out = hum.moe_gemm(d13, p13, d2, p2, dev(xb), dev(ids), dev(wts), cfg=c)
    torch.cuda.synchronize()
    ref = oracle.moe.moe_forward(o13, w13, o2, w2, xb, ids, wts, act)
    assert_tol(out, ref, f"three stages act={act} wm={wm} t={t}")


@pytest.mark.parametrize("act", ["bf16", "mxfp8"])
@pytest.mark.parametrize("tile", [(1, 1, 4, 1, 8), (0, 2, 4, 4, 1)], ids=["stream", "tile"])
def test_moe_split_k(act, tile):
    e, h, inter, k, t = 4, 2048, 256, 2, 3
    w13, w2, d13, o13, d2, o2, p13, p2 = _layer(710, e, h, inter, act)
    ids, wts = synth.routing(711, t, e, k)
    xb = synth.bf16_normal(synth.rng(712), (t, h))
    out = hum.moe_gemm(d13, p13, d2, p2, dev(xb), dev(ids), dev(wts), cfg=cfg(tile, split=2))
    torch.cuda.synchronize()
    ref = oracle.moe.moe_forward(o13, w13, o2, w2, xb, ids, wts, act)
    assert_tol(out, ref, f"split act={act}")


def test_moe_stream_wave_n2_bf16():
    e, h, inter, k, t = 8, 256, 128, 2, 9
    w13, w2, d13, o13, d2, o2, p13, p2 = _layer(705, e, h, inter, "bf16")
    ids, wts = synth.routing(706, t, e, k)
    xb = synth.bf16_normal(synth.rng(707), (t, h))
    out = hum.moe_gemm(d13, p13, d2, p2, dev(xb), dev(ids), dev(wts), cfg=cfg((1, 1, 2, 1, 8)))
    torch.cuda.synchronize()
    ref = oracle.moe.moe_forward(o13, w13, o2, w2, xb, ids, wts, "bf16")
    assert_tol(out, ref, "stream wave_n=2")


@pytest.mark.parametrize("act", ["bf16", "mxfp8", "mxfp4"])
def test_moe_skewed_and_empty_experts(act):
    e, h, inter, k, t = 16, 1024, 512, 4, 200
    w13, w2, d13, o13, d2, o2, p13, p2 = _layer(720, e, h, inter, act)
    ids, wts = synth.routing(721, t, e, k, zipf_s=1.5)
    ids[:, 0] = 3                                  # one expert gets every token
    ids = np.where(ids == 7, 8, ids).astype(np.int32)   # expert 7 gets none
    ids[:, 1] = np.where(ids[:, 1] == 3, 11, ids[:, 1])
    xb = synth.bf16_normal(synth.rng(722), (t, h))
    out = hum.moe_gemm(d13, p13, d2, p2, dev(xb), dev(ids), dev(wts))
    torch.cuda.synchronize()
    ref = oracle.moe.moe_forward(o13, w13, o2, w2, xb, ids, wts, act)
    assert_tol(out, ref, f"skewed act={act}")


def test_moe_single_expert_equals_dense_chain():
    """E = 1, top-1, w = 1: the layer is dense gate_up -> SwiGLU -> dense down."""
    h, inter, t = 256, 128, 11
    w13, w2, d13, o13, d2, o2, p13, p2 = _layer(730, 1, h, inter, "bf16")
    ids = np.zeros((t, 1), np.int32)
    wts = np.ones((t, 1), np.float32)
    xb = synth.bf16_normal(synth.rng(731), (t, h))
    x = dev(xb)
    out = hum.moe_gemm(d13, p13, d2, p2, x, dev(ids), dev(wts))
    hh = hum.linear(d13, p13, x).float()                # bf16-rounded h
    torch.cuda.synchronize()
    ref = oracle.moe.moe_forward(o13, w13, o2, w2, xb, ids, wts, "bf16")
    assert_tol(out, ref, "E=1 vs oracle")
    gate, up = hh[:, :inter], hh[:, inter:]
    a = (gate / (1 + torch.exp(-gate)) * up).to(torch.bfloat16)
    chain = hum.linear(d2, p2, a)
    torch.cuda.synchronize()
    assert_tol(out, chain.float().cpu().numpy().astype(np.float64), "E=1 vs dense chain")


@pytest.mark.parametrize("act", ["bf16", "mxfp8", "mxfp4"])
@pytest.mark.parametrize("t", [1, 16, 100, 500, 1200])
def test_moe_default_selection_every_regime(act, t):
    """The selector's choices over the rows-per-expert range (decode kernel,
    16-row tiles, decode gate_up with a tiled down GEMM, larger tiles)."""
    e, h, inter, k = 8, 1024, 512, 2
    w13, w2, d13, o13, d2, o2, p13, p2 = _layer(740, e, h, inter, act)
    ids, wts = synth.routing(741 + t, t, e, k)
    xb = synth.bf16_normal(synth.rng(742 + t), (t, h))
    print(f"case moe default act={act} t={t}", flush=True)
    out = hum.moe_gemm(d13, p13, d2, p2, dev(xb), dev(ids), dev(wts))
    torch.cuda.synchronize()
    ref = oracle.moe.moe_forward(o13, w13, o2, w2, xb, ids, wts, act)
    assert_tol(out, ref, f"default act={act} t={t}")


@pytest.mark.parametrize("act", ["bf16", "mxfp8", "mxfp4"])
def test_moe_zero_tokens_is_a_no_op(act):
    e, h, inter, k = 8, 256, 128, 2
    w13, w2, d13, o13, d2, o2, p13, p2 = _layer(750, e, h, inter, act)
    x = torch.empty((0, h), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((0, k), dtype=torch.int32, device="cuda")
    wts = torch.empty((0, k), dtype=torch.float32, device="cuda")
    out = hum.moe_gemm(d13, p13, d2, p2, x, ids, wts)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (0, h)


# ---- grouped_masked layout ---------------------------------------------------

_UNTOUCHED = 0x3F81  # bf16 bits of 1.0078125: rows past a count must keep it


def _masked_case(seed, e, max_m, h, counts):
    xb = synth.bf16_normal(synth.rng(seed), (e, max_m, h))
    cnt = np.asarray(counts, dtype=np.int32)
    out = torch.full((e, max_m, h), _UNTOUCHED, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    return xb, cnt, out


def _check_masked(out, ref, valid, what):
    bits = out.view(torch.int16).cpu().numpy()
    assert np.all(bits[~valid] == _UNTOUCHED), f"{what}: rows past a count were written"
    if valid.any():
        assert_tol(out[torch.from_numpy(valid).cuda()], ref[valid], what)


@pytest.mark.parametrize("act", ["bf16", "mxfp8", "mxfp4"])
@pytest.mark.parametrize("tile", MOE_TILES, ids=lambda t: "t" + "".join(map(str, t)))
def test_moe_masked_every_tile(act, tile):
    e, h, inter, max_m = 8, 1024, 512, 128
    w13, w2, d13, o13, d2, o2, p13, p2 = _layer(720, e, h, inter, act)
    xb, cnt, out = _masked_case(721, e, max_m, h, [128, 0, 1, 17, 33, 140, 5, 100])
    print(f"case moe masked act={act} tile={tile}", flush=True)
    if act == "mxfp4" and tile[0] == 1:
        with pytest.raises(hum.HumError, match="tile config not available"):
            hum.moe_gemm_masked(d13, p13, d2, p2, dev(xb), dev(cnt), 16, out=out, cfg=cfg(tile))
        return
    hum.moe_gemm_masked(d13, p13, d2, p2, dev(xb), dev(cnt), 16, out=out, cfg=cfg(tile))
    torch.cuda.synchronize()
    ref, valid = oracle.moe.moe_masked(o13, w13, o2, w2, xb, cnt, act)
    _check_masked(out, ref, valid, f"masked act={act} tile={tile}")


@pytest.mark.parametrize("act", ["bf16", "mxfp8", "mxfp4"])
@pytest.mark.parametrize("expected_m", [1, 20, 200])
def test_moe_masked_selector(act, expected_m):
    """Default tiles from expected_m; max_m = 48 makes 64-row tiles step down."""
    e, h, inter, max_m = 8, 1024, 512, 48
    w13, w2, d13, o13, d2, o2, p13, p2 = _layer(730, e, h, inter, act)
    g = synth.rng(731 + expected_m)
    xb, cnt, out = _masked_case(732 + expected_m, e, max_m, h, g.integers(0, max_m + 1, size=e))
    hum.moe_gemm_masked(d13, p13, d2, p2, dev(xb), dev(cnt), expected_m, out=out)
    torch.cuda.synchronize()
    ref, valid = oracle.moe.moe_masked(o13, w13, o2, w2, xb, cnt, act)
    _check_masked(out, ref, valid, f"masked act={act} expected_m={expected_m}")


@pytest.mark.parametrize("act", ["bf16", "mxfp8"])
def test_moe_masked_equals_indexed_top1(act):
    """Tokens routed top-1 with weight 1, laid out per expert: each masked
    row equals that token's indexed-layer output bitwise (same tile kernels;
    each row is summed in one order whatever the other rows are)."""
    e, h, inter, t, max_m = 8, 256, 128, 40, 16
    w13, w2, d13, o13, d2, o2, p13, p2 = _layer(740, e, h, inter, act)
    g = synth.rng(741)
    ids = g.integers(0, e, size=(t, 1)).astype(np.int32)
    cnt_all = np.bincount(ids[:, 0], minlength=e)
    keep = np.ones(t, dtype=bool)
    for ex in range(e):   # at most max_m tokens per expert
        keep[np.nonzero(ids[:, 0] == ex)[0][max_m:]] = False
    ids = ids[keep]
    t = ids.shape[0]
    wts = np.ones((t, 1), dtype=np.float32)
    xb = synth.bf16_normal(synth.rng(742), (t, h))
    xm = np.zeros((e, max_m, h), dtype=np.uint16)
    slot = np.zeros(t, dtype=np.int64)
    cnt = np.zeros(e, dtype=np.int32)
    for tt in range(t):
        ex = int(ids[tt, 0])
        slot[tt] = ex * max_m + cnt[ex]
        xm[ex, cnt[ex]] = xb[tt]
        cnt[ex] += 1
    assert cnt.sum() == t and cnt_all.sum() >= t
    tile = (0, 1, 4, 4, 1)
    ind = hum.moe_gemm(d13, p13, d2, p2, dev(xb), dev(ids), dev(wts), cfg=cfg(tile))
    msk = hum.moe_gemm_masked(d13, p13, d2, p2, dev(xm), dev(cnt), max_m, cfg=cfg(tile))
    torch.cuda.synchronize()
    got = msk.view(torch.int16).reshape(e * max_m, h).cpu().numpy()[slot]
    assert np.array_equal(got, ind.view(torch.int16).cpu().numpy())


def test_moe_masked_edges():
    e, h, inter = 4, 256, 128
    w13, w2, d13, o13, d2, o2, p13, p2 = _layer(750, e, h, inter, "bf16")
    empty = torch.zeros((e, 0, h), dtype=torch.bfloat16, device="cuda")
    cnt = dev(np.zeros(e, dtype=np.int32))
    assert hum.moe_gemm_masked(d13, p13, d2, p2, empty, cnt, 4).shape == (e, 0, h)
    with pytest.raises(hum.HumError, match="multiple of 16"):
        hum.moe_gemm_masked(d13, p13, d2, p2, torch.zeros((e, 24, h), dtype=torch.bfloat16, device="cuda"), cnt, 4)
    with pytest.raises(hum.HumError, match="must divide max_m"):
        hum.moe_gemm_masked(d13, p13, d2, p2, torch.zeros((e, 48, h), dtype=torch.bfloat16, device="cuda"), cnt, 4,
                            cfg=cfg((0, 2, 4, 4, 1)))
    # all counts zero: nothing written
    xb, c0, out = _masked_case(751, e, 32, h, [0, 0, 0, 0])
    hum.moe_gemm_masked(d13, p13, d2, p2, dev(xb), dev(c0), 4, out=out)
    torch.cuda.synchronize()
    assert np.all(out.view(torch.int16).cpu().numpy() == _UNTOUCHED)


@pytest.mark.parametrize("act", ["bf16", "mxfp8", "mxfp4"])
@pytest.mark.parametrize("t", [40, 13])
def test_moe_invalid_expert_ids_contribute_nothing(act, t):
    """Slots routed to an id outside [0, E) (-1: an expert held elsewhere, or
    E itself) add nothing: the same as a valid id with weight 0 (13 tokens x
    top-3: the one-wave sort)."""
    e, h, inter, k = 8, 256, 128, 3
    w13, w2, d13, o13, d2, o2, p13, p2 = _layer(760, e, h, inter, act)
    ids, wts = synth.routing(761, t, e, k)
    bad = np.zeros_like(ids, dtype=bool)
    bad[::3, 0] = True
    bad[1::5, 2] = True
    ids_bad = ids.copy()
    ids_bad[bad] = -1
    ids_bad[7, 1] = e
    bad[7, 1] = True
    xb = synth.bf16_normal(synth.rng(762), (t, h))
    # a first call leaves other rows in the workspace's slot buffer
    hum.moe_gemm(d13, p13, d2, p2, dev(xb), dev(ids), dev(wts))
    out = hum.moe_gemm(d13, p13, d2, p2, dev(xb), dev(ids_bad), dev(wts))
    torch.cuda.synchronize()
    ids_ref = np.where(bad, 0, ids).astype(np.int32)
    wts_ref = np.where(bad, 0.0, wts).astype(np.float32)
    ref = oracle.moe.moe_forward(o13, w13, o2, w2, xb, ids_ref, wts_ref, act)
    assert_tol(out, ref, f"invalid ids act={act}")


@pytest.mark.parametrize("act", ["bf16", "mxfp8"])
@pytest.mark.parametrize("t", [1, 2, 5])
def test_moe_wide_hidden_decode(act, t):
    """H = 5120 (40 K-blocks): the gate_up decode kernel's K range would
    overflow LDS at 16 rows without more split-K; the selector must pick a
    configuration that runs."""
    e, h, inter, k = 16, 5120, 256, 8
    w13, w2, d13, o13, d2, o2, p13, p2 = _layer(770, e, h, inter, act)
    ids, wts = synth.routing(771 + t, t, e, k)
    xb = synth.bf16_normal(synth.rng(772 + t), (t, h))
    print(f"case moe wide act={act} t={t} up={hum.moe_select_config(d13, d2, t, k, gate_up=True)}", flush=True)
    out = hum.moe_gemm(d13, p13, d2, p2, dev(xb), dev(ids), dev(wts))
    torch.cuda.synchronize()
    ref = oracle.moe.moe_forward(o13, w13, o2, w2, xb, ids, wts, act)
    assert_tol(out, ref, f"wide act={act} t={t}")


@pytest.mark.parametrize("act", ["bf16", "mxfp8"])
@pytest.mark.parametrize("t,k,e", [(1, 8, 128), (7, 8, 128), (4, 16, 40), (5, 3, 7), (21, 3, 16), (2, 8, 512)])
def test_moe_decode_routing_matches_align(act, t, k, e):
    """At most 64 routed slots: the gate_up decode kernel routes the slots
    itself (no align launch) and leaves the sorted rows, block map and live
    row count for the down GEMM.  The layer must equal, bit for bit, the same
    kernels run stage by stage after the align."""
    h, inter = 512, 256
    w13, w2, d13, o13, d2, o2, p13, p2 = _layer(780 + t, e, h, inter, act)
    ids, wts = synth.routing(781 + t, t, e, k)
    xb = synth.bf16_normal(synth.rng(782 + t), (t, h))
    up = hum.moe_select_config(d13, d2, t, k, gate_up=True)
    dn = hum.moe_select_config(d13, d2, t, k)
    assert up.kind == hum.KERNEL_STREAM and up.block_m == 16 and dn.block_m == 16, (up, dn)
    print(f"case moe routing act={act} t={t} k={k} e={e}", flush=True)
    x, di, dw = dev(xb), dev(ids), dev(wts)
    out = hum.moe_gemm(d13, p13, d2, p2, x, di, dw)
    srt, off, _ = hum.moe_align(di, e, 16)
    if act == "bf16":
        a, a_s, epi = x, None, "swiglu_bf16"
    else:
        a, a_s = hum.quant_act("mxfp8", x)
        epi = "swiglu_mxfp8"
    mid = hum.moe_grouped_gemm(d13, p13, a, srt, off, 16, t, k, a_mode="gather", epilogue=epi, a_scales=a_s, cfg=up)
    ia, ia_s = (mid, None) if act == "bf16" else mid
    y = hum.moe_grouped_gemm(d2, p2, ia, srt, off, 16, t, k, a_mode="sorted", epilogue="scatter", a_scales=ia_s,
                             cfg=dn)
    ref = hum.moe_reduce(y, dw)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    o = oracle.moe.moe_forward(o13, w13, o2, w2, xb, ids, wts, act)
    assert_tol(out, o, f"routing act={act} t={t}")


@pytest.mark.parametrize("t", [1, 3, 8])
def test_w4a4_decode_gate_up_matches_tiles_and_oracle(t):
    """W4A4 layers of up to 64 routed slots run gate_up on the E4M3 x E2M1
    decode kernel (the MXFP4 activations handed over as the E4M3 bytes of the
    same values, the SwiGLU output requantized to MXFP4) and down on the
    16-row W4A4 tile: the layer matches the all-tile path (the same products,
    summed by another matrix instruction) and the oracle."""
    e, h, inter, k = 16, 1024, 512, 4
    w13, w2, d13, o13, d2, o2, p13, p2 = _layer(770, e, h, inter, "mxfp4")
    assert hum.moe_select_config(d13, d2, t, k, gate_up=True).kind == hum.KERNEL_STREAM
    ids, wts = synth.routing(771 + t, t, e, k)
    xb = synth.bf16_normal(synth.rng(772 + t), (t, h))
    print(f"case w4a4 decode gate_up t={t}", flush=True)
    out = hum.moe_gemm(d13, p13, d2, p2, dev(xb), dev(ids), dev(wts))
    out_tiles = hum.moe_gemm(d13, p13, d2, p2, dev(xb), dev(ids), dev(wts), cfg=cfg((0, 1, 4, 4, 1)))
    torch.cuda.synchronize()
    ref = oracle.moe.moe_forward(o13, w13, o2, w2, xb, ids, wts, "mxfp4")
    assert_tol(out, ref, f"decode gate_up t={t}")
    assert_tol(out, out_tiles.float().cpu().numpy().astype(np.float64), f"decode vs tiles t={t}")


@pytest.mark.parametrize("act", ["bf16", "mxfp8", "mxfp4"])
@pytest.mark.parametrize("t", [1, 5])
def test_moe_decode_tokens_without_routed_slots(act, t):
    """Decode sizes (in-kernel routing, no align launch): a token none of
    whose slots is routed here (every id outside [0, E)) gets a zero row,
    whatever `out` held; partly routed tokens sum their routed slots only;
    the next call on the same workspace is unaffected."""
    e, h, inter, k = 8, 512, 256, 4
    w13, w2, d13, o13, d2, o2, p13, p2 = _layer(790, e, h, inter, act)
    ids, wts = synth.routing(791 + t, t, e, k)
    bad = np.zeros_like(ids, dtype=bool)
    bad[0, :] = True
    if t > 2:
        bad[2, 1] = True
    ids_bad = np.where(bad, -1, ids).astype(np.int32)
    if t > 2:
        ids_bad[2, 1] = e
    xb = synth.bf16_normal(synth.rng(792 + t), (t, h))
    out = torch.full((t, h), 7.0, dtype=torch.bfloat16, device="cuda")
    print(f"case moe unrouted tokens act={act} t={t}", flush=True)
    hum.moe_gemm(d13, p13, d2, p2, dev(xb), dev(ids_bad), dev(wts), out=out)
    torch.cuda.synchronize()
    assert torch.equal(out[0].view(torch.int16), torch.zeros(h, dtype=torch.int16, device="cuda"))
    ids_ref = np.where(bad, 0, ids).astype(np.int32)
    wts_ref = np.where(bad, 0.0, wts).astype(np.float32)
    ref = oracle.moe.moe_forward(o13, w13, o2, w2, xb, ids_ref, wts_ref, act)
    if t > 1:
        assert_tol(out[1:], ref[1:], f"partly routed act={act} t={t}")
    out2 = hum.moe_gemm(d13, p13, d2, p2, dev(xb), dev(ids), dev(wts))
    torch.cuda.synchronize()
    assert_tol(out2, oracle.moe.moe_forward(o13, w13, o2, w2, xb, ids, wts, act), f"next call act={act} t={t}")
