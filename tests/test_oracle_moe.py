"""Pins of the oracle's MoE pieces: align against Python's sorted(), the
reduce against its special cases, and the layer against a loop of dense
layers and the E=1 / top-1 / w=1 reduction to dense -> SwiGLU -> dense."""
import numpy as np
import pytest

from oracle import gemm as G
from oracle import moe as M
from oracle.formats import decode_bf16, encode_bf16
from synth import bf16_bits, moe_weights_mxfp4, routing


@pytest.mark.parametrize("t,k,e,bm", [(1, 8, 128, 16), (37, 8, 16, 4), (64, 2, 8, 1), (5, 3, 40, 64)])
def test_align_vs_sorted(t, k, e, bm):
    g = np.random.default_rng(t * 131 + e)
    ids = g.integers(0, e, size=(t, k)).astype(np.int32)
    srt, off, cnt = M.align(ids, e, bm)
    flat = ids.reshape(-1).tolist()
    order = sorted(range(t * k), key=lambda f: (flat[f], f))
    assert cnt.sum() == t * k
    assert off[0] == 0 and np.all(np.diff(off) >= 0) and np.all(off % bm == 0)
    pos = 0
    for ex in range(e):
        seg = srt[off[ex]:off[ex + 1]]
        real = [f for f in seg if f != t * k]
        assert real == order[pos:pos + cnt[ex]]
        assert all(f == t * k for f in seg[cnt[ex]:])
        assert len(seg) == -(-cnt[ex] // bm) * bm
        pos += cnt[ex]
    assert np.all(srt[off[e]:] == t * k)
    assert len(srt) == M.align_capacity(t, k, e, bm)


def test_align_block1_is_permutation():
    g = np.random.default_rng(5)
    ids = g.integers(0, 10, size=(50, 4))
    srt, off, cnt = M.align(ids, 10, 1)
    assert sorted(srt.tolist()) == list(range(200))
    assert np.array_equal(off[1:], np.cumsum(cnt))


def test_reduce_special_cases():
    g = np.random.default_rng(6)
    y = g.standard_normal((10, 7))
    out = M.reduce(y, np.ones((10, 1), np.float32), 1)
    assert np.array_equal(out, y)
    w = np.array([[0.25, 0.5, 0.25]], np.float32)
    yy = np.repeat(g.standard_normal((1, 7)), 3, axis=0)
    assert np.allclose(M.reduce(yy, w, 3), yy[:1], rtol=0, atol=1e-15)


def _small_layer(seed, e, hdim, inter):
    w13 = moe_weights_mxfp4(seed, e, 2 * inter, hdim)
    w2 = moe_weights_mxfp4(seed + 1, e, hdim, inter)
    d13 = G.WeightDesc("e2m1", "group", 32, "e8m0", False, False, e, 2 * inter, hdim)
    d2 = G.WeightDesc("e2m1", "group", 32, "e8m0", False, False, e, hdim, inter)
    return d13, w13, d2, w2


def _fp8_layer(seed, e, hdim, inter, gran):
    from synth import quant_weights
    gs = 128 if gran == "block" else 0
    w13 = quant_weights(seed, "e4m3", gran, gs, "f32", e, 2 * inter, hdim, scale_lo=0.0005, scale_hi=0.002)
    w2 = quant_weights(seed + 1, "e4m3", gran, gs, "f32", e, hdim, inter, scale_lo=0.0005, scale_hi=0.002)
    d13 = G.WeightDesc("e4m3", gran, gs, "f32", False, False, e, 2 * inter, hdim)
    d2 = G.WeightDesc("e4m3", gran, gs, "f32", False, False, e, hdim, inter)
    return d13, w13, d2, w2


def _fp8_qdq_ref(act):
    """Independent restatement of the FP8 stage rules for the loop below:
    the input row quantized by its own rule, the SwiGLU output rounded to
    bf16 first."""
    from oracle import quant as Q
    if act == "fp8_token":
        q = lambda a: Q.dequant_fp8_per_token(*Q.quant_fp8_per_token(np.asarray(a, np.float32)))
    else:
        q = lambda a: Q.dequant_fp8_group(*Q.quant_fp8_group(np.asarray(a, np.float32)))
    return q, (lambda a: q(decode_bf16(encode_bf16(a))))


@pytest.mark.parametrize("act", ["bf16", "mxfp8", "mxfp4", "fp8_token", "fp8_group"])
def test_moe_equals_loop_of_dense(act):
    e, hdim, inter, t, k = 6, 64, 32, 9, 3
    if act.startswith("fp8"):
        hdim, inter = 256, 128
        d13, w13, d2, w2 = _fp8_layer(30, e, hdim, inter, "block" if act == "fp8_group" else "channel")
        q_in, q_mid = _fp8_qdq_ref(act)
    else:
        d13, w13, d2, w2 = _small_layer(30, e, hdim, inter)
        qdq = {"mxfp8": M.qdq_mxfp8, "mxfp4": M.qdq_mxfp4}.get(act)
        q_in = (lambda a: a) if act == "bf16" else qdq
        q_mid = (lambda a: decode_bf16(encode_bf16(a))) if act == "bf16" else qdq
    g = np.random.default_rng(31)
    x = bf16_bits(g.standard_normal((t, hdim)).astype(np.float32))
    ids, wts = routing(32, t, e, k)
    out = M.moe_forward(d13, w13, d2, w2, x, ids, wts, act)
    a_in = q_in(decode_bf16(x))
    ref = np.zeros_like(out)
    for tt in range(t):
        for j in range(k):
            ex = int(ids[tt, j])
            h = G.linear(d13, a_in[tt:tt + 1], w13["codes"], w13["scales"], expert=ex)
            a = M.silu(h[:, :inter]) * h[:, inter:]
            a = q_mid(a)
            y = G.linear(d2, a, w2["codes"], w2["scales"], expert=ex)
            ref[tt] += float(wts[tt, j]) * y[0]
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_moe_single_expert_top1_is_dense_swiglu_dense():
    hdim, inter, t = 64, 32, 5
    d13, w13, d2, w2 = _small_layer(40, 1, hdim, inter)
    g = np.random.default_rng(41)
    x = bf16_bits(g.standard_normal((t, hdim)).astype(np.float32))
    ids = np.zeros((t, 1), np.int32)
    wts = np.ones((t, 1), np.float32)
    out = M.moe_forward(d13, w13, d2, w2, x, ids, wts, "bf16")
    w_gu = G.dequant_weight(d13, w13["codes"], w13["scales"])[0]
    w_dn = G.dequant_weight(d2, w2["codes"], w2["scales"])[0]
    h = decode_bf16(x) @ w_gu.T
    gate, up = h[:, :inter], h[:, inter:]
    a = gate * (1.0 / (1.0 + np.exp(-gate))) * up
    a = decode_bf16(encode_bf16(a))
    assert np.allclose(out, a @ w_dn.T, rtol=1e-13, atol=0)


def test_silu_closed_form_points():
    assert M.silu(0.0) == 0.0
    assert abs(M.silu(1.0) - 1.0 / (1.0 + np.exp(-1.0))) < 1e-16
    assert M.silu(-1000.0) == 0.0
    assert M.silu(1000.0) == 1000.0


def test_routing_generator_properties():
    ids, w = routing(7, 100, 128, 8)
    assert ids.shape == (100, 8) and w.dtype == np.float32
    assert all(len(set(r)) == 8 for r in ids.tolist())
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6)
    assert np.all(np.diff(w, axis=1) <= 1e-7)
    ids_z, _ = routing(8, 4096, 128, 8, zipf_s=1.1)
    cnt = np.bincount(ids_z.reshape(-1), minlength=128)
    assert cnt.max() > 5 * np.median(cnt)


@pytest.mark.parametrize("act", ["bf16", "mxfp8", "mxfp4"])
def test_masked_layout_equals_loop_of_dense(act):
    """grouped_masked: every valid row of every expert buffer is that
    expert's dense -> SwiGLU -> dense on the row alone; counts clamp to
    [0, max_m]; the other rows are not defined (zero, flagged invalid)."""
    e, hdim, inter, max_m = 4, 64, 32, 5
    d13, w13, d2, w2 = _small_layer(50, e, hdim, inter)
    g = np.random.default_rng(51)
    x = bf16_bits(g.standard_normal((e, max_m, hdim)).astype(np.float32))
    counts = np.array([5, 0, 2, 9], dtype=np.int32)
    out, valid = M.moe_masked(d13, w13, d2, w2, x, counts, act)
    assert valid.sum(axis=1).tolist() == [5, 0, 2, 5]
    qdq = {"mxfp8": M.qdq_mxfp8, "mxfp4": M.qdq_mxfp4}.get(act)
    for ex in range(e):
        for i in range(max_m):
            if not valid[ex, i]:
                assert not out[ex, i].any()
                continue
            a_in = decode_bf16(x[ex, i:i + 1])
            a_in = a_in if act == "bf16" else qdq(a_in)
            h = G.linear(d13, a_in, w13["codes"], w13["scales"], expert=ex)
            a = M.silu(h[:, :inter]) * h[:, inter:]
            a = decode_bf16(encode_bf16(a)) if act == "bf16" else qdq(a)
            y = G.linear(d2, a, w2["codes"], w2["scales"], expert=ex)[0]
            assert np.allclose(out[ex, i], y, rtol=1e-12, atol=1e-12 * np.abs(y).max()), (ex, i)
