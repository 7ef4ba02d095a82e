"""GPU: batch-invariant selection (HUM_SELECT_BATCH_INVARIANT).

With the configuration the library selects under the flag for each m, a
row's bf16 result must be bitwise the same whatever m is and whichever rows
surround it, for every weight / activation format; the results also meet the
oracle's bf16-output tolerance.  The MoE layer's tokens likewise must not
depend on the other tokens of the call."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_packed_amd as hum
import synth
from gpu_util import assert_tol, descs, dev, prepare

pytestmark = pytest.mark.gpu

# name -> (weight dtype, granularity, group, scale dtype, zero point, activation format)
FORMATS = {
    "uint4_zp_g128": ("uint4", "group", 128, "bf16", True, "bf16"),
    "int4_channel_f32": ("int4", "channel", 0, "f32", False, "bf16"),
    "e4m3_fp8_token": ("e4m3", "channel", 0, "f32", False, "fp8_token"),
    "e4m3_bf16": ("e4m3", "channel", 0, "f32", False, "bf16"),
    "int8_bf16": ("int8", "channel", 0, "f32", False, "bf16"),
    "e4m3_block128": ("e4m3", "block", 128, "f32", False, "fp8_group"),
    "mxfp4_bf16": ("e2m1", "group", 32, "e8m0", False, "bf16"),
    "nvfp4_bf16": ("e2m1", "group", 16, "e4m3", False, "bf16"),
    "mxint4_bf16": ("int4", "group", 32, "e8m0", False, "bf16"),
    "mxfp4_mxfp8": ("e2m1", "group", 32, "e8m0", False, "mxfp8"),
    "mxfp4_mxfp4": ("e2m1", "group", 32, "e8m0", False, "mxfp4"),
}

_QUANT = {
    "fp8_token": (oracle.quant.quant_fp8_per_token, oracle.quant.dequant_fp8_per_token),
    "mxfp8": (oracle.quant.quant_mxfp8, oracle.quant.dequant_mxfp8),
    "mxfp4": (oracle.quant.quant_mxfp4, oracle.quant.dequant_mxfp4),
    "fp8_group": (oracle.quant.quant_fp8_group, oracle.quant.dequant_fp8_group),
}


def _oracle_acts(act, xb):
    x = oracle.formats.decode_bf16(xb)
    if act == "bf16":
        return x
    q, deq = _QUANT[act]
    codes, scales = q(x.astype(np.float32))
    return deq(codes, scales)


@pytest.mark.parametrize("name", list(FORMATS))
def test_dense_rows_independent_of_m(name):
    wd, gran, gs, sd, zero, act = FORMATS[name]
    n, k, m_full = 304, 1024, 300     # N not a multiple of any tile width
    seed = synth.seed_for(11, list(FORMATS).index(name))
    w = synth.quant_weights(seed, wd, gran, gs, sd, 1, n, k, zero=zero)
    hd, od = descs(wd, gran, gs, sd, 1, n, k, zero=zero, act=act)
    packed = prepare(hd, w, sd)
    xb = synth.bf16_normal(synth.rng(seed + 1), (m_full, k))
    xd = dev(xb)
    print(f"case invariance {name}", flush=True)
    c = hum.select_config(hd, m_full, batch_invariant=True)
    assert c.kind == hum.KERNEL_TILE and c.split_k == 1
    full = hum.linear(hd, packed, xd, batch_invariant=True)
    torch.cuda.synchronize()
    ref = oracle.gemm.linear(od, _oracle_acts(act, xb), w["codes"], w["scales"], w.get("zeros"))
    assert_tol(full, ref, name)
    full_bits = full.view(torch.int16).cpu().numpy()
    for r0, m in ((0, 1), (0, 7), (0, 16), (0, 17), (3, 64), (100, 129), (0, 257), (299, 1)):
        c = hum.select_config(hd, m, batch_invariant=True)
        assert c.kind == hum.KERNEL_TILE and c.split_k == 1, (m, c)
        part = hum.linear(hd, packed, xd[r0:r0 + m], batch_invariant=True)
        torch.cuda.synchronize()
        got = part.view(torch.int16).cpu().numpy()
        assert np.array_equal(got, full_bits[r0:r0 + m]), f"{name}: rows {r0}..{r0 + m} differ from the m = {m_full} run"


@pytest.mark.parametrize("act", ["bf16", "mxfp8", "mxfp4"])
def test_moe_tokens_independent_of_batch(act):
    e, h, inter, topk, t_full = 8, 256, 128, 2, 70
    seed = synth.seed_for(12, ["bf16", "mxfp8", "mxfp4"].index(act))
    w13 = synth.moe_weights_mxfp4(seed, e, 2 * inter, h)
    w2 = synth.moe_weights_mxfp4(seed + 1, e, h, inter)
    d13, o13 = descs("e2m1", "group", 32, "e8m0", e, 2 * inter, h, act=act)
    d2, o2 = descs("e2m1", "group", 32, "e8m0", e, h, inter, act=act)
    p13, p2 = prepare(d13, w13, "e8m0"), prepare(d2, w2, "e8m0")
    ids, wts = synth.routing(seed + 2, t_full, e, topk)
    xb = synth.bf16_normal(synth.rng(seed + 3), (t_full, h))
    print(f"case moe invariance act={act}", flush=True)
    for t in (1, 9, 70):
        assert hum.moe_select_config(d13, d2, t, topk, batch_invariant=True).kind == hum.KERNEL_TILE
    full = hum.moe_gemm(d13, p13, d2, p2, dev(xb), dev(ids), dev(wts), batch_invariant=True)
    torch.cuda.synchronize()
    assert_tol(full, oracle.moe.moe_forward(o13, w13, o2, w2, xb, ids, wts, act), f"moe act={act}")
    full_bits = full.view(torch.int16).cpu().numpy()
    for t0, t1 in ((0, 1), (5, 6), (0, 9), (30, 70), (69, 70)):
        part = hum.moe_gemm(d13, p13, d2, p2, dev(xb[t0:t1]), dev(ids[t0:t1]), dev(wts[t0:t1]),
                            batch_invariant=True)
        torch.cuda.synchronize()
        got = part.view(torch.int16).cpu().numpy()
        assert np.array_equal(got, full_bits[t0:t1]), f"act={act}: tokens {t0}..{t1} differ from the T = {t_full} run"


def test_default_selection_is_not_invariant():
    """Control: the default selection's decode kernel (M <= 16) splits K over
    waves, so its sums round differently from the tile kernel's; without the
    flag, row 0 of an M = 1 call differs from row 0 of an M = 300 call."""
    wd, gran, gs, sd, zero, act = FORMATS["uint4_zp_g128"]
    n, k = 304, 1024
    seed = synth.seed_for(11, 0)
    w = synth.quant_weights(seed, wd, gran, gs, sd, 1, n, k, zero=zero)
    hd, _ = descs(wd, gran, gs, sd, 1, n, k, zero=zero, act=act)
    packed = prepare(hd, w, sd)
    xd = dev(synth.bf16_normal(synth.rng(seed + 1), (300, k)))
    assert hum.select_config(hd, 1).kind == hum.KERNEL_STREAM
    one = hum.linear(hd, packed, xd[:1])
    full = hum.linear(hd, packed, xd)
    torch.cuda.synchronize()
    assert not torch.equal(one.view(torch.int16), full[:1].view(torch.int16))
