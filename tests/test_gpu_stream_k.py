"""GPU: Stream-K dense GEMM (hum_tile_config.stream_k > 0).

Workgroups take equal shares of the tiles' K-blocks laid end to end; a tile
shared by several is summed by the last of them to finish, in segment order.
Checked here:
* exact-integer cases bit for bit against the oracle on every Stream-K
  instance, for workgroup counts that give one segment per tile, shares
  spanning several tiles, and one K-block per workgroup (the most segments);
* random cases against the oracle at the bf16-output bound, ragged M and N;
* run-to-run bitwise determinism (the sum order does not depend on which
  workgroup finishes last);
* the per-tile counters are left at zero: calls of different shapes on one
  workspace, with a MoE layer's use of the same workspace in between."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_packed_amd as hum
import synth
from gpu_util import assert_bf16_exact, assert_tol, descs, dev, prepare

pytestmark = pytest.mark.gpu

# (format, kind, wave_m, wave_n, stages): every compiled Stream-K instance
SK_TILES = [
    ("uint4", 0, 2, 2, 3), ("uint4", 0, 2, 4, 3), ("uint4", 2, 4, 2, 3), ("uint4", 2, 4, 4, 3), ("uint4", 2, 4, 4, 2),
    ("e4m3", 0, 2, 2, 3), ("e4m3", 0, 4, 4, 2), ("e4m3", 0, 8, 2, 2),
    ("e2m1", 0, 2, 2, 3), ("e2m1", 2, 4, 4, 3),
    ("e2m1_mxfp8", 0, 2, 2, 3), ("e2m1_mxfp8", 0, 8, 2, 2),
    ("e2m1_mxfp4", 0, 2, 2, 3), ("e2m1_mxfp4", 0, 4, 4, 3),
    ("e4m3_block", 0, 2, 2, 3), ("e4m3_block", 0, 8, 2, 2),
    ("e4m3_bf16", 0, 2, 2, 3), ("int8", 0, 2, 2, 3), ("nvfp4", 0, 2, 2, 3), ("mxint4", 0, 2, 2, 3),
    ("int3", 0, 2, 2, 3), ("uint2", 0, 2, 2, 3), ("int1", 0, 2, 2, 3), ("e2m3", 0, 2, 2, 3), ("e3m2", 0, 2, 2, 3),
    ("e2m1", 0, 1, 2, 3),
]


def sk_cfg(kind, wm, wn, stages, groups):
    c = hum.TileConfig()
    c.kind, c.wave_m, c.wave_n, c.waves_n, c.waves_k = kind, wm, wn, 4, 1
    c.stages, c.split_k, c.block_m, c.stream_k = stages, 1, 16 * wm, groups
    return c


def _case(fmt, m, n, k, exact, seed):
    """(hum desc, oracle desc, packed, activations, oracle reference)."""
    g = synth.rng(seed)
    if exact:
        xb = synth.bf16_bits(g.integers(-8, 9, size=(m, k)).astype(np.float32))
    else:
        xb = synth.bf16_normal(g, (m, k))
    a = oracle.formats.decode_bf16(xb)
    if fmt == "uint4":
        w = synth.quant_weights(seed, "uint4", "group", 128, "bf16", 1, n, k, zero=True)
        if exact:
            w["scales"] = synth.bf16_bits(np.ldexp(1.0, g.integers(-5, -2, size=(1, n, k // 128))).astype(np.float32))
        hd, od = descs("uint4", "group", 128, "bf16", 1, n, k, zero=True)
        packed = prepare(hd, w, "bf16")
        ref = oracle.gemm.linear(od, a, w["codes"], w["scales"], w["zeros"])
        return hd, packed, xb, ref
    if fmt in ("e2m1", "e2m1_mxfp8", "e2m1_mxfp4"):
        act = {"e2m1": "bf16", "e2m1_mxfp8": "mxfp8", "e2m1_mxfp4": "mxfp4"}[fmt]
        lo, hi = (126, 127) if exact else (119, 123)
        w = synth.quant_weights(seed, "e2m1", "group", 32, "e8m0", 1, n, k, e8m0_lo=lo, e8m0_hi=hi)
        hd, od = descs("e2m1", "group", 32, "e8m0", 1, n, k, act=act)
        packed = prepare(hd, w, "e8m0")
        if act == "mxfp8":
            q, s = oracle.quant.quant_mxfp8(a.astype(np.float32))
            a = oracle.quant.dequant_mxfp8(q, s)
        elif act == "mxfp4":
            q, s = oracle.quant.quant_mxfp4(a.astype(np.float32))
            a = oracle.quant.dequant_mxfp4(q, s)
        return hd, packed, xb, oracle.gemm.linear(od, a, w["codes"], w["scales"])
    if fmt in ("e4m3", "e4m3_bf16"):
        act = "fp8_token" if fmt == "e4m3" else "bf16"
        w = synth.quant_weights(seed, "e4m3", "channel", 0, "f32", 1, n, k)
        if exact:
            w["scales"] = np.ldexp(1.0, g.integers(-8, -5, size=(1, n, 1))).astype(np.float32)
        hd, od = descs("e4m3", "channel", 0, "f32", 1, n, k, act=act)
        packed = prepare(hd, w, "f32")
        if act == "fp8_token":
            q, s = oracle.quant.quant_fp8_per_token(a.astype(np.float32))
            a = oracle.quant.dequant_fp8_per_token(q, s)
        return hd, packed, xb, oracle.gemm.linear(od, a, w["codes"], w["scales"])
    if fmt == "e4m3_block":
        w = synth.quant_weights(seed, "e4m3", "block", 128, "f32", 1, n, k)
        if exact:
            w["scales"] = np.ldexp(1.0, g.integers(-8, -5, size=w["scales"].shape)).astype(np.float32)
        hd, od = descs("e4m3", "block", 128, "f32", 1, n, k, act="fp8_group")
        packed = prepare(hd, w, "f32")
        q, s = oracle.quant.quant_fp8_group(a.astype(np.float32))
        a = oracle.quant.dequant_fp8_group(q, s)
        return hd, packed, xb, oracle.gemm.linear(od, a, w["codes"], w["scales"])
    if fmt in ("int3", "uint2", "int1"):
        zero = fmt.startswith("u")
        w = synth.quant_weights(seed, fmt, "group", 128, "bf16", 1, n, k, zero=zero)
        if exact:
            w["scales"] = synth.bf16_bits(np.ldexp(1.0, g.integers(-5, -2, size=(1, n, k // 128))).astype(np.float32))
        hd, od = descs(fmt, "group", 128, "bf16", 1, n, k, zero=zero)
        packed = prepare(hd, w, "bf16")
        return hd, packed, xb, oracle.gemm.linear(od, a, w["codes"], w["scales"], w.get("zeros"))
    if fmt in ("e2m3", "e3m2"):
        lo, hi = (126, 127) if exact else (119, 123)
        w = synth.quant_weights(seed, fmt, "group", 32, "e8m0", 1, n, k, e8m0_lo=lo, e8m0_hi=hi)
        hd, od = descs(fmt, "group", 32, "e8m0", 1, n, k)
        packed = prepare(hd, w, "e8m0")
        return hd, packed, xb, oracle.gemm.linear(od, a, w["codes"], w["scales"])
    if fmt == "nvfp4":
        lo, hi = (0x30, 0x38) if exact else (0x18, 0x38)
        w = synth.quant_weights(seed, "e2m1", "group", 16, "e4m3", 1, n, k, global_scale=not exact,
                                e4m3_lo=lo, e4m3_hi=hi)
        hd, od = descs("e2m1", "group", 16, "e4m3", 1, n, k, glob=not exact)
        packed = prepare(hd, w, "e4m3")
        return hd, packed, xb, oracle.gemm.linear(od, a, w["codes"], w["scales"], None, w.get("global_scale"))
    if fmt == "mxint4":
        lo, hi = (125, 127) if exact else (119, 123)
        w = synth.quant_weights(seed, "int4", "group", 32, "e8m0", 1, n, k, e8m0_lo=lo, e8m0_hi=hi)
        hd, od = descs("int4", "group", 32, "e8m0", 1, n, k)
        packed = prepare(hd, w, "e8m0")
        return hd, packed, xb, oracle.gemm.linear(od, a, w["codes"], w["scales"])
    assert fmt == "int8"
    w = synth.quant_weights(seed, "int8", "channel", 0, "f32", 1, n, k)
    w["scales"] = np.ldexp(1.0, g.integers(-12, -9, size=(1, n, 1))).astype(np.float32)
    hd, od = descs("int8", "channel", 0, "f32", 1, n, k)
    packed = prepare(hd, w, "f32")
    return hd, packed, xb, oracle.gemm.linear(od, a, w["codes"], w["scales"])


def _tiles(m, n, wm, wn):
    return -(-m // (16 * wm)) * -(-n // (64 * wn))


@pytest.mark.parametrize("tile", SK_TILES, ids=lambda t: "-".join(map(str, t)))
def test_stream_k_exact_every_instance(tile):
    """Exact-integer operands: every Stream-K instance bit for bit against the
    oracle, at workgroup counts from a few (shares span tiles) to one
    K-block each."""
    fmt, kind, wm, wn, st = tile
    m, n, k = 45, 448, 1024
    exact_act = fmt not in ("e4m3", "e2m1_mxfp8", "e2m1_mxfp4", "e4m3_block")
    hd, packed, xb, ref = _case(fmt, m, n, k, exact=True, seed=synth.seed_of("sk", tile))
    iters = _tiles(m, n, wm, wn) * (k // 128)
    for groups in sorted({3, 7, max(1, iters // 3), iters}):
        print(f"case stream-k exact {tile} groups={groups}", flush=True)
        out = hum.linear(hd, packed, dev(xb), cfg=sk_cfg(kind, wm, wn, st, groups))
        torch.cuda.synchronize()
        if exact_act:
            assert_bf16_exact(out, ref, f"{tile} groups={groups}")
        else:
            # quantized activations: the oracle's quantizer sets the values;
            # integer codes and power-of-two scales keep the sums exact only
            # up to the activation scales, so the bf16-output bound applies
            assert_tol(out, ref, f"{tile} groups={groups}")


@pytest.mark.parametrize("tile", [SK_TILES[0], SK_TILES[3], SK_TILES[7], SK_TILES[9], SK_TILES[11], SK_TILES[13]],
                         ids=lambda t: "-".join(map(str, t)))
@pytest.mark.parametrize("m", [17, 300])
def test_stream_k_random_vs_oracle_and_deterministic(tile, m):
    fmt, kind, wm, wn, st = tile
    n, k = 600, 2048
    hd, packed, xb, ref = _case(fmt, m, n, k, exact=False, seed=synth.seed_of("skr", tile, m))
    iters = _tiles(m, n, wm, wn) * (k // 128)
    for groups in (5, max(1, iters // 2 + 1), 512):
        c = sk_cfg(kind, wm, wn, st, groups)
        print(f"case stream-k random {tile} m={m} groups={groups}", flush=True)
        out1 = hum.linear(hd, packed, dev(xb), cfg=c)
        out2 = hum.linear(hd, packed, dev(xb), cfg=c)
        torch.cuda.synchronize()
        assert torch.equal(out1, out2), f"{tile} m={m} groups={groups}: not bitwise repeatable"
        assert_tol(out1, ref, f"{tile} m={m} groups={groups}")


def test_stream_k_counters_survive_workspace_reuse():
    """Stream-K calls of different shapes on one explicit workspace, with a
    MoE layer writing its own scratch into the same buffer in between: the
    tile counters stay valid (left at zero by every call)."""
    ws = hum.Workspace("cuda")
    results = []
    for m, groups in ((33, 11), (300, 64), (33, 11)):
        hd, packed, xb, ref = _case("uint4", m, 512, 1024, exact=True, seed=71 + m)
        c = sk_cfg(2, 4, 4, 3, groups)
        buf = ws.get(hum.linear_workspace_bytes(hd, m, cfg=c))
        out = hum.linear(hd, packed, dev(xb), cfg=c, workspace=buf)
        torch.cuda.synchronize()
        assert_bf16_exact(out, ref, f"m={m} groups={groups}")
        results.append(out)
        # a MoE layer on the same workspace
        e, h, inter = 8, 256, 128
        w13 = synth.moe_weights_mxfp4(5, e, 2 * inter, h)
        w2 = synth.moe_weights_mxfp4(6, e, h, inter)
        d13, _ = descs("e2m1", "group", 32, "e8m0", e, 2 * inter, h)
        d2, _ = descs("e2m1", "group", 32, "e8m0", e, h, inter)
        ids, wts = synth.routing(7, 64, e, 2)
        x = synth.bf16_normal(synth.rng(8), (64, h))
        mbuf = ws.get(hum.moe_workspace_bytes(d13, d2, 64, 2))
        hum.moe_gemm(d13, prepare(d13, w13, "e8m0"), d2, prepare(d2, w2, "e8m0"), dev(x), dev(ids), dev(wts),
                     workspace=mbuf)
        torch.cuda.synchronize()
    assert torch.equal(results[0], results[2])
