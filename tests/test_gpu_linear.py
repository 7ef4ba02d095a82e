"""GPU: dense quantized GEMM (hum_linear) against the oracle.

* exact-integer cases (integer activations, power-of-two scales, integer
  zero points) must match bf16(oracle) bit for bit for every compiled tile
  configuration and split-K factor;
* random cases must meet the bf16-output tolerance;
* edge cases: M = 1, ragged N (not a multiple of any tile), bias, global
  scale, G = K, repeat-run determinism."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_packed_amd as hum
import synth
from gpu_util import assert_bf16_exact, assert_tol, descs, dev, prepare

pytestmark = pytest.mark.gpu

# (kind, wave_m, wave_n, waves_n, waves_k[, stages]): every compiled dense instance
STREAM_TILES = [(1, 1, 1, 1, 8), (1, 1, 2, 1, 8), (1, 1, 4, 1, 8), (1, 1, 1, 1, 4), (1, 1, 1, 1, 15), (1, 1, 2, 1, 15),
                (1, 1, 4, 1, 15)]
TILE_TILES = [(0, 1, 4, 4, 1), (0, 2, 2, 4, 1), (0, 2, 4, 4, 1), (0, 4, 2, 4, 1), (0, 4, 4, 4, 1),
              (0, 8, 2, 4, 1), (0, 8, 4, 4, 1),
              (0, 2, 2, 4, 1, 3), (0, 2, 4, 4, 1, 3), (0, 4, 2, 4, 1, 3), (0, 4, 4, 4, 1, 3), (0, 8, 2, 4, 1, 3)]
DENSE_TILES = STREAM_TILES + TILE_TILES
# 32x32-block tiles (INT and MXFP4 weights with bf16 activations)
TILE32_TILES = [(2, 2, 2, 4, 1), (2, 2, 4, 4, 1), (2, 4, 2, 4, 1), (2, 4, 4, 4, 1), (2, 8, 2, 4, 1),
                (2, 2, 2, 4, 1, 3), (2, 2, 4, 4, 1, 3), (2, 4, 2, 4, 1, 3), (2, 4, 4, 4, 1, 3)]


def cfg(t, split):
    c = hum.TileConfig()
    c.kind, c.wave_m, c.wave_n, c.waves_n, c.waves_k = t[:5]
    c.stages = t[5] if len(t) > 5 else 0
    c.split_k = split
    c.block_m = 16 * t[1]
    return c


def rows_for(tile, m):
    """The stream kernel takes at most 16 rows."""
    return min(m, 13) if tile[0] == 1 else m


def stream_fits(tile, m, k, split, chunk_per_row_kb=16):
    """A dense stream launch gives each of its waves_k waves a contiguous
    K range whose activation rows it copies in at most 8 16-byte chunks per
    lane; longer ranges are rejected (a larger split_k fits)."""
    if tile[0] != 1:
        return True
    kb, kw = k // 128, tile[4]
    kbps = -(-(-(-kb // split)) // kw) * kw
    return m * (-(-kbps // kw)) * chunk_per_row_kb <= 512


def _int_exact_case(seed, wd, m, n, k, gs, zero):
    g = synth.rng(seed)
    w = synth.quant_weights(seed, wd, "group", gs, "bf16", 1, n, k, zero=zero)
    ng = k // gs
    w["scales"] = synth.bf16_bits(np.ldexp(1.0, g.integers(-5, -2, size=(1, n, ng))).astype(np.float32))
    xb = synth.bf16_bits(g.integers(-8, 9, size=(m, k)).astype(np.float32))
    return w, xb


@pytest.mark.parametrize("tile", DENSE_TILES + TILE32_TILES, ids=lambda t: "t" + "".join(map(str, t)))
@pytest.mark.parametrize("split", [1, 2, 4])
def test_int_exact_every_tile(tile, split):
    m, n, k, gs = rows_for(tile, 37), 640, 2048, 128
    w, xb = _int_exact_case(31, "uint4", m, n, k, gs, True)
    hd, od = descs("uint4", "group", gs, "bf16", 1, n, k, zero=True)
    print(f"case uint4 exact tile={tile} split={split}", flush=True)
    packed = prepare(hd, w, "bf16")
    if not stream_fits(tile, m, k, split):
        with pytest.raises(hum.HumError, match="raise split_k"):
            hum.linear(hd, packed, dev(xb), cfg=cfg(tile, split))
        return
    out = hum.linear(hd, packed, dev(xb), cfg=cfg(tile, split))
    torch.cuda.synchronize()
    ref = oracle.gemm.linear(od, oracle.formats.decode_bf16(xb), w["codes"], w["scales"], w["zeros"])
    assert_bf16_exact(out, ref, f"tile={tile} split={split}")


@pytest.mark.parametrize("tile", DENSE_TILES + TILE32_TILES, ids=lambda t: "t" + "".join(map(str, t)))
def test_int4_sym_exact_every_tile(tile):
    m, n, k, gs = 5, 200, 1024, 256
    w, xb = _int_exact_case(32, "int4", m, n, k, gs, False)
    hd, od = descs("int4", "group", gs, "bf16", 1, n, k)
    packed = prepare(hd, w, "bf16")
    out = hum.linear(hd, packed, dev(xb), cfg=cfg(tile, 2))
    torch.cuda.synchronize()
    ref = oracle.gemm.linear(od, oracle.formats.decode_bf16(xb), w["codes"], w["scales"])
    assert_bf16_exact(out, ref, f"tile={tile}")


LOWBIT = [("int3", False), ("uint3", True), ("int2", False), ("uint2", True), ("int1", False), ("uint1", True)]


@pytest.mark.parametrize("wd,zero", LOWBIT, ids=lambda v: str(v))
@pytest.mark.parametrize("tile", DENSE_TILES + TILE32_TILES, ids=lambda t: "t" + "".join(map(str, t)))
def test_lowbit_int_exact_every_tile(wd, zero, tile):
    """INT3 / INT2 / INT1 (signed and unsigned with zero points): exact-integer
    cases bit for bit on every compiled tile, split 1 for the 3- and 2-bit
    codes and 2 for all (the split-K partial path)."""
    m, n, k, gs = rows_for(tile, 21), 336, 1024, 128
    w, xb = _int_exact_case(synth.seed_of(wd, tile), wd, m, n, k, gs, zero)
    hd, od = descs(wd, "group", gs, "bf16", 1, n, k, zero=zero)
    packed = prepare(hd, w, "bf16")
    ref = oracle.gemm.linear(od, oracle.formats.decode_bf16(xb), w["codes"], w["scales"], w.get("zeros"))
    for split in ((1, 2) if wd[-1] in "32" else (2,)):
        print(f"case {wd} exact tile={tile} split={split}", flush=True)
        out = hum.linear(hd, packed, dev(xb), cfg=cfg(tile, split))
        torch.cuda.synchronize()
        assert_bf16_exact(out, ref, f"{wd} tile={tile} split={split}")


@pytest.mark.parametrize("wd,gran,gs,sd,zero", [("int3", "group", 128, "bf16", False),
                                                ("uint3", "group", 256, "bf16", True),
                                                ("int2", "channel", 0, "f32", False),
                                                ("uint2", "group", 128, "bf16", True),
                                                ("int1", "group", 128, "f32", False),
                                                ("uint1", "tensor", 0, "bf16", True)])
@pytest.mark.parametrize("m", [1, 7, 16, 64, 300])
def test_lowbit_random_vs_oracle(wd, gran, gs, sd, zero, m):
    """Low-bit integer weights on random data with the selector's
    configuration, ragged N, a bias and a global scale."""
    n, k = 600, 2048
    w = synth.quant_weights(synth.seed_of(wd, gran, m), wd, gran, gs, sd, 1, n, k, zero=zero, global_scale=True)
    hd, od = descs(wd, gran, gs, sd, 1, n, k, zero=zero, glob=True)
    xb = synth.bf16_normal(synth.rng(synth.seed_of("x", wd, m)), (m, k))
    bias = synth.bf16_normal(synth.rng(synth.seed_of("b", wd)), (n,))
    packed = prepare(hd, w, sd)
    print(f"case {wd} random m={m}", flush=True)
    out = hum.linear(hd, packed, dev(xb), bias=dev(bias))
    torch.cuda.synchronize()
    ref = oracle.gemm.linear(od, oracle.formats.decode_bf16(xb), w["codes"], w["scales"], w.get("zeros"),
                             w.get("global_scale"), bias_bits=bias)
    assert_tol(out, ref, f"{wd} {gran} m={m}")


@pytest.mark.parametrize("wd", ["e2m3", "e3m2"])
@pytest.mark.parametrize("tile", DENSE_TILES, ids=lambda t: "t" + "".join(map(str, t)))
def test_mxfp6_exact_every_tile(wd, tile):
    """MXFP6 (E2M3 / E3M2 with E8M0 per 32) x integer activations: every FP6
    code, scales 2^-1 .. 2^0, all sums exact in fp32 -- bit for bit on every
    compiled tile, split 1 and 2."""
    m, n, k = rows_for(tile, 19), 208, 1024
    g = synth.rng(synth.seed_of("fp6x", wd))
    xb = synth.bf16_bits(g.integers(-8, 9, size=(m, k)).astype(np.float32))
    w = synth.quant_weights(synth.seed_of("fp6w", wd), wd, "group", 32, "e8m0", 1, n, k, e8m0_lo=126, e8m0_hi=127)
    hd, od = descs(wd, "group", 32, "e8m0", 1, n, k)
    packed = prepare(hd, w, "e8m0")
    ref = oracle.gemm.linear(od, oracle.formats.decode_bf16(xb), w["codes"], w["scales"])
    for split in (1, 2):
        print(f"case {wd} exact tile={tile} split={split}", flush=True)
        if not stream_fits(tile, m, k, split):
            continue
        out = hum.linear(hd, packed, dev(xb), cfg=cfg(tile, split))
        torch.cuda.synchronize()
        assert_bf16_exact(out, ref, f"{wd} tile={tile} split={split}")


@pytest.mark.parametrize("wd", ["e2m3", "e3m2"])
@pytest.mark.parametrize("m", [1, 9, 64, 300])
def test_mxfp6_random_vs_oracle(wd, m):
    """MXFP6 weights on random data at the selector's configuration, ragged N,
    a bias and a global scale."""
    n, k = 600, 2048
    w = synth.quant_weights(synth.seed_of("fp6r", wd, m), wd, "group", 32, "e8m0", 1, n, k, global_scale=True)
    hd, od = descs(wd, "group", 32, "e8m0", 1, n, k, glob=True)
    xb = synth.bf16_normal(synth.rng(synth.seed_of("fp6rx", wd, m)), (m, k))
    bias = synth.bf16_normal(synth.rng(synth.seed_of("fp6rb", wd)), (n,))
    packed = prepare(hd, w, "e8m0")
    print(f"case {wd} random m={m}", flush=True)
    out = hum.linear(hd, packed, dev(xb), bias=dev(bias))
    torch.cuda.synchronize()
    ref = oracle.gemm.linear(od, oracle.formats.decode_bf16(xb), w["codes"], w["scales"], None, w["global_scale"],
                             bias_bits=bias)
    assert_tol(out, ref, f"{wd} m={m}")


@pytest.mark.parametrize("tile", DENSE_TILES + TILE32_TILES, ids=lambda t: "t" + "".join(map(str, t)))
def test_mxfp4_bf16_exact_every_tile(tile):
    m, n, k = 9, 96, 1024
    g = synth.rng(33)
    w = synth.quant_weights(33, "e2m1", "group", 32, "e8m0", 1, n, k, e8m0_lo=126, e8m0_hi=127)
    xb = synth.bf16_bits(g.integers(-8, 9, size=(m, k)).astype(np.float32))
    hd, od = descs("e2m1", "group", 32, "e8m0", 1, n, k)
    packed = prepare(hd, w, "e8m0")
    out = hum.linear(hd, packed, dev(xb), cfg=cfg(tile, 1))
    torch.cuda.synchronize()
    ref = oracle.gemm.linear(od, oracle.formats.decode_bf16(xb), w["codes"], w["scales"])
    assert_bf16_exact(out, ref, f"tile={tile}")


@pytest.mark.parametrize("tile", DENSE_TILES, ids=lambda t: "t" + "".join(map(str, t)))
def test_mxfp4_mxfp8_exact_every_tile(tile):
    """Dense W4A8: integer activations in [-8, 8] quantize to MXFP8 exactly
    (shared exponent 2^-5, codes 32 x), E2M1 x E8M0 weights are exact, and
    every partial sum is exact in fp32: bitwise equal to the oracle."""
    m, n, k = rows_for(tile, 19), 96, 1024
    g = synth.rng(34)
    w = synth.quant_weights(34, "e2m1", "group", 32, "e8m0", 1, n, k, e8m0_lo=126, e8m0_hi=127)
    xb = synth.bf16_bits(g.integers(-8, 9, size=(m, k)).astype(np.float32))
    hd, od = descs("e2m1", "group", 32, "e8m0", 1, n, k, act="mxfp8")
    packed = prepare(hd, w, "e8m0")
    print(f"case w4a8 exact tile={tile}", flush=True)
    out = hum.linear(hd, packed, dev(xb), cfg=cfg(tile, 2))
    torch.cuda.synchronize()
    q, e = oracle.quant.quant_mxfp8(oracle.formats.decode_bf16(xb).astype(np.float32))
    a = oracle.quant.dequant_mxfp8(q, e)
    ref = oracle.gemm.linear(od, a, w["codes"], w["scales"])
    assert_bf16_exact(out, ref, f"tile={tile}")


@pytest.mark.parametrize("split", [1, 2])
@pytest.mark.parametrize("tile", TILE_TILES, ids=lambda t: "t" + "".join(map(str, t)))
def test_mxfp4_mxfp4_exact_every_tile(tile, split):
    """Dense W4A4: activations drawn from the E2M1 grid with one +-4 or +-6
    per 32-block quantize to MXFP4 exactly (block scale 2^0), E2M1 x E8M0
    weights are exact, and every partial sum is exact in fp32: bitwise equal
    to the oracle."""
    m, n, k = 19, 96, 1024
    g = synth.rng(36)
    w = synth.quant_weights(36, "e2m1", "group", 32, "e8m0", 1, n, k, e8m0_lo=126, e8m0_hi=127)
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    x = grid[g.integers(0, 8, size=(m, k))] * np.where(g.integers(0, 2, size=(m, k)) == 1, -1.0, 1.0)
    x[:, ::32] = np.where(g.integers(0, 2, size=(m, k // 32)) == 1, 4.0, -6.0)
    xb = oracle.formats.encode_bf16(x)
    hd, od = descs("e2m1", "group", 32, "e8m0", 1, n, k, act="mxfp4")
    packed = prepare(hd, w, "e8m0")
    print(f"case w4a4 exact tile={tile} split={split}", flush=True)
    out = hum.linear(hd, packed, dev(xb), cfg=cfg(tile, split))
    torch.cuda.synchronize()
    q, e = oracle.quant.quant_mxfp4(oracle.formats.decode_bf16(xb))
    a = oracle.quant.dequant_mxfp4(q, e)
    assert np.array_equal(a, oracle.formats.decode_bf16(xb))
    ref = oracle.gemm.linear(od, a, w["codes"], w["scales"])
    assert_bf16_exact(out, ref, f"tile={tile}")


@pytest.mark.parametrize("split", [1, 2])
@pytest.mark.parametrize("tile", STREAM_TILES, ids=lambda t: "t" + "".join(map(str, t)))
def test_w4a4_decode_kernel_exact(tile, split):
    """Dense W4A4 on the decode kernel (E4M3 x E2M1: the MXFP4 activations
    handed over as the E4M3 bytes of the same values): the exact case of
    the tile test above, bitwise equal to the oracle, on every decode
    configuration."""
    m, n, k = 13, 96, 1024
    g = synth.rng(37)
    w = synth.quant_weights(37, "e2m1", "group", 32, "e8m0", 1, n, k, e8m0_lo=126, e8m0_hi=127)
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    x = grid[g.integers(0, 8, size=(m, k))] * np.where(g.integers(0, 2, size=(m, k)) == 1, -1.0, 1.0)
    x[:, ::32] = np.where(g.integers(0, 2, size=(m, k // 32)) == 1, 4.0, -6.0)
    xb = oracle.formats.encode_bf16(x)
    hd, od = descs("e2m1", "group", 32, "e8m0", 1, n, k, act="mxfp4")
    packed = prepare(hd, w, "e8m0")
    print(f"case w4a4 decode exact tile={tile} split={split}", flush=True)
    out = hum.linear(hd, packed, dev(xb), cfg=cfg(tile, split))
    torch.cuda.synchronize()
    ref = oracle.gemm.linear(od, oracle.formats.decode_bf16(xb), w["codes"], w["scales"])
    assert_bf16_exact(out, ref, f"tile={tile} split={split}")
    # pre-quantized W4A4 activations (E2M1 codes) are refused on the decode kernel
    q, s = hum.quant_act("mxfp4", dev(xb))
    with pytest.raises(hum.HumError, match="quantizes its activations itself"):
        hum.linear(hd, packed, q, a_scales=s, cfg=cfg(tile, split))


@pytest.mark.parametrize("m", [1, 7, 16, 100, 300])
def test_w4a4_dense_random_vs_oracle(m):
    """Dense W4A4 (MXFP4 weights x MXFP4 activations) at the selector's config."""
    n, k = 640, 2048
    w = synth.moe_weights_mxfp4(synth.seed_for(6, m), 1, n, k)
    xb = synth.bf16_normal(synth.rng(synth.seed_for(6, 100 + m)), (m, k))
    hd, od = descs("e2m1", "group", 32, "e8m0", 1, n, k, act="mxfp4")
    packed = prepare(hd, w, "e8m0")
    out = hum.linear(hd, packed, dev(xb))
    torch.cuda.synchronize()
    q, e = oracle.quant.quant_mxfp4(oracle.formats.decode_bf16(xb))
    ref = oracle.gemm.linear(od, oracle.quant.dequant_mxfp4(q, e), w["codes"], w["scales"])
    assert_tol(out, ref, f"w4a4 m={m}")


@pytest.mark.parametrize("split", [1, 2])
@pytest.mark.parametrize("tile", TILE_TILES, ids=lambda t: "t" + "".join(map(str, t)))
def test_fp8_block_exact_every_tile(tile, split):
    """Block-scaled FP8: every 128-group of a row holds small integers times a
    power of two with one +-448 * 2^e, so its scale is 2^e and the codes are
    exact; weights are E4M3 codes of small integers with power-of-two block
    scales; every K-block's MFMA sum, scale product and accumulation is then
    exact in fp32: bitwise equal to the oracle."""
    m, n, k = 37, 272, 1024
    g = synth.rng(38)
    ints = g.integers(-8, 9, size=(m, k)).astype(np.float64)
    ints[:, ::128] = np.where(g.integers(0, 2, size=(m, k // 128)) == 1, 448.0, -448.0)
    # (exponent ranges kept narrow: the fp32 sums of a row then span < 2^24)
    x = ints * np.ldexp(1.0, g.integers(-6, -3, size=(m, k // 128))).repeat(128, axis=1)
    xb = oracle.formats.encode_bf16(x)
    wv = g.integers(-8, 9, size=(1, n, k)).astype(np.float64)
    codes = oracle.formats.encode_e4m3(wv)
    scales = np.ldexp(1.0, g.integers(-9, -7, size=(1, -(-n // 128), k // 128))).astype(np.float32)
    w = {"codes": codes, "scales": scales}
    hd, od = descs("e4m3", "block", 128, "f32", 1, n, k, act="fp8_group")
    packed = prepare(hd, w, "f32")
    print(f"case fp8 block exact tile={tile} split={split}", flush=True)
    out = hum.linear(hd, packed, dev(xb), cfg=cfg(tile, split))
    torch.cuda.synchronize()
    q, s = oracle.quant.quant_fp8_group(oracle.formats.decode_bf16(xb).astype(np.float32))
    a = oracle.quant.dequant_fp8_group(q, s)
    assert np.array_equal(a, oracle.formats.decode_bf16(xb))
    ref = oracle.gemm.linear(od, a, w["codes"], w["scales"])
    assert_bf16_exact(out, ref, f"tile={tile}")


@pytest.mark.parametrize("split", [1, 2])
@pytest.mark.parametrize("tile", STREAM_TILES, ids=lambda t: "t" + "".join(map(str, t)))
def test_fp8_block_decode_kernel_exact(tile, split):
    """Block-scaled FP8 on the decode kernel, which quantizes each row's
    K-blocks itself (the group rule: s = amax / 448 per row and 128 along K):
    the exact case of the tile test above, bitwise equal to the oracle, on
    every decode configuration; pre-quantized activations are refused
    there."""
    m, n, k = 13, 272, 1024
    g = synth.rng(40)
    ints = g.integers(-8, 9, size=(m, k)).astype(np.float64)
    ints[:, ::128] = np.where(g.integers(0, 2, size=(m, k // 128)) == 1, 448.0, -448.0)
    ints[3, 128:256] = 0.0                               # an all-zero group: scale 1
    x = ints * np.ldexp(1.0, g.integers(-6, -3, size=(m, k // 128))).repeat(128, axis=1)
    xb = oracle.formats.encode_bf16(x)
    codes = oracle.formats.encode_e4m3(g.integers(-8, 9, size=(1, n, k)).astype(np.float64))
    scales = np.ldexp(1.0, g.integers(-9, -7, size=(1, -(-n // 128), k // 128))).astype(np.float32)
    w = {"codes": codes, "scales": scales}
    hd, od = descs("e4m3", "block", 128, "f32", 1, n, k, act="fp8_group")
    packed = prepare(hd, w, "f32")
    print(f"case fp8 block decode exact tile={tile} split={split}", flush=True)
    out = hum.linear(hd, packed, dev(xb), cfg=cfg(tile, split))
    torch.cuda.synchronize()
    q, s = oracle.quant.quant_fp8_group(oracle.formats.decode_bf16(xb).astype(np.float32))
    a = oracle.quant.dequant_fp8_group(q, s)
    assert np.array_equal(a, oracle.formats.decode_bf16(xb))
    ref = oracle.gemm.linear(od, a, w["codes"], w["scales"])
    assert_bf16_exact(out, ref, f"tile={tile} split={split}")
    qa, sa = hum.quant_act("fp8_group", dev(xb))
    with pytest.raises(hum.HumError, match="quantizes its activations itself"):
        hum.linear(hd, packed, qa, a_scales=sa, cfg=cfg(tile, split))


@pytest.mark.parametrize("tile,m,k", [((1, 1, 4, 1, 8), 1, 32768), ((1, 1, 2, 1, 8), 2, 8192), ((1, 1, 1, 1, 4), 2, 8192)],
                         ids=lambda v: "-".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_fp8_block_decode_kernel_long_k(tile, m, k):
    """Block-scaled FP8 on the decode kernel with long K ranges per wave (32
    K-blocks of four sub-tiles at K = 32768: 128 block scales staged per
    wave) against the oracle, ragged N."""
    n = 328
    w = synth.quant_weights(synth.seed_for(7, 50 + m), "e4m3", "block", 128, "f32", 1, n, k,
                            scale_lo=0.0005, scale_hi=0.002)
    xb = synth.bf16_normal(synth.rng(synth.seed_for(7, 150 + m)), (m, k))
    hd, od = descs("e4m3", "block", 128, "f32", 1, n, k, act="fp8_group")
    packed = prepare(hd, w, "f32")
    print(f"case fp8 block decode long k tile={tile} m={m}", flush=True)
    out = hum.linear(hd, packed, dev(xb), cfg=cfg(tile, 1))
    torch.cuda.synchronize()
    q, s = oracle.quant.quant_fp8_group(oracle.formats.decode_bf16(xb).astype(np.float32))
    ref = oracle.gemm.linear(od, oracle.quant.dequant_fp8_group(q, s), w["codes"], w["scales"])
    assert_tol(out, ref, f"fp8 block long k m={m} tile={tile}")


@pytest.mark.parametrize("m", [1, 7, 16, 100, 300])
def test_fp8_block_dense_random_vs_oracle(m):
    """Block-scaled FP8 W8A8 at the selector's config (ragged N)."""
    n, k = 600, 2048
    w = synth.quant_weights(synth.seed_for(7, m), "e4m3", "block", 128, "f32", 1, n, k,
                            scale_lo=0.0005, scale_hi=0.002)
    xb = synth.bf16_normal(synth.rng(synth.seed_for(7, 100 + m)), (m, k))
    hd, od = descs("e4m3", "block", 128, "f32", 1, n, k, act="fp8_group")
    packed = prepare(hd, w, "f32")
    out = hum.linear(hd, packed, dev(xb))
    torch.cuda.synchronize()
    q, s = oracle.quant.quant_fp8_group(oracle.formats.decode_bf16(xb).astype(np.float32))
    ref = oracle.gemm.linear(od, oracle.quant.dequant_fp8_group(q, s), w["codes"], w["scales"])
    assert_tol(out, ref, f"fp8 block m={m}")


@pytest.mark.parametrize("tile", DENSE_TILES, ids=lambda t: "t" + "".join(map(str, t)))
def test_fp8_weights_bf16_act_exact_every_tile(tile):
    """W8A16 with E4M3 weights: integer bf16 activations in [-8, 8], E4M3
    codes of integers in [-8, 8] with power-of-two per-channel scales; every
    sum is exact in fp32: bitwise equal to the oracle (decode and tile
    kernels alike)."""
    m, n, k = rows_for(tile, 23), 272, 1024
    g = synth.rng(39)
    xb = synth.bf16_bits(g.integers(-8, 9, size=(m, k)).astype(np.float32))
    codes = oracle.formats.encode_e4m3(g.integers(-8, 9, size=(1, n, k)).astype(np.float64))
    scales = np.ldexp(1.0, g.integers(-9, -6, size=(1, n, 1))).astype(np.float32)
    w = {"codes": codes, "scales": scales}
    hd, od = descs("e4m3", "channel", 0, "f32", 1, n, k, act="bf16")
    packed = prepare(hd, w, "f32")
    print(f"case w8a16 fp8 exact tile={tile}", flush=True)
    if not stream_fits(tile, m, k, 2):
        with pytest.raises(hum.HumError, match="raise split_k"):
            hum.linear(hd, packed, dev(xb), cfg=cfg(tile, 2))
        return
    out = hum.linear(hd, packed, dev(xb), cfg=cfg(tile, 2))
    torch.cuda.synchronize()
    ref = oracle.gemm.linear(od, oracle.formats.decode_bf16(xb), w["codes"], w["scales"])
    assert_bf16_exact(out, ref, f"tile={tile}")


@pytest.mark.parametrize("m", [1, 4, 16, 100, 300])
def test_fp8_weights_bf16_act_random_vs_oracle(m):
    """W8A16 with E4M3 weights (per-channel scales) at the selector's config."""
    n, k = 600, 2048
    w = synth.dense_w8a8(synth.seed_for(8, m), 1, n, k)
    xb = synth.bf16_normal(synth.rng(synth.seed_for(8, 100 + m)), (m, k))
    hd, od = descs("e4m3", "channel", 0, "f32", 1, n, k, act="bf16")
    packed = prepare(hd, w, "f32")
    out = hum.linear(hd, packed, dev(xb))
    torch.cuda.synchronize()
    ref = oracle.gemm.linear(od, oracle.formats.decode_bf16(xb), w["codes"], w["scales"])
    assert_tol(out, ref, f"w8a16 fp8 m={m}")


@pytest.mark.parametrize("tile", DENSE_TILES, ids=lambda t: "t" + "".join(map(str, t)))
def test_int8_weights_exact_every_tile(tile):
    """W8A16 with INT8 weights: integer bf16 activations in [-8, 8], every
    INT8 code (-128..127), power-of-two per-channel scales; all sums are
    exact in fp32: bitwise equal to the oracle (decode and tile kernels)."""
    m, n, k = rows_for(tile, 23), 272, 1024
    g = synth.rng(41)
    xb = synth.bf16_bits(g.integers(-8, 9, size=(m, k)).astype(np.float32))
    codes = g.integers(0, 256, size=(1, n, k), dtype=np.uint8)
    scales = np.ldexp(1.0, g.integers(-12, -8, size=(1, n, 1))).astype(np.float32)
    w = {"codes": codes, "scales": scales}
    hd, od = descs("int8", "channel", 0, "f32", 1, n, k)
    packed = prepare(hd, w, "f32")
    print(f"case w8a16 int8 exact tile={tile}", flush=True)
    if not stream_fits(tile, m, k, 2):
        with pytest.raises(hum.HumError, match="raise split_k"):
            hum.linear(hd, packed, dev(xb), cfg=cfg(tile, 2))
        return
    out = hum.linear(hd, packed, dev(xb), cfg=cfg(tile, 2))
    torch.cuda.synchronize()
    ref = oracle.gemm.linear(od, oracle.formats.decode_bf16(xb), w["codes"], w["scales"])
    assert_bf16_exact(out, ref, f"tile={tile}")


@pytest.mark.parametrize("gran", ["channel", "tensor"])
@pytest.mark.parametrize("m", [1, 4, 16, 100, 300])
def test_int8_weights_random_vs_oracle(m, gran):
    """W8A16 with INT8 weights at the selector's config."""
    n, k = 600, 2048
    w = synth.quant_weights(synth.seed_for(9, m), "int8", gran, 0, "f32", 1, n, k, scale_lo=0.0002, scale_hi=0.001)
    xb = synth.bf16_normal(synth.rng(synth.seed_for(9, 100 + m)), (m, k))
    hd, od = descs("int8", gran, 0, "f32", 1, n, k)
    packed = prepare(hd, w, "f32")
    out = hum.linear(hd, packed, dev(xb))
    torch.cuda.synchronize()
    ref = oracle.gemm.linear(od, oracle.formats.decode_bf16(xb), w["codes"], w["scales"])
    assert_tol(out, ref, f"w8a16 int8 m={m} {gran}")


@pytest.mark.parametrize("tile", DENSE_TILES, ids=lambda t: "t" + "".join(map(str, t)))
def test_nvfp4_exact_every_tile(tile):
    """NVFP4 x bf16: every E2M1 code, power-of-two E4M3 group scales (one per
    16 along K), a power-of-two tensor scale and integer activations in
    [-8, 8]: all sums exact in fp32, so bitwise equal to the oracle (decode
    and tile kernels)."""
    m, n, k = rows_for(tile, 23), 272, 1024
    g = synth.rng(43)
    xb = synth.bf16_bits(g.integers(-8, 9, size=(m, k)).astype(np.float32))
    w = synth.quant_weights(43, "e2m1", "group", 16, "e4m3", 1, n, k, global_scale=True)
    w["scales"] = (g.integers(5, 10, size=w["scales"].shape) << 3).astype(np.uint8)   # 2^-2 .. 2^2
    w["global_scale"] = np.array([0.5], np.float32)
    hd, od = descs("e2m1", "group", 16, "e4m3", 1, n, k, glob=True)
    packed = prepare(hd, w, "e4m3")
    print(f"case nvfp4 exact tile={tile}", flush=True)
    if not stream_fits(tile, m, k, 2):
        with pytest.raises(hum.HumError, match="raise split_k"):
            hum.linear(hd, packed, dev(xb), cfg=cfg(tile, 2))
        return
    out = hum.linear(hd, packed, dev(xb), cfg=cfg(tile, 2))
    torch.cuda.synchronize()
    ref = oracle.gemm.linear(od, oracle.formats.decode_bf16(xb), w["codes"], w["scales"], None, w["global_scale"])
    assert_bf16_exact(out, ref, f"tile={tile}")


@pytest.mark.parametrize("m", [1, 7, 16, 100, 300])
def test_nvfp4_random_vs_oracle(m):
    """NVFP4 x bf16 at the selector's config: random E4M3 group scales
    (subnormal to 1) and a tensor scale."""
    n, k = 600, 2048
    w = synth.quant_weights(synth.seed_for(10, m), "e2m1", "group", 16, "e4m3", 1, n, k, global_scale=True,
                            e4m3_lo=0x04, e4m3_hi=0x38)
    xb = synth.bf16_normal(synth.rng(synth.seed_for(10, 100 + m)), (m, k))
    hd, od = descs("e2m1", "group", 16, "e4m3", 1, n, k, glob=True)
    packed = prepare(hd, w, "e4m3")
    out = hum.linear(hd, packed, dev(xb))
    torch.cuda.synchronize()
    ref = oracle.gemm.linear(od, oracle.formats.decode_bf16(xb), w["codes"], w["scales"], None, w["global_scale"])
    assert_tol(out, ref, f"nvfp4 m={m}")


@pytest.mark.parametrize("tile", DENSE_TILES, ids=lambda t: "t" + "".join(map(str, t)))
def test_mxint4_exact_every_tile(tile):
    """MXINT4 x bf16: every INT4 code, E8M0 scales 2^-3 .. 2^1 per 32 along
    K, integer activations in [-8, 8]: all sums exact in fp32, so bitwise
    equal to the oracle (decode and tile kernels)."""
    m, n, k = rows_for(tile, 23), 272, 1024
    g = synth.rng(47)
    xb = synth.bf16_bits(g.integers(-8, 9, size=(m, k)).astype(np.float32))
    w = synth.quant_weights(47, "int4", "group", 32, "e8m0", 1, n, k, e8m0_lo=124, e8m0_hi=128)
    hd, od = descs("int4", "group", 32, "e8m0", 1, n, k)
    packed = prepare(hd, w, "e8m0")
    print(f"case mxint4 exact tile={tile}", flush=True)
    if not stream_fits(tile, m, k, 2):
        with pytest.raises(hum.HumError, match="raise split_k"):
            hum.linear(hd, packed, dev(xb), cfg=cfg(tile, 2))
        return
    out = hum.linear(hd, packed, dev(xb), cfg=cfg(tile, 2))
    torch.cuda.synchronize()
    ref = oracle.gemm.linear(od, oracle.formats.decode_bf16(xb), w["codes"], w["scales"])
    assert_bf16_exact(out, ref, f"tile={tile}")


@pytest.mark.parametrize("m", [1, 7, 16, 100, 300])
def test_mxint4_random_vs_oracle(m):
    """MXINT4 x bf16 at the selector's config."""
    n, k = 600, 2048
    w = synth.quant_weights(synth.seed_for(12, m), "int4", "group", 32, "e8m0", 1, n, k)
    xb = synth.bf16_normal(synth.rng(synth.seed_for(12, 100 + m)), (m, k))
    hd, od = descs("int4", "group", 32, "e8m0", 1, n, k)
    packed = prepare(hd, w, "e8m0")
    out = hum.linear(hd, packed, dev(xb))
    torch.cuda.synchronize()
    ref = oracle.gemm.linear(od, oracle.formats.decode_bf16(xb), w["codes"], w["scales"])
    assert_tol(out, ref, f"mxint4 m={m}")


@pytest.mark.parametrize("m", [1, 7, 16, 100, 300])
def test_w4a8_dense_random_vs_oracle(m):
    """Dense W4A8 (MXFP4 weights x MXFP8 activations) at the selector's config."""
    n, k = 640, 2048
    w = synth.moe_weights_mxfp4(synth.seed_for(5, m), 1, n, k)
    xb = synth.bf16_normal(synth.rng(synth.seed_for(5, 100 + m)), (m, k))
    hd, od = descs("e2m1", "group", 32, "e8m0", 1, n, k, act="mxfp8")
    packed = prepare(hd, w, "e8m0")
    out = hum.linear(hd, packed, dev(xb))
    torch.cuda.synchronize()
    q, e = oracle.quant.quant_mxfp8(oracle.formats.decode_bf16(xb).astype(np.float32))
    ref = oracle.gemm.linear(od, oracle.quant.dequant_mxfp8(q, e), w["codes"], w["scales"])
    assert_tol(out, ref, f"w4a8 m={m}")


def test_workload_dense_int4_sym_g128_tiny():
    """Dense W4A16 INT4 symmetric G128, M=16 N=512 K=1024 (selector config)."""
    case = synth.dense_w4a16(synth.seed_for(1), 16, 512, 1024, group=128)
    hd, od = descs("int4", "group", 128, "bf16", 1, 512, 1024)
    packed = prepare(hd, case, "bf16")
    out = hum.linear(hd, packed, dev(case["x"]))
    torch.cuda.synchronize()
    ref = oracle.gemm.linear(od, oracle.formats.decode_bf16(case["x"]), case["codes"], case["scales"])
    assert_tol(out, ref, "cfg1")


@pytest.mark.parametrize("m", [1, 4, 16, 33, 64, 130, 300])
def test_uint4_zp_random_vs_oracle(m):
    n, k = 640, 2048
    case = synth.dense_w4a16(synth.seed_for(2, m), m, n, k, group=128, asym=True)
    hd, od = descs("uint4", "group", 128, "bf16", 1, n, k, zero=True)
    packed = prepare(hd, case, "bf16")
    out = hum.linear(hd, packed, dev(case["x"]))
    torch.cuda.synchronize()
    ref = oracle.gemm.linear(od, oracle.formats.decode_bf16(case["x"]), case["codes"], case["scales"], case["zeros"])
    assert_tol(out, ref, f"m={m}")


@pytest.mark.parametrize("tile", DENSE_TILES, ids=lambda t: "t" + "".join(map(str, t)))
def test_fp8_w8a8_every_tile(tile):
    m, n, k = rows_for(tile, 21), 320, 1024
    case = synth.dense_w8a8(synth.seed_for(3, 7), m, n, k)
    hd, od = descs("e4m3", "channel", 0, "f32", 1, n, k, act="fp8_token")
    packed = prepare(hd, case, "f32")
    out = hum.linear(hd, packed, dev(case["x"]), cfg=cfg(tile, 2))
    torch.cuda.synchronize()
    q, s = oracle.quant.quant_fp8_per_token(oracle.formats.decode_bf16(case["x"]).astype(np.float32))
    a = oracle.quant.dequant_fp8_per_token(q, s)
    ref = oracle.gemm.linear(od, a, case["codes"], case["scales"])
    assert_tol(out, ref, f"tile={tile}")


@pytest.mark.parametrize("m", [1, 16, 128, 257])
def test_fp8_w8a8_selector_vs_oracle(m):
    n, k = 7168 // 8, 2048
    case = synth.dense_w8a8(synth.seed_for(3, m), m, n, k)
    hd, od = descs("e4m3", "channel", 0, "f32", 1, n, k, act="fp8_token")
    packed = prepare(hd, case, "f32")
    out = hum.linear(hd, packed, dev(case["x"]))
    torch.cuda.synchronize()
    q, s = oracle.quant.quant_fp8_per_token(oracle.formats.decode_bf16(case["x"]).astype(np.float32))
    ref = oracle.gemm.linear(od, oracle.quant.dequant_fp8_per_token(q, s), case["codes"], case["scales"])
    assert_tol(out, ref, f"m={m}")


@pytest.mark.parametrize("tile", STREAM_TILES, ids=lambda t: "t" + "".join(map(str, t)))
@pytest.mark.parametrize("m,k", [(1, 1024), (3, 1024), (8, 1024), (16, 1024), (2, 7168), (5, 384), (1, 8192)])
def test_fp8_w8a8_decode_quantizes_in_kernel(tile, m, k):
    """Per-token FP8 activations on the decode kernel without split-K are
    quantized inside the kernel: the output equals the quantizer launch
    followed by the same kernel bit for bit (same codes and scales), and
    meets the oracle's tolerance.  Rows: an all-zero row (scale 1), a row of
    large values and N(0,1) rows; K ranges that leave waves without
    K-blocks."""
    n = 320
    if not stream_fits(tile, m, k, 1, 8):
        pytest.skip("K range per wave too long for this tile at split 1")
    kb, kw = k // 128, tile[4]
    fused = m * -(-kb // kw) * 8 <= 256   # else the quantizer launch runs (same result)
    case = synth.dense_w8a8(synth.seed_for(3, 40 + m), m, n, k)
    xb = case["x"].copy()
    if m >= 3:
        xb[0] = 0
        big = oracle.formats.decode_bf16(xb[1]) * 3e3
        xb[1] = torch.from_numpy(big.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    hd, od = descs("e4m3", "channel", 0, "f32", 1, n, k, act="fp8_token")
    packed = prepare(hd, case, "f32")
    x = dev(xb)
    print(f"case fp8 in-kernel quant tile={tile} m={m} k={k} fused={fused}", flush=True)
    o_fused = hum.linear(hd, packed, x, cfg=cfg(tile, 1))
    q, s = hum.quant_act("fp8_token", x)
    o_two = hum.linear(hd, packed, q, a_scales=s, cfg=cfg(tile, 1))
    torch.cuda.synchronize()
    assert torch.equal(o_fused.view(torch.int16), o_two.view(torch.int16)), f"tile={tile} m={m} k={k}"
    qo, so = oracle.quant.quant_fp8_per_token(oracle.formats.decode_bf16(xb).astype(np.float32))
    ref = oracle.gemm.linear(od, oracle.quant.dequant_fp8_per_token(qo, so), case["codes"], case["scales"])
    assert_tol(o_fused, ref, f"tile={tile} m={m} k={k}")


def test_fp8_prequantized_activations_match_internal_quant():
    m, n, k = 33, 256, 1024
    case = synth.dense_w8a8(91, m, n, k)
    hd, _ = descs("e4m3", "channel", 0, "f32", 1, n, k, act="fp8_token")
    packed = prepare(hd, case, "f32")
    x = dev(case["x"])
    q, s = hum.quant_act("fp8_token", x)
    o1 = hum.linear(hd, packed, x)
    o2 = hum.linear(hd, packed, q, a_scales=s)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_bias_and_global_scale():
    m, n, k = 12, 100, 768
    w = synth.quant_weights(41, "uint4", "group", 256, "f32", 1, n, k, zero=True, global_scale=True,
                            scale_lo=0.01, scale_hi=0.05)
    g = synth.rng(42)
    xb = synth.bf16_normal(g, (m, k))
    bias = synth.bf16_normal(g, (n,))
    hd, od = descs("uint4", "group", 256, "f32", 1, n, k, zero=True, glob=True)
    packed = prepare(hd, w, "f32")
    out = hum.linear(hd, packed, dev(xb), bias=dev(bias))
    torch.cuda.synchronize()
    ref = oracle.gemm.linear(od, oracle.formats.decode_bf16(xb), w["codes"], w["scales"], w["zeros"],
                             w["global_scale"], bias_bits=bias)
    assert_tol(out, ref, "bias+global")


def test_channel_and_tensor_scales():
    m, n, k = 8, 64, 512
    for gran in ("channel", "tensor"):
        w = synth.quant_weights(43, "int4", gran, 0, "f32", 1, n, k)
        xb = synth.bf16_normal(synth.rng(44), (m, k))
        hd, od = descs("int4", gran, 0, "f32", 1, n, k)
        out = hum.linear(hd, prepare(hd, w, "f32"), dev(xb))
        torch.cuda.synchronize()
        ref = oracle.gemm.linear(od, oracle.formats.decode_bf16(xb), w["codes"], w["scales"])
        assert_tol(out, ref, gran)


def test_zero_codes_equal_zero_point_give_zero():
    """q == z everywhere -> exactly zero output (integer activations keep
    every fp32 partial sum exact, so the offset correction cancels exactly);
    with real-valued activations the residue stays at fp32 rounding level."""
    m, n, k = 4, 48, 256
    w = synth.quant_weights(45, "uint4", "group", 128, "bf16", 1, n, k, zero=True)
    w["codes"] = synth.pack_nibbles(np.repeat(w["zeros"], 128, axis=2))
    hd, _ = descs("uint4", "group", 128, "bf16", 1, n, k, zero=True)
    packed = prepare(hd, w, "bf16")
    xi = synth.bf16_bits(synth.rng(46).integers(-8, 9, size=(m, k)).astype(np.float32))
    out = hum.linear(hd, packed, dev(xi))
    xr = synth.bf16_normal(synth.rng(46), (m, k))
    out_r = hum.linear(hd, packed, dev(xr))
    torch.cuda.synchronize()
    assert torch.all(out.float() == 0)
    # bound: fp32 rounding of the two K-block sums, |sum a*(128+z)| * s * 2^-20
    a = np.abs(oracle.formats.decode_bf16(xr)).sum(axis=1)
    bound = a * 143 * 0.02 * 2.0 ** -20
    assert np.all(np.abs(out_r.float().cpu().numpy()) <= bound[:, None])


def test_repeat_runs_are_bitwise_identical():
    m, n, k = 3, 2048, 4096
    case = synth.dense_w4a16(47, m, n, k, group=128, asym=True)
    hd, _ = descs("uint4", "group", 128, "bf16", 1, n, k, zero=True)
    packed = prepare(hd, case, "bf16")
    x = dev(case["x"])
    c = hum.select_config(hd, m)
    assert c.split_k > 1
    o1 = hum.linear(hd, packed, x).clone()
    o2 = hum.linear(hd, packed, x)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("fmt", ["uint4", "e4m3", "e4m3_block", "e4m3_bf16", "int8", "nvfp4", "mxint4", "e2m1_mxfp8", "e2m1_mxfp4"])
def test_empty_m_is_a_no_op(fmt):
    """M = 0: a valid call that writes nothing (every format's path)."""
    n, k = 256, 512
    if fmt == "uint4":
        w = synth.quant_weights(50, "uint4", "group", 128, "bf16", 1, n, k, zero=True)
        hd, _ = descs("uint4", "group", 128, "bf16", 1, n, k, zero=True)
        packed = prepare(hd, w, "bf16")
    elif fmt == "e4m3":
        w = synth.dense_w8a8(synth.seed_for(3, 50), 1, n, k)
        hd, _ = descs("e4m3", "channel", 0, "f32", 1, n, k, act="fp8_token")
        packed = prepare(hd, w, "f32")
    elif fmt == "mxint4":
        w = synth.quant_weights(synth.seed_for(3, 56), "int4", "group", 32, "e8m0", 1, n, k)
        hd, _ = descs("int4", "group", 32, "e8m0", 1, n, k)
        packed = prepare(hd, w, "e8m0")
    elif fmt == "nvfp4":
        w = synth.quant_weights(synth.seed_for(3, 55), "e2m1", "group", 16, "e4m3", 1, n, k)
        hd, _ = descs("e2m1", "group", 16, "e4m3", 1, n, k)
        packed = prepare(hd, w, "e4m3")
    elif fmt == "int8":
        w = synth.quant_weights(synth.seed_for(3, 54), "int8", "channel", 0, "f32", 1, n, k)
        hd, _ = descs("int8", "channel", 0, "f32", 1, n, k)
        packed = prepare(hd, w, "f32")
    elif fmt == "e4m3_bf16":
        w = synth.dense_w8a8(synth.seed_for(3, 53), 1, n, k)
        hd, _ = descs("e4m3", "channel", 0, "f32", 1, n, k, act="bf16")
        packed = prepare(hd, w, "f32")
    elif fmt == "e4m3_block":
        w = synth.quant_weights(52, "e4m3", "block", 128, "f32", 1, n, k)
        hd, _ = descs("e4m3", "block", 128, "f32", 1, n, k, act="fp8_group")
        packed = prepare(hd, w, "f32")
    else:
        w = synth.moe_weights_mxfp4(51, 1, n, k)
        hd, _ = descs("e2m1", "group", 32, "e8m0", 1, n, k, act=fmt.split("_")[1])
        packed = prepare(hd, w, "e8m0")
    x = torch.empty((0, k), dtype=torch.bfloat16, device="cuda")
    out = hum.linear(hd, packed, x)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (0, n)


@pytest.mark.parametrize("wd", ["uint4", "e2m1"])
@pytest.mark.parametrize("tile", TILE32_TILES, ids=lambda t: "t" + "".join(map(str, t)))
@pytest.mark.parametrize("m", [33, 300])
def test_tile32_random_vs_oracle(wd, tile, m):
    """32x32-block tiles on random data, ragged M and N, bias (MXFP4 also
    with a global scale), against the oracle at the bf16-output bound."""
    n, k = 592, 1024
    if wd == "uint4":
        w = synth.quant_weights(950 + m, "uint4", "group", 128, "bf16", 1, n, k, zero=True)
        hd, od = descs("uint4", "group", 128, "bf16", 1, n, k, zero=True)
        sd = "bf16"
    else:
        w = synth.quant_weights(951 + m, "e2m1", "group", 32, "e8m0", 1, n, k, global_scale=True)
        hd, od = descs("e2m1", "group", 32, "e8m0", 1, n, k, glob=True)
        sd = "e8m0"
    xb = synth.bf16_normal(synth.rng(952 + m), (m, k))
    bias = synth.bf16_normal(synth.rng(953), (n,))
    packed = prepare(hd, w, sd)
    for split in (1, 2):
        out = hum.linear(hd, packed, dev(xb), bias=dev(bias), cfg=cfg(tile, split))
        torch.cuda.synchronize()
        ref = oracle.gemm.linear(od, oracle.formats.decode_bf16(xb), w["codes"], w["scales"], w.get("zeros"),
                                 w.get("global_scale"), bias_bits=bias)
        assert_tol(out, ref, f"{wd} tile={tile} m={m} split={split}")
