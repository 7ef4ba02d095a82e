"""Pins of the oracle's dequantization and dense layer: a pure-Python
Fraction triple loop with scalar decoders of its own, and the invariants the
description implies (G = K equals per-channel, q == z gives zero output,
exact-integer cases equal to the bit)."""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import gemm as G
from oracle.formats import decode_bf16
from synth import bf16_bits, pack_bits, pack_nibbles, seed_of

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def s_int4(c):
    return c - 16 if c >= 8 else c


def s_int8(c):
    return c - 256 if c >= 128 else c


def s_intb(c, b):
    return c - (1 << b) if c >= (1 << (b - 1)) else c


def s_fp6(c, ebits):
    """FP6 code -> exact rational from its bit fields (OCP MX: E2M3 bias 1,
    E3M2 bias 3; exponent 0 subnormal)."""
    mbits, bias = 5 - ebits, (1 if ebits == 2 else 3)
    s, e, m = c >> 5, (c >> mbits) & ((1 << ebits) - 1), c & ((1 << mbits) - 1)
    v = Fraction(m, 1 << mbits) * Fraction(2) ** (1 - bias) if e == 0 else \
        (1 + Fraction(m, 1 << mbits)) * Fraction(2) ** (e - bias)
    return -v if s else v


def s_e2m1(c):
    v = E2M1[c & 7]
    return -v if c & 8 else v


def s_e4m3(c):
    return float(torch.tensor([c], dtype=torch.uint8).view(torch.float8_e4m3fn).float()[0])


def s_bf16(b):
    return struct.unpack("<f", struct.pack("<I", int(b) << 16))[0]


def s_scale(v, dtype):
    if dtype == "bf16":
        return Fraction(s_bf16(v))
    if dtype == "f32":
        return Fraction(float(np.float32(v)))
    if dtype == "e4m3":
        return Fraction(s_e4m3(int(v)))
    return Fraction(2) ** (int(v) - 127)


def brute_linear(desc, a_vals, codes_unpacked, scales, zeros, gscale):
    """C[m][n] with exact rationals, one scalar at a time."""
    dec = {"int4": s_int4, "uint4": lambda c: c, "int8": s_int8, "e2m1": s_e2m1, "e4m3": s_e4m3,
           "int3": lambda c: s_intb(c, 3), "int2": lambda c: s_intb(c, 2), "int1": lambda c: s_intb(c, 1),
           "uint3": lambda c: c, "uint2": lambda c: c, "uint1": lambda c: c,
           "e2m3": lambda c: s_fp6(c, 2), "e3m2": lambda c: s_fp6(c, 3)}[desc.weight_dtype]
    m, k = len(a_vals), desc.k
    out = []
    for i in range(m):
        row = []
        for n in range(desc.n):
            acc = Fraction(0)
            for kk in range(k):
                if desc.scale_gran == "block":
                    gi, ni = kk // desc.group_size, n // desc.group_size
                elif desc.scale_gran == "group":
                    gi, ni = kk // desc.group_size, n
                elif desc.scale_gran == "channel":
                    gi, ni = 0, n
                else:
                    gi, ni = 0, 0
                v = Fraction(dec(int(codes_unpacked[n][kk])))
                if desc.has_zero:
                    v -= int(zeros[ni][gi])
                w = v * s_scale(scales[ni][gi], desc.scale_dtype)
                if desc.has_global:
                    w *= Fraction(float(np.float32(gscale)))
                acc += Fraction(float(a_vals[i][kk])) * w
            row.append(acc)
        out.append(row)
    return out


CASES = [
    ("int4", "group", 16, "bf16", False, False),
    ("uint4", "group", 16, "bf16", True, False),
    ("uint4", "channel", 0, "f32", True, True),
    ("int4", "tensor", 0, "f32", False, True),
    ("e2m1", "group", 32, "e8m0", False, False),
    ("e2m1", "group", 16, "bf16", False, True),
    ("e4m3", "channel", 0, "f32", False, False),
    ("e4m3", "block", 16, "f32", False, False),
    ("int8", "channel", 0, "f32", False, False),
    ("e2m1", "group", 16, "e4m3", False, True),
    ("int4", "group", 32, "e8m0", False, False),
    ("int8", "tensor", 0, "f32", False, True),
    ("int3", "group", 16, "bf16", False, False),
    ("uint3", "group", 32, "bf16", True, False),
    ("int2", "channel", 0, "f32", False, False),
    ("uint2", "group", 16, "f32", True, True),
    ("int1", "group", 32, "bf16", False, False),
    ("uint1", "tensor", 0, "f32", True, False),
    ("e2m3", "group", 32, "e8m0", False, False),
    ("e3m2", "group", 32, "e8m0", False, True),
]
BITS = {"int3": 3, "uint3": 3, "int2": 2, "uint2": 2, "int1": 1, "uint1": 1, "e2m3": 6, "e3m2": 6}


@pytest.mark.parametrize("wd,gran,gs,sd,zp,gl", CASES)
def test_linear_vs_fraction_brute_force(wd, gran, gs, sd, zp, gl):
    g = np.random.default_rng(seed_of(wd, gran, gs, sd))
    m, n, k = 3, (40 if gran == "block" else 5), 64
    desc = G.WeightDesc(wd, gran, gs, sd, zp, gl, 1, n, k)
    ng = desc.groups()
    sn = 1 if gran == "tensor" else (-(-n // gs) if gran == "block" else n)
    if wd == "e4m3":
        cu = g.integers(0, 256, size=(n, k))
        cu = np.where((cu & 0x7F) == 0x7F, 0x7E, cu).astype(np.uint8)
        codes = cu[None]
    elif wd == "int8":
        cu = g.integers(0, 256, size=(n, k)).astype(np.uint8)
        codes = cu[None]
    elif wd in BITS:
        cu = g.integers(0, 1 << BITS[wd], size=(n, k)).astype(np.uint8)
        codes = pack_bits(cu, BITS[wd])[None]
    else:
        cu = g.integers(0, 16, size=(n, k)).astype(np.uint8)
        codes = pack_nibbles(cu)[None]
    if sd == "bf16":
        sc = bf16_bits(g.uniform(0.005, 0.02, size=(sn, ng)).astype(np.float32))
    elif sd == "f32":
        sc = g.uniform(0.01, 0.1, size=(sn, ng)).astype(np.float32)
    elif sd == "e4m3":
        sc = g.integers(0x08, 0x7F, size=(sn, ng)).astype(np.uint8)   # positive finite, subnormals included
    else:
        sc = g.integers(119, 124, size=(sn, ng)).astype(np.uint8)
    zeros = g.integers(0, 1 << BITS.get(wd, 4), size=(sn, ng)).astype(np.uint8) if zp else None
    gsc = np.array([0.75], np.float32)
    a_bits = bf16_bits(g.standard_normal((m, k)).astype(np.float32))
    a = decode_bf16(a_bits)
    got = G.linear(desc, a, codes, sc[None], None if zeros is None else zeros[None], gsc)
    ref = brute_linear(desc, a.tolist(), cu, sc, zeros, gsc[0])
    for i in range(m):
        for j in range(n):
            r = float(ref[i][j])
            assert abs(got[i, j] - r) <= 1e-12 * max(1.0, abs(r)), (i, j, got[i, j], r)


def test_exact_integer_case_is_exact():
    # Integer activations and power-of-two scales: every product and partial
    # sum is exactly representable, so the fp64 result equals the rational one.
    g = np.random.default_rng(20)
    m, n, k = 4, 6, 128
    desc = G.WeightDesc("uint4", "group", 32, "bf16", True, False, 1, n, k)
    cu = g.integers(0, 16, size=(n, k)).astype(np.uint8)
    sc = bf16_bits(np.full((n, 4), 2.0 ** -4, np.float32))
    z = g.integers(0, 16, size=(n, 4)).astype(np.uint8)
    a = g.integers(-8, 9, size=(m, k)).astype(np.float64)
    got = G.linear(desc, a, pack_nibbles(cu)[None], sc[None], z[None])
    ref = brute_linear(desc, a.tolist(), cu, sc, z, None)
    assert all(got[i, j] == ref[i][j] for i in range(m) for j in range(n))


def test_group_equals_k_is_channel():
    g = np.random.default_rng(21)
    n, k = 8, 256
    cu = pack_nibbles(g.integers(0, 16, size=(1, n, k)).astype(np.uint8))
    sc = bf16_bits(g.uniform(0.005, 0.02, size=(1, n, 1)).astype(np.float32))
    z = g.integers(0, 16, size=(1, n, 1)).astype(np.uint8)
    a = decode_bf16(bf16_bits(g.standard_normal((5, k)).astype(np.float32)))
    d_g = G.WeightDesc("uint4", "group", k, "bf16", True, False, 1, n, k)
    d_c = G.WeightDesc("uint4", "channel", 0, "bf16", True, False, 1, n, k)
    assert np.array_equal(G.linear(d_g, a, cu, sc, z), G.linear(d_c, a, cu, sc, z))


def test_codes_equal_zero_point_give_zero():
    g = np.random.default_rng(22)
    n, k, gs = 8, 256, 128
    z = g.integers(0, 16, size=(1, n, k // gs)).astype(np.uint8)
    cu = np.repeat(z, gs, axis=2)
    sc = bf16_bits(g.uniform(0.005, 0.02, size=(1, n, k // gs)).astype(np.float32))
    a = decode_bf16(bf16_bits(g.standard_normal((3, k)).astype(np.float32)))
    d = G.WeightDesc("uint4", "group", gs, "bf16", True, False, 1, n, k)
    out = G.linear(d, a, pack_nibbles(cu), sc, z)
    assert np.all(out == 0)
    # symmetric all-zero codes
    d2 = G.WeightDesc("int4", "group", gs, "bf16", False, False, 1, n, k)
    out2 = G.linear(d2, a, np.zeros((1, n, k // 2), np.uint8), sc)
    assert np.all(out2 == 0)


def test_dequant_weight_per_expert_selection():
    g = np.random.default_rng(23)
    e, n, k = 3, 4, 64
    d = G.WeightDesc("e2m1", "group", 32, "e8m0", False, False, e, n, k)
    codes = pack_nibbles(g.integers(0, 16, size=(e, n, k)).astype(np.uint8))
    sc = g.integers(119, 124, size=(e, n, 2)).astype(np.uint8)
    full = G.dequant_weight(d, codes, sc)
    for i in range(e):
        assert np.array_equal(G.dequant_weight(d, codes, sc, experts=[i])[0], full[i])
        # one element by hand
        c = int(codes[i, 1, 3] >> 4)            # k = 7 -> high nibble of byte 3
        assert full[i, 1, 7] == s_e2m1(c) * math.ldexp(1.0, int(sc[i, 1, 0]) - 127)


def test_w4a4_mxfp4_linear_vs_fraction_brute_force():
    """MXFP4 activations x MXFP4 weights (W4A4): the oracle's composition
    (activation dequant, weight dequant, float64 product) against a scalar
    Fraction sum over E2M1 codes and E8M0 exponents."""
    g = np.random.default_rng(40)
    m, n, k = 3, 5, 64
    from oracle import quant as Q
    x = g.standard_normal((m, k)) * 2.0
    qa, ea = Q.quant_mxfp4(x)
    wc = g.integers(0, 256, size=(1, n, k // 2)).astype(np.uint8)
    we = g.integers(120, 134, size=(1, n, k // 32)).astype(np.uint8)
    od = G.WeightDesc("e2m1", "group", 32, "e8m0", False, False, 1, n, k)
    got = G.linear(od, G.activations("mxfp4", q=qa, scales=ea), wc, we)
    vals = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    dec = lambda c: Fraction(vals[c & 7]) * (-1 if c & 8 else 1)
    for i in range(m):
        for j in range(n):
            acc = Fraction(0)
            for kk in range(k):
                ca = (int(qa[i, kk // 2]) >> (4 * (kk & 1))) & 0xF
                cw = (int(wc[0, j, kk // 2]) >> (4 * (kk & 1))) & 0xF
                sa = Fraction(2) ** (int(ea[i, kk // 32]) - 127)
                sw = Fraction(2) ** (int(we[0, j, kk // 32]) - 127)
                acc += dec(ca) * sa * dec(cw) * sw
            assert got[i, j] == float(acc)


def test_int8_per_channel_equals_integer_matmul():
    """Integer activations, INT8 codes and power-of-two per-channel scales:
    the layer is an integer matrix product (numpy int64) times the scale."""
    g = np.random.default_rng(81)
    m, n, k = 4, 6, 256
    cu = g.integers(0, 256, size=(n, k)).astype(np.uint8)
    q = cu.view(np.int8).astype(np.int64)
    x = g.integers(-20, 21, size=(m, k)).astype(np.int64)
    sc = np.ldexp(1.0, g.integers(-12, -4, size=(n, 1))).astype(np.float32)
    desc = G.WeightDesc("int8", "channel", 0, "f32", False, False, 1, n, k)
    got = G.linear(desc, x.astype(np.float64), cu[None], sc[None])
    ref = (x @ q.T).astype(np.float64) * sc[:, 0].astype(np.float64)[None, :]
    assert np.array_equal(got, ref)


def test_nvfp4_group_scales_per_16():
    """NVFP4: each 16-element group of a row takes its own E4M3 scale; a
    single nonzero code in group g picks up exactly scale g (times the
    global scale)."""
    n, k = 2, 64
    desc = G.WeightDesc("e2m1", "group", 16, "e4m3", False, True, 1, n, k)
    cu = np.zeros((n, k), np.uint8)
    cu[0, 17] = 0x2   # +1.0 in group 1
    cu[1, 63] = 0xF   # -6.0 in group 3
    sc = np.array([[0x38, 0x30, 0x40, 0x48], [0x38, 0x39, 0x3A, 0x3C]], np.uint8)   # 1, .5, 2, 4 / 1, 1.125, 1.25, 1.5
    w = G.dequant_weight(desc, pack_nibbles(cu)[None], sc[None], global_scale=np.array([0.5], np.float32))[0]
    assert w[0, 17] == 0.5 * 0.5 and np.count_nonzero(w[0]) == 1
    assert w[1, 63] == -6.0 * 1.5 * 0.5 and np.count_nonzero(w[1]) == 1


def _e4m3_frac(c):
    """E4M3 "FN" code -> exact rational, from its bit fields (sign, 4-bit
    exponent with bias 7, 3-bit mantissa; exponent 0 is subnormal with
    quantum 2^-9).  NaN codes are never passed."""
    c = int(c)
    s, e, m = c >> 7, (c >> 3) & 15, c & 7
    assert not (e == 15 and m == 7)
    v = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -v if s else v


def _f32_frac(x):
    """The exact value of a float32, through its IEEE bit pattern."""
    b = struct.unpack("<I", struct.pack("<f", float(np.float32(x))))[0]
    s, e, f = b >> 31, (b >> 23) & 0xFF, b & 0x7FFFFF
    v = Fraction(f, 1 << 23) * Fraction(2) ** -126 if e == 0 else (1 + Fraction(f, 1 << 23)) * Fraction(2) ** (e - 127)
    return -v if s else v


@pytest.mark.parametrize("m,n,k", [(3, 5, 64), (64, 3, 64), (4, 4, 128)])
def test_fp8_token_x_fp8_channel_vs_fraction_brute_force(m, n, k):
    """The per-token FP8 x per-channel E4M3 (W8A8) reference as the tests
    compose it -- the quantizer's codes and f32 row scales, dequantized by
    activations("fp8_token") / dequant_fp8_per_token, times the weight through
    linear_fp8_e4m3 and through linear() -- against a Fraction sum of
    v(qa[m,k]) * s_a[m] * v(qw[n,k]) * s_w[n] with bit-field decoders of its
    own.  Row scales differ per row and the shapes include M == K and M == N,
    so a scale broadcast along the wrong axis changes the result; scales are
    not powers of two, so a dequantized operand rounded to f32 (instead of
    the exact product) moves every sum by about 2^-24 relative."""
    from oracle import quant as Q
    g = np.random.default_rng(300 + m + n + k)
    xf = np.clip(g.standard_normal((m, k)), -1.9, 1.9).astype(np.float32)
    for i in range(m):                       # a distinct amax (hence scale) per row
        xf[i, (5 * i) % k] = (2.0 + i / 16.0) * (-1.0 if i & 1 else 1.0)
    x = bf16_bits(xf)
    qa, sa = Q.quant_fp8_per_token(decode_bf16(x).astype(np.float32))
    assert len(set(sa.tolist())) == m        # distinct row scales
    cw = g.integers(0, 256, size=(n, k))
    cw = np.where((cw & 0x7F) == 0x7F, 0x7E, cw).astype(np.uint8)
    sw = g.uniform(1e-3, 4e-3, size=n).astype(np.float32)
    a = G.activations("fp8_token", q=qa, scales=sa)
    # the dequantized activations: exactly v(q) * fl32(s)
    for i in range(m):
        for kk in range(0, k, 7):
            assert Fraction(float(a[i, kk])) == _e4m3_frac(qa[i, kk]) * _f32_frac(sa[i])
    assert np.array_equal(a, Q.dequant_fp8_per_token(qa, sa))
    got1 = G.linear_fp8_e4m3(a, cw, sw)
    od = G.WeightDesc("e4m3", "channel", 0, "f32", False, False, 1, n, k)
    got2 = G.linear(od, a, cw[None], sw.reshape(1, n, 1))
    for i in range(m):
        for j in range(n):
            terms = [_e4m3_frac(qa[i, kk]) * _f32_frac(sa[i]) * _e4m3_frac(cw[j, kk]) * _f32_frac(sw[j])
                     for kk in range(k)]
            ref = sum(terms, Fraction(0))
            bound = 1e-13 * float(sum(abs(t) for t in terms))
            assert abs(got1[i, j] - float(ref)) <= bound, (i, j, got1[i, j], float(ref))
            assert abs(got2[i, j] - float(ref)) <= bound, (i, j, got2[i, j], float(ref))


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_bit_stream_unpacking_against_big_integer(bits):
    """Code k of a canonical b-bit row is bits b*k .. b*k+b-1 of the row read
    as one little-endian integer: checked through Python's arbitrary
    precision integers, and for b = 4 against the nibble reading."""
    from oracle.formats import unpack_bits, unpack_nibbles
    g = np.random.default_rng(90 + bits)
    rows = g.integers(0, 256, size=(3, 12 * bits)).astype(np.uint8)
    got = unpack_bits(rows, bits)
    assert got.shape == (3, 96)
    for r in range(3):
        big = int.from_bytes(bytes(rows[r].tolist()), "little")
        want = [(big >> (bits * kk)) & ((1 << bits) - 1) for kk in range(96)]
        assert got[r].tolist() == want
    if bits == 4:
        assert np.array_equal(got, unpack_nibbles(rows))


def test_int3_stream_golden_bytes():
    """Eight 3-bit codes 1..7, 0 written out by hand: 1 + 2*8 + 3*64 + 4*512
    + 5*4096 + 6*32768 + 7*262144 = 0x1F58D1, little-endian bytes D1 58 1F;
    as INT3 they read 1, 2, 3, -4, -3, -2, -1, 0."""
    from oracle.formats import decode_weight_codes
    row = np.array([[0xD1, 0x58, 0x1F]], np.uint8)
    assert decode_weight_codes(row, "uint3")[0].tolist() == [1, 2, 3, 4, 5, 6, 7, 0]
    assert decode_weight_codes(row, "int3")[0].tolist() == [1, 2, 3, -4, -3, -2, -1, 0]
    assert np.array_equal(pack_bits(np.array([[1, 2, 3, 4, 5, 6, 7, 0]], np.uint8), 3), row)


@pytest.mark.parametrize("wd,vals", [("int1", [0, -1]), ("int2", [0, 1, -2, -1]),
                                     ("int3", [0, 1, 2, 3, -4, -3, -2, -1]),
                                     ("uint2", [0, 1, 2, 3]), ("uint1", [0, 1])])
def test_low_bit_integer_value_sets(wd, vals):
    """Every code of a b-bit integer format, one per element of an 8-code
    row: the values are the two's complement (or unsigned) range."""
    from oracle.formats import decode_weight_codes
    b = BITS[wd]
    codes = np.array([list(range(1 << b)) * (8 // (1 << b)) if (1 << b) <= 8 else list(range(8))], np.uint8)
    got = decode_weight_codes(pack_bits(codes, b), wd)[0]
    assert got.tolist() == (vals * (8 // len(vals)))


@pytest.mark.parametrize("wd", ["uint1", "uint2", "uint3"])
def test_low_bit_codes_equal_zero_point_give_zero(wd):
    g = np.random.default_rng(24)
    b = BITS[wd]
    n, k, gs = 8, 256, 64
    z = g.integers(0, 1 << b, size=(1, n, k // gs)).astype(np.uint8)
    cu = np.repeat(z, gs, axis=2)
    sc = bf16_bits(g.uniform(0.005, 0.02, size=(1, n, k // gs)).astype(np.float32))
    a = decode_bf16(bf16_bits(g.standard_normal((3, k)).astype(np.float32)))
    d = G.WeightDesc(wd, "group", gs, "bf16", True, False, 1, n, k)
    assert np.all(G.linear(d, a, pack_bits(cu, b), sc, z) == 0)


@pytest.mark.parametrize("wd", ["e2m3", "e3m2"])
def test_fp6_values_match_ocp_table(wd):
    """Every FP6 code against the OCP MX v1.0 value table (golden file), both
    signs, through the canonical 6-bit stream."""
    import os
    from oracle.formats import decode_weight_codes
    path = os.path.join(os.path.dirname(__file__), "golden", f"{wd}_values.txt")
    table = {}
    for ln in open(path):
        if ln.startswith("#") or not ln.strip():
            continue
        c, v = ln.split()
        table[int(c, 16)] = float(v)
    assert len(table) == 32
    codes = np.arange(64, dtype=np.uint8)[None, :]
    got = decode_weight_codes(pack_bits(codes, 6), wd)[0]
    for c in range(64):
        want = table[c & 31] * (-1.0 if c & 32 else 1.0)
        assert got[c] == want and np.signbit(got[c]) == bool(c & 32), (c, got[c], want)
    assert got.max() == (7.5 if wd == "e2m3" else 28.0)
