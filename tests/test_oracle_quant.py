"""Pins of the oracle's activation quantizers: closed-form properties,
representable round trips and an independent scalar re-derivation that uses
Python's math.frexp and Fractions instead of the vectorised code."""
import math
from fractions import Fraction

import numpy as np

from oracle import formats as F
from oracle import quant as Q
from synth import bf16_bits


def _bf16_vals(g, shape, scale=1.0):
    return F.decode_bf16(bf16_bits((g.standard_normal(shape) * scale).astype(np.float32))).astype(np.float32)


def test_fp8_token_amax_maps_to_448():
    g = np.random.default_rng(10)
    x = _bf16_vals(g, (64, 256))
    q, s = Q.quant_fp8_per_token(x)
    am = np.abs(x).argmax(axis=1)
    top = q[np.arange(64), am]
    sign = np.signbit(x[np.arange(64), am])
    assert np.all(top == np.where(sign, 0xFE, 0x7E))
    assert s.dtype == np.float32
    # fl32(amax / 448) written with Fractions
    for i in range(64):
        amax = Fraction(float(np.abs(x[i]).max()))
        ref = np.float32(float(amax / 448))
        assert s[i] == ref


def test_fp8_token_zero_row_and_signed_zero():
    x = np.zeros((2, 64), np.float32)
    x[1, 3] = -0.0
    q, s = Q.quant_fp8_per_token(x)
    assert s.tolist() == [1.0, 1.0]
    assert q[0].tolist() == [0] * 64
    assert q[1, 3] == 0x80


def test_fp8_token_representable_round_trip():
    g = np.random.default_rng(11)
    codes = g.integers(0, 0x7F, size=(32, 128)).astype(np.uint8)
    codes |= (g.integers(0, 2, size=codes.shape) << 7).astype(np.uint8)
    codes[:, 5] = 0x7E                       # row amax hits 448 exactly
    codes = np.where((codes & 0x7F) > 0x7E, 0x7E, codes).astype(np.uint8)
    s = np.ldexp(1.0, g.integers(-10, 4, size=32)).astype(np.float32)
    x = (F.decode_e4m3(codes) * s[:, None]).astype(np.float32)
    q, s2 = Q.quant_fp8_per_token(x)
    assert np.array_equal(s2, s)
    assert np.array_equal(q, codes)


def _mx_scalar(block):
    """Independent scalar statement of the MX scale rule."""
    amax = max(abs(float(v)) for v in block)
    if amax == 0:
        e = 127
    else:
        _, ex = math.frexp(amax)
        e = min(max((ex - 1) - 8 + 127, 0), 254)
    x_scale = Fraction(2) ** (e - 127)
    vals = F.decode_e4m3(np.arange(0x7F))
    out = []
    for v in block:
        t = Fraction(float(v)) / x_scale
        a = min(abs(t), Fraction(448))
        best = min(range(0x7F), key=lambda c: (abs(Fraction(vals[c]) - a), c & 1))
        code = best | (0x80 if (float(v) < 0 or (float(v) == 0 and math.copysign(1, float(v)) < 0)) else 0)
        out.append(code)
    return e, out


def test_mxfp8_matches_scalar_statement():
    g = np.random.default_rng(12)
    x = _bf16_vals(g, (4, 64), scale=3.0)
    x[1, :32] = 0.0
    x[2, 32:] *= 1e-30
    q, e = Q.quant_mxfp8(x)
    for r in range(4):
        for b in range(2):
            es, codes = _mx_scalar(x[r, 32 * b:32 * b + 32])
            assert e[r, b] == es
            assert q[r, 32 * b:32 * b + 32].tolist() == codes


def test_mxfp8_exponent_minimal():
    g = np.random.default_rng(13)
    x = _bf16_vals(g, (128, 256), scale=10.0)
    q, e = Q.quant_mxfp8(x)
    amax = np.abs(x.reshape(128, 8, 32)).max(axis=2).astype(np.float64)
    X = np.ldexp(1.0, e.astype(np.int64) - 127)
    assert np.all(amax / X < 512) and np.all(amax / (X / 2) >= 512)


def test_mxfp8_representable_round_trip():
    g = np.random.default_rng(14)
    codes = g.integers(0, 0x7E, size=(16, 128)).astype(np.uint8)
    codes |= (g.integers(0, 2, size=codes.shape) << 7).astype(np.uint8)
    codes[:, ::32] = 0x78 | g.integers(0, 7, size=(16, 4)).astype(np.uint8)  # 256..448
    e = g.integers(110, 140, size=(16, 4)).astype(np.uint8)
    x = Q.dequant_mxfp8(codes, e)
    q2, e2 = Q.quant_mxfp8(x)
    assert np.array_equal(e2, e) and np.array_equal(q2, codes)


def _mx4_scalar(block):
    """Independent scalar statement of the MX scale rule with E2M1 elements."""
    amax = max(abs(float(v)) for v in block)
    if amax == 0:
        e = 127
    else:
        _, ex = math.frexp(amax)
        e = min(max((ex - 1) - 2 + 127, 0), 254)
    x_scale = Fraction(2) ** (e - 127)
    vals = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    out = []
    for v in block:
        t = Fraction(float(v)) / x_scale
        a = min(abs(t), Fraction(6))
        best = min(range(8), key=lambda c: (abs(Fraction(vals[c]) - a), c & 1))
        code = best | (8 if (float(v) < 0 or (float(v) == 0 and math.copysign(1, float(v)) < 0)) else 0)
        out.append(code)
    return e, out


def test_mxfp4_matches_scalar_statement():
    g = np.random.default_rng(15)
    x = _bf16_vals(g, (4, 64), scale=3.0)
    x[1, :32] = 0.0
    x[2, 32:] *= 1e-30
    x[3, 7] = -0.0
    q, e = Q.quant_mxfp4(x)
    codes = F.unpack_nibbles(q)
    for r in range(4):
        for b in range(2):
            es, ref = _mx4_scalar(x[r, 32 * b:32 * b + 32])
            assert e[r, b] == es
            assert codes[r, 32 * b:32 * b + 32].tolist() == ref


def test_mxfp4_exponent_minimal():
    g = np.random.default_rng(16)
    x = _bf16_vals(g, (128, 256), scale=10.0)
    q, e = Q.quant_mxfp4(x)
    amax = np.abs(x.reshape(128, 8, 32)).max(axis=2).astype(np.float64)
    X = np.ldexp(1.0, e.astype(np.int64) - 127)
    assert np.all(amax / X < 8) and np.all(amax / (X / 2) >= 8)


def test_mxfp4_representable_round_trip():
    g = np.random.default_rng(17)
    codes = g.integers(0, 16, size=(16, 128)).astype(np.uint8)
    codes[:, ::32] = 6 | (g.integers(0, 2, size=(16, 4)) * 9).astype(np.uint8)  # +-4 or +-6 (amax in [4, 8))
    e = g.integers(110, 140, size=(16, 4)).astype(np.uint8)
    packed = F.pack_nibbles(codes)
    x = Q.dequant_mxfp4(packed, e)
    q2, e2 = Q.quant_mxfp4(x)
    assert np.array_equal(e2, e) and np.array_equal(q2, packed)



def test_fp8_group_amax_maps_to_448_per_group():
    g = np.random.default_rng(18)
    x = _bf16_vals(g, (16, 512))
    x[3, 128:256] = 0.0
    q, s = Q.quant_fp8_group(x)
    assert s.shape == (16, 4) and s.dtype == np.float32
    assert s[3, 1] == 1.0 and np.all(q[3, 128:256] == 0)
    for r in range(16):
        for b in range(4):
            blk = x[r, 128 * b:128 * b + 128]
            amax = Fraction(float(np.abs(blk).max()))
            if amax == 0:
                continue
            assert s[r, b] == np.float32(float(amax / 448))
            j = int(np.abs(blk).argmax())
            assert q[r, 128 * b + j] == (0xFE if blk[j] < 0 else 0x7E)


def test_fp8_group_equals_per_token_on_each_group():
    g = np.random.default_rng(19)
    x = _bf16_vals(g, (8, 384), scale=5.0)
    q, s = Q.quant_fp8_group(x)
    for b in range(3):
        qt, st = Q.quant_fp8_per_token(x[:, 128 * b:128 * b + 128])
        assert np.array_equal(q[:, 128 * b:128 * b + 128], qt) and np.array_equal(s[:, b], st)


def test_fp8_group_representable_round_trip():
    g = np.random.default_rng(20)
    codes = g.integers(0, 0x7F, size=(8, 256)).astype(np.uint8)
    codes |= (g.integers(0, 2, size=codes.shape) << 7).astype(np.uint8)
    codes = np.where((codes & 0x7F) > 0x7E, 0x7E, codes).astype(np.uint8)
    codes[:, 5] = 0x7E
    codes[:, 133] = 0xFE
    s = np.ldexp(1.0, g.integers(-10, 4, size=(8, 2))).astype(np.float32)
    x = Q.dequant_fp8_group(codes, s).astype(np.float32)
    q2, s2 = Q.quant_fp8_group(x)
    assert np.array_equal(s2, s) and np.array_equal(q2, codes)
