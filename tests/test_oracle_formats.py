"""Pins of the oracle's number formats against things other than itself:
published format tables (tests/golden), PyTorch's own dtype conversions,
two's-complement arithmetic and brute-force nearest-value search."""
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#")[0].strip()
            if not line:
                continue
            c, v = line.split()
            out[int(c, 16)] = float(v)
    return out


def test_int4_two_complement():
    c = np.arange(16, dtype=np.uint8)
    ref = ((c.astype(np.int8) << 4).astype(np.int8) >> 4).astype(np.float64)
    assert np.array_equal(F.decode_int4(c), ref)
    assert np.array_equal(F.decode_uint4(c), c.astype(np.float64))


def test_int8_two_complement():
    c = np.arange(256, dtype=np.uint8)
    v = F.decode_int8(c)
    assert np.array_equal(v, c.view(np.int8).astype(np.float64))
    assert v.min() == -128 and v.max() == 127 and v[0x80] == -128 and v[0xFF] == -1
    assert np.array_equal(F.decode_weight_codes(c.reshape(1, 2, 128), "int8").ravel(), v)


def test_e2m1_golden_table():
    tab = _read_table("e2m1_values.txt")
    got = F.decode_e2m1(np.arange(16))
    for c in range(16):
        assert got[c] == tab[c]
        assert math.copysign(1, got[c]) == math.copysign(1, tab[c])


def test_e4m3_all_codes_vs_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    got = F.decode_e4m3(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert nan.sum() == 2
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))


def test_e4m3_golden_specials():
    tab = _read_table("e4m3_special.txt")
    got = F.decode_e4m3(np.arange(256))
    for c, v in tab.items():
        if math.isnan(v):
            assert math.isnan(got[c])
        else:
            assert got[c] == v and math.copysign(1, got[c]) == math.copysign(1, v)


def test_e8m0_closed_form():
    got = F.decode_e8m0(np.arange(256))
    for c in range(255):
        assert got[c] == math.ldexp(1.0, c - 127)
    assert math.isnan(got[255])


def test_bf16_decode_all_patterns_vs_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    got = F.decode_bf16(bits)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan].astype(np.float64), got[~nan])


def test_bf16_encode_vs_torch_on_float32():
    g = np.random.default_rng(1)
    x = np.concatenate([
        g.standard_normal(20000).astype(np.float32),
        (g.standard_normal(2000) * 1e-39).astype(np.float32),   # subnormals
        (g.standard_normal(2000) * 3e38).astype(np.float32),    # near overflow
        # exact ties: bf16 value + half an ulp
        ((np.arange(1, 2001, dtype=np.uint32) << 16) | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0], dtype=np.float32),
    ])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = F.encode_bf16(x.astype(np.float64))
    assert np.array_equal(ref, got)


def _nearest_brute(v, table_vals, table_codes, maxv):
    """Nearest representable value by exhaustive search; ties -> even code."""
    a = min(abs(Fraction(v)), Fraction(maxv))
    best = None
    for val, code in zip(table_vals, table_codes):
        d = abs(Fraction(val) - a)
        key = (d, code & 1)
        if best is None or key < best[0]:
            best = (key, val)
    return math.copysign(best[1], v)


def test_e4m3_round_brute_force():
    codes = np.arange(0x7F)                       # non-negative finite codes
    vals = F.decode_e4m3(codes)
    g = np.random.default_rng(2)
    xs = np.concatenate([g.standard_normal(300) * 50, g.standard_normal(200) * 0.01,
                         g.uniform(-600, 600, 100),
                         # exact midpoints between neighbours
                         (vals[1:] + vals[:-1]) / 2, -(vals[1:] + vals[:-1]) / 2])
    got = F.round_e4m3(xs)
    for x, r in zip(xs, got):
        ref = _nearest_brute(float(x), vals.tolist(), codes.tolist(), 448.0)
        assert r == ref, (x, r, ref)


def test_e4m3_encode_vs_torch_on_clamped_float32():
    g = np.random.default_rng(3)
    x = np.concatenate([g.standard_normal(50000) * 30, g.standard_normal(5000) * 1e-3]).astype(np.float32)
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.encode_e4m3(x.astype(np.float64))
    assert np.array_equal(ref, got)


def test_e4m3_encode_saturates_and_keeps_signed_zero():
    got = F.encode_e4m3(np.array([1e9, -1e9, 449.0, 470.0, -0.0, -1e-9, 1e-9]))
    assert got.tolist() == [0x7E, 0xFE, 0x7E, 0x7E, 0x80, 0x80, 0x00]


def test_e4m3_round_trip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    assert np.array_equal(F.encode_e4m3(F.decode_e4m3(codes)), codes.astype(np.uint8))


def test_floor_log2_exact_at_powers_of_two():
    for e in range(-140, 128):
        v = math.ldexp(1.0, e)
        assert F.floor_log2(v) == e
        assert F.floor_log2(math.nextafter(v, 0)) == e - 1 or v == 5e-324


def test_unpack_nibbles_order():
    p = np.array([[0x21, 0xF0]], dtype=np.uint8)
    assert F.unpack_nibbles(p).tolist() == [[1, 2, 0, 15]]


def test_bf16_encode_float64_brute():
    # Values not representable in float32: compare with an exact search over
    # the two neighbouring bf16 values.
    g = np.random.default_rng(4)
    xs = g.standard_normal(500) * np.exp(g.uniform(-20, 20, 500))
    got = F.decode_bf16(F.encode_bf16(xs))
    for x, r in zip(xs, got):
        bits = struct.unpack("<I", struct.pack("<f", np.float32(x)))[0] >> 16
        cands = set()
        for b in (bits - 1, bits, bits + 1):
            cands.add(struct.unpack("<f", struct.pack("<I", (b & 0xFFFF) << 16))[0])
        cands = sorted(cands, key=lambda c: (abs(Fraction(c) - Fraction(float(x))),
                                              (struct.unpack("<I", struct.pack("<f", c))[0] >> 16) & 1))
        assert r == cands[0], (x, r, cands)


def test_e2m1_round_brute_force():
    codes = np.arange(8)                          # non-negative codes
    vals = F.decode_e2m1(codes)
    g = np.random.default_rng(5)
    xs = np.concatenate([g.standard_normal(300) * 3, g.uniform(-9, 9, 200), g.standard_normal(50) * 0.2,
                         # exact midpoints between neighbours, both signs
                         (vals[1:] + vals[:-1]) / 2, -(vals[1:] + vals[:-1]) / 2])
    got = F.round_e2m1(xs)
    for x, r in zip(xs, got):
        ref = _nearest_brute(float(x), vals.tolist(), codes.tolist(), 6.0)
        assert r == ref, (x, r, ref)


def test_e2m1_encode_round_trip_and_signed_zero():
    codes = np.arange(16, dtype=np.uint8)
    assert np.array_equal(F.encode_e2m1(F.decode_e2m1(codes)), codes)
    assert F.encode_e2m1(np.array([-0.0, -0.2, 0.2, 100.0, -100.0])).tolist() == [8, 8, 0, 7, 15]


def test_pack_nibbles_inverts_unpack():
    g = np.random.default_rng(6)
    p = g.integers(0, 256, size=(5, 12)).astype(np.uint8)
    assert np.array_equal(F.pack_nibbles(F.unpack_nibbles(p)), p)
