"""Oracle number formats (TEST INFRASTRUCTURE ONLY).

The pages name the formats (INT4/UINT4, MXFP4 = E2M1 elements with E8M0
block scales, FP8 E4M3, BF16) in "Announcing Humming: Fast, Flexible Kernels
for Quantized Inference", sections "Background" and "WnA16"; they never give
bit layouts.  The readings below are the OCP definitions:

* INT4: two's complement nibble, values -8..7.  UINT4: 0..15.
* INTb / UINTb for b = 1, 2, 3 (section "WnA16" lists INT1, INT2 and INT3
  among the shared dequantization path's widths; section "Quantization
  support" of the aireiter.com review names GPTQ INT3 checkpoints): the
  same two's complement / unsigned reading at b bits (INT3 -4..3, INT2
  -2..1, INT1 -1..0; UINTb 0..2^b-1).  Canonical packing is an LSB-first
  bit stream along K: code k of a row occupies bits b*k .. b*k+b-1 of the
  row's bytes read as one little-endian integer (for b = 4 this is the
  nibble packing, even k in the low nibble; for b = 3 it is the GPTQ
  3-bit stream, whose 32-bit words, little-endian, hold the same bits).
* INT8: two's complement byte, values -128..127 (one code per byte; the
  pages list INT8 among the weight widths without a layout).
* E2M1 (OCP MX v1.0): sign, 2 exponent bits (bias 1), 1 mantissa bit;
  magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}; no Inf/NaN.
* E4M3 "FN" (OCP FP8): sign, 4 exponent bits (bias 7), 3 mantissa bits;
  exponent field 0 is subnormal with quantum 2^-9; codes 0x7F/0xFF are NaN;
  no Inf; largest finite 448.
* E8M0 (OCP MX v1.0): 2^(c-127); c = 255 is NaN.
* FP6 E2M3 / E3M2 (OCP MX v1.0; the WnA16 section of the announcement runs
  FP4 to FP8 weights): sign, 2 (3) exponent bits with bias 1 (3), 3 (2)
  mantissa bits; exponent 0 is subnormal (quantum 2^-3 / 2^-4); no Inf/NaN;
  max 7.5 / 28.  Canonical packing: the LSB-first 6-bit stream along K
  (codes [E][N][K*6/8]), with an E8M0 scale per 32 along K (MXFP6).
* BF16: the upper 16 bits of an IEEE float32.

Encoders round to nearest, ties to even, and saturate (E4M3, E2M1) where
noted.
All values are returned as float64.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def decode_int4(c):
    c = np.asarray(c, dtype=np.int64) & 0xF
    return np.where(c >= 8, c - 16, c).astype(np.float64)


def decode_int8(c):
    c = np.asarray(c, dtype=np.int64) & 0xFF
    return np.where(c >= 128, c - 256, c).astype(np.float64)


def decode_uint4(c):
    return (np.asarray(c, dtype=np.int64) & 0xF).astype(np.float64)


def _e2m1_closed_form(c):
    c = np.asarray(c, dtype=np.int64) & 0xF
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return np.where(s == 1, -mag, mag).astype(np.float64)


def _e4m3_closed_form(c):
    c = np.asarray(c, dtype=np.int64) & 0xFF
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag).astype(np.float64)


# The closed forms above evaluated once per code; decoding a tensor looks
# its codes up (the same values, without re-evaluating the closed form per
# element).
_E2M1_VALUES = _e2m1_closed_form(np.arange(16))
_E4M3_VALUES = _e4m3_closed_form(np.arange(256))


def _code_index(c, mask):
    c = np.asarray(c)
    return (c & mask) if c.dtype == np.uint8 else (c.astype(np.int64) & mask)


def decode_e2m1(c):
    return np.take(_E2M1_VALUES, _code_index(c, 0xF))


def decode_e4m3(c):
    return np.take(_E4M3_VALUES, _code_index(c, 0xFF))


def decode_e8m0(c):
    c = np.asarray(c, dtype=np.int64) & 0xFF
    v = np.ldexp(1.0, c - 127)
    return np.where(c == 255, np.nan, v).astype(np.float64)


def decode_bf16(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def decode_f32(x):
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def _rne(x):
    # NumPy's round() is round-half-to-even.
    return np.round(x)


def encode_bf16(x):
    """float64 values -> bf16 bit patterns, one RNE rounding of the exact
    value (8 significant bits, subnormal quantum 2^-133)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)                      # a = f * 2^e, f in [0.5, 1)
    e = np.where(a == 0, -200, e)
    q_exp = np.maximum(e - 8, -133)          # quantum exponent
    r = np.ldexp(_rne(np.ldexp(a, -q_exp)), q_exp)
    r = np.where(r > 3.3895313892515355e38, np.inf, r)
    r = np.where(np.isnan(a), np.nan, r)
    r = np.copysign(r, x)
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def round_e4m3(v):
    """float64 -> nearest E4M3 value (RNE), saturated to +-448, signed zero
    kept.  Returns float64 values that are exactly representable."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, e = np.frexp(a)                      # a in [2^(e-1), 2^e)
    e = np.where(a == 0, -200, e)
    q_exp = np.maximum(e - 4, -9)            # 3 mantissa bits, subnormal 2^-9
    r = np.ldexp(_rne(np.ldexp(a, -q_exp)), q_exp)
    r = np.minimum(r, E4M3_MAX)
    return np.copysign(r, v)


def encode_e4m3(v):
    """float64 -> E4M3 code (uint8), RNE with saturation to +-448."""
    r = round_e4m3(v)
    sign = np.signbit(r).astype(np.int64)
    a = np.abs(r)
    _, e = np.frexp(a)
    ub = e - 1                               # unbiased exponent of a normal
    normal = a >= 2.0 ** -6
    exp_field = np.where(normal, ub + 7, 0)
    man = np.where(normal, np.ldexp(a, -ub) * 8.0 - 8.0, np.ldexp(a, 9))
    man = np.where(a == 0, 0, man)
    exp_field = np.where(a == 0, 0, exp_field)
    code = (sign << 7) | (exp_field.astype(np.int64) << 3) | man.astype(np.int64)
    return code.astype(np.uint8)


E2M1_MAX = 6.0
E2M1_VALUES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def round_e2m1(v):
    """float64 -> nearest E2M1 value (RNE on the one mantissa bit; quantum
    0.5 below 2, 1 in [2, 4), 2 from 4), saturated to +-6, signed zero
    kept.  Returns float64 values that are exactly representable."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, e = np.frexp(a)                      # a in [2^(e-1), 2^e)
    e = np.where(a == 0, -200, e)
    q_exp = np.maximum(e - 2, -1)            # 1 mantissa bit, subnormal quantum 2^-1
    r = np.ldexp(_rne(np.ldexp(a, -q_exp)), q_exp)
    r = np.minimum(r, E2M1_MAX)
    return np.copysign(r, v)


def encode_e2m1(v):
    """float64 -> E2M1 code (uint8, one code per byte), RNE with saturation
    to +-6; the sign bit follows the sign of the (rounded) value."""
    r = round_e2m1(v)
    sign = np.signbit(r).astype(np.int64)
    idx = np.searchsorted(np.asarray(E2M1_VALUES), np.abs(r))
    return ((sign << 3) | idx).astype(np.uint8)


def pack_nibbles(codes):
    """uint8 [..., K] (one 4-bit code each) -> uint8 [..., K/2]; even k in
    the low nibble (the inverse of unpack_nibbles)."""
    c = np.asarray(codes, dtype=np.uint8) & 0xF
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def floor_log2(a):
    """Exact floor(log2 a) for finite a > 0, read from the exponent field."""
    _, e = np.frexp(np.asarray(a, dtype=np.float64))
    return e - 1


def decode_scale(scales, dtype: str):
    if dtype == "bf16":
        return decode_bf16(scales)
    if dtype == "f32":
        return decode_f32(scales)
    if dtype == "e8m0":
        return decode_e8m0(scales)
    if dtype == "e4m3":
        # NVFP4's group scales are E4M3 codes
        return decode_e4m3(scales)
    raise ValueError(f"unknown scale dtype {dtype}")


def unpack_nibbles(packed):
    """uint8 [..., K/2] -> uint8 [..., K]; even k from the low nibble."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def _decode_minifloat(c, ebits: int, mbits: int, bias: int):
    """Sign / exponent / mantissa fields -> value; exponent 0 is subnormal."""
    c = np.asarray(c, dtype=np.int64)
    s = (c >> (ebits + mbits)) & 1
    e = (c >> mbits) & ((1 << ebits) - 1)
    m = c & ((1 << mbits) - 1)
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), 1 - bias - mbits),
                   np.ldexp(1.0 + np.ldexp(m.astype(np.float64), -mbits), e - bias))
    return np.where(s == 1, -mag, mag).astype(np.float64)


def decode_e2m3(c):
    return _decode_minifloat(c, 2, 3, 1)


def decode_e3m2(c):
    return _decode_minifloat(c, 3, 2, 3)


INT_BITS = {"int1": 1, "int2": 2, "int3": 3, "uint1": 1, "uint2": 2, "uint3": 3}


def unpack_bits(packed, bits: int):
    """uint8 [..., K*bits/8] LSB-first bit stream -> uint8 [..., K] codes.

    Bit i of the row is bit (i % 8) of byte i // 8; code k is the bits
    bits*k .. bits*k + bits - 1, least significant first."""
    p = np.asarray(packed, dtype=np.uint8)
    stream = np.unpackbits(p, axis=-1, bitorder="little")          # [..., 8 * bytes]
    k = stream.shape[-1] // bits
    b = stream[..., :k * bits].reshape(p.shape[:-1] + (k, bits)).astype(np.int64)
    weights = np.left_shift(1, np.arange(bits, dtype=np.int64))
    return (b * weights).sum(axis=-1).astype(np.uint8)


def decode_intb(c, bits: int):
    """b-bit two's complement code -> value in [-2^(b-1), 2^(b-1) - 1]."""
    c = np.asarray(c, dtype=np.int64) & ((1 << bits) - 1)
    return np.where(c >= (1 << (bits - 1)), c - (1 << bits), c).astype(np.float64)


def decode_weight_codes(codes, weight_dtype: str):
    """Canonical code array -> float64 element values v(q)."""
    if weight_dtype in ("e2m3", "e3m2"):
        q = unpack_bits(codes, 6)
        return decode_e2m3(q) if weight_dtype == "e2m3" else decode_e3m2(q)
    if weight_dtype in INT_BITS:
        b = INT_BITS[weight_dtype]
        q = unpack_bits(codes, b)
        if weight_dtype.startswith("u"):
            return q.astype(np.float64)
        return decode_intb(q, b)
    if weight_dtype in ("int4", "uint4", "e2m1"):
        q = unpack_nibbles(codes)
        return {"int4": decode_int4, "uint4": decode_uint4,
                "e2m1": decode_e2m1}[weight_dtype](q)
    if weight_dtype == "e4m3":
        return decode_e4m3(codes)
    if weight_dtype == "int8":
        return decode_int8(codes)
    raise ValueError(f"unknown weight dtype {weight_dtype}")
