"""Oracle activation quantizers (TEST INFRASTRUCTURE ONLY).

The pages use two dynamic activation formats: "tokenwise FP8" for the
W4A8 serving test ("Announcing Humming: Fast, Flexible Kernels for Quantized
Inference", section "End-to-end inference performance") and MXFP8 (section
"Choosing the activation type"; group-32 MXFP8 activations in the "H100,
W4A8 and group-32" section of the aireiter.com review).  They give no
scaling rule; the readings taken here are:

* per-token FP8: s_m = fl32(amax_m / 448) (1.0 for an all-zero row),
  q = E4M3_RNE_SAT(fl32(x / s_m)), an IEEE float32 division by the stored
  scale.
* MXFP8 (OCP MX v1.0 scale rule): per block of 32 along K,
  E = clamp(floor(log2 amax) - 8 + 127, 0, 254) (8 = emax of E4M3), an
  all-zero block takes E = 127; X = 2^(E-127); q = E4M3_RNE_SAT(x / X).
  floor(log2) is read from the exponent field, never from a rounded log.
* per-token-group FP8 (the activations of block-scaled FP8 W8A8, section
  "W8A8 / W4A8 / W4A4"; groups of 128 along K, the page gives no shape):
  the per-token rule applied to each group of 128: s = fl32(amax / 448)
  (1.0 for an all-zero group), q = E4M3_RNE_SAT(fl32(x / s)).
* MXFP4 activations (the W4A4 = MXFP4 x MXFP4 combination of the section
  "W8A8 / W4A8 / W4A4"): the same OCP rule with the emax of E2M1 (2):
  E = clamp(floor(log2 amax) - 2 + 127, 0, 254), an all-zero block takes
  E = 127; q = E2M1_RNE_SAT(x / X).  A block's largest element lands in
  [4, 8) before rounding and saturates to 6 above 6 (the OCP rule's own
  clipping).
"""
from __future__ import annotations

import numpy as np

from .formats import (decode_e2m1, decode_e4m3, decode_e8m0, encode_e2m1, encode_e4m3, floor_log2, pack_nibbles,
                      unpack_nibbles)


def quant_fp8_per_token(x_f32):
    """x: float32 [M, K] (bf16 values widened) -> (codes uint8 [M,K], scale f32 [M])."""
    x = np.asarray(x_f32, dtype=np.float32)
    amax = np.abs(x).max(axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    r = (x / s[:, None]).astype(np.float32)          # IEEE fp32 division
    return encode_e4m3(r.astype(np.float64)), s


def dequant_fp8_per_token(codes, s):
    return decode_e4m3(codes) * np.asarray(s, np.float32).astype(np.float64)[:, None]


def mxfp8_exponent(amax):
    amax = np.asarray(amax, dtype=np.float64)
    safe = np.where(amax > 0, amax, 1.0)
    e = np.clip(floor_log2(safe) - 8 + 127, 0, 254)
    return np.where(amax > 0, e, 127).astype(np.int64)


def quant_mxfp8(x):
    """x: [M, K] (any float dtype; taken as exact float64), K % 32 == 0
    -> (codes uint8 [M, K], E8M0 codes uint8 [M, K/32])."""
    x = np.asarray(x, dtype=np.float64)
    m, k = x.shape
    assert k % 32 == 0
    xb = x.reshape(m, k // 32, 32)
    e = mxfp8_exponent(np.abs(xb).max(axis=2))
    scaled = xb / np.ldexp(1.0, e - 127)[..., None]
    return encode_e4m3(scaled).reshape(m, k), e.astype(np.uint8)


def dequant_mxfp8(codes, e8m0):
    m, k = codes.shape
    v = decode_e4m3(codes).reshape(m, k // 32, 32)
    return (v * decode_e8m0(e8m0)[..., None]).reshape(m, k)


def mxfp4_exponent(amax):
    amax = np.asarray(amax, dtype=np.float64)
    safe = np.where(amax > 0, amax, 1.0)
    e = np.clip(floor_log2(safe) - 2 + 127, 0, 254)
    return np.where(amax > 0, e, 127).astype(np.int64)


def quant_mxfp4(x):
    """x: [M, K] (any float dtype; taken as exact float64), K % 32 == 0
    -> (packed codes uint8 [M, K/2], even k in the low nibble;
        E8M0 codes uint8 [M, K/32])."""
    x = np.asarray(x, dtype=np.float64)
    m, k = x.shape
    assert k % 32 == 0
    xb = x.reshape(m, k // 32, 32)
    e = mxfp4_exponent(np.abs(xb).max(axis=2))
    scaled = xb / np.ldexp(1.0, e - 127)[..., None]
    return pack_nibbles(encode_e2m1(scaled).reshape(m, k)), e.astype(np.uint8)


def dequant_mxfp4(packed, e8m0):
    m = packed.shape[0]
    v = decode_e2m1(unpack_nibbles(packed))
    k = v.shape[1]
    return (v.reshape(m, k // 32, 32) * decode_e8m0(e8m0)[..., None]).reshape(m, k)


def quant_fp8_group(x_f32, group: int = 128):
    """x: float32 [M, K] (bf16 values widened), K % group == 0
    -> (codes uint8 [M, K], scales f32 [M, K/group])."""
    x = np.asarray(x_f32, dtype=np.float32)
    m, k = x.shape
    assert k % group == 0
    xg = x.reshape(m, k // group, group)
    amax = np.abs(xg).max(axis=2) if k else np.zeros((m, 0), np.float32)
    s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    r = (xg / s[..., None]).astype(np.float32)         # IEEE fp32 division
    return encode_e4m3(r.astype(np.float64)).reshape(m, k), s


def dequant_fp8_group(codes, s, group: int = 128):
    m, k = codes.shape
    v = decode_e4m3(codes).reshape(m, k // group, group)
    return (v * np.asarray(s, np.float32).astype(np.float64)[..., None]).reshape(m, k)
