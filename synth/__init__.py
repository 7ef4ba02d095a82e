"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws random numbers and lays them out in the canonical
("standard format") host layout that both the CPU oracle and the GPU library
consume.  It holds none of the method's arithmetic: no dequantization, no
GEMM, no activation quantizer, no routing sort.  Where an input has to be
rounded to a storage type (bf16 activations, FP8 weights of the W8A8 case)
the rounding is done by PyTorch's own dtype conversion, which is a library
routine and not part of what is being tested.

Canonical host layout (every array is a NumPy array on the host):

* 4-bit codes: ``uint8 [E][N][K/2]``, two codes per byte, the even k in the
  low nibble.  8-bit codes: ``uint8 [E][N][K]``.
* scales: ``[E][N][K/G]``; bf16 as ``uint16`` bit patterns, f32 as
  ``float32``, E8M0 as ``uint8`` exponent codes.
* zero points: ``uint8 [E][N][K/G]`` holding uint4 values (0..15).
* second-level (global) scale: ``float32 [E]``.
* bf16 activations: ``uint16 [M][K]`` bit patterns.

The weight formats, scale granularities and zero points follow the
quantization description of "Announcing Humming: Fast, Flexible Kernels for
Quantized Inference", section "Unified quantization representation"; the
workload shapes and value distributions are those of the dense W4A16, dense
W8A8 and MoE W4A16 / W4A8 workloads measured in that post's "Performance"
section, with the sizes fixed here.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "rng", "seed_for", "seed_of", "bf16_bits", "bf16_normal", "pack_nibbles", "pack_bits", "INT_BITS",
    "dense_w4a16", "dense_w8a8", "moe_weights_mxfp4", "routing", "quant_weights",
    "DENSE_SWEEP_M", "FP8_SWEEP_M", "MOE_W4A16_T", "MOE_W4A8_T",
]

DENSE_SWEEP_M = (1, 4, 16, 64, 256, 1024, 4096)
FP8_SWEEP_M = (1, 16, 128, 1024, 4096)
MOE_W4A16_T = (1, 16, 64, 512, 4096)
MOE_W4A8_T = (1, 64, 1024, 8192)


def seed_of(*parts) -> int:
    """A stable 16-bit seed from any printable values (CRC-32 of their repr;
    unlike hash(), the same in every process)."""
    import zlib
    return zlib.crc32(repr(parts).encode()) & 0xFFFF


def seed_for(config: int, index: int = 0) -> int:
    """Seed convention: 1000 * workload number + sweep index."""
    return 1000 * int(config) + int(index)


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(int(seed)))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16), rounded by torch."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_normal(g: np.random.Generator, shape) -> np.ndarray:
    """bf16 ~ N(0,1): float32 normal draws rounded to bf16."""
    return bf16_bits(g.standard_normal(shape, dtype=np.float32))


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """uint8 codes (0..15) [..., K] -> uint8 [..., K/2], even k in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    assert c.shape[-1] % 2 == 0
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


INT_BITS = {"int1": 1, "int2": 2, "int3": 3, "uint1": 1, "uint2": 2, "uint3": 3}


def pack_bits(codes: np.ndarray, bits: int) -> np.ndarray:
    """uint8 codes (0 .. 2^bits - 1) [..., K] -> uint8 [..., K*bits/8]: an
    LSB-first bit stream along K (code k at bits bits*k .. bits*k+bits-1 of
    the row read as one little-endian integer)."""
    c = np.asarray(codes, dtype=np.uint8)
    assert (c.shape[-1] * bits) % 8 == 0
    planes = [(c >> i) & 1 for i in range(bits)]                   # bit i of every code
    stream = np.stack(planes, axis=-1).reshape(c.shape[:-1] + (c.shape[-1] * bits,))
    return np.packbits(stream, axis=-1, bitorder="little")


def _uniform_bf16(g, lo, hi, shape):
    return bf16_bits(g.uniform(lo, hi, size=shape).astype(np.float32))


def dense_w4a16(seed: int, m: int, n: int, k: int, group: int = 128,
                asym: bool = False, num_experts: int = 1,
                scale_lo: float = 0.005, scale_hi: float = 0.02,
                zero_lo: int = 6, zero_hi: int = 9):
    """Group-quantized 4-bit weights with bf16 scales and bf16 activations.

    ``asym=False``: signed INT4 codes uniform in [-8, 7] (two's complement
    nibbles), no zero point.  ``asym=True``: UINT4 codes uniform in [0, 15]
    with uint4 zero points uniform in [zero_lo, zero_hi] per group.
    """
    g = rng(seed)
    e = num_experts
    kg = k // group
    if asym:
        codes = g.integers(0, 16, size=(e, n, k), dtype=np.uint8)
        zeros = g.integers(zero_lo, zero_hi + 1, size=(e, n, kg), dtype=np.uint8)
    else:
        v = g.integers(-8, 8, size=(e, n, k), dtype=np.int8)
        codes = (v & 0xF).astype(np.uint8)
        zeros = None
    scales = _uniform_bf16(g, scale_lo, scale_hi, (e, n, kg))
    x = bf16_normal(g, (m, k))
    return {
        "codes": pack_nibbles(codes),
        "scales": scales,
        "zeros": zeros,
        "x": x,
        "m": m, "n": n, "k": k, "group": group, "num_experts": e,
        "weight_dtype": "uint4" if asym else "int4",
    }


def quant_weights(seed: int, weight_dtype: str, scale_gran: str, group: int,
                  scale_dtype: str, num_experts: int, n: int, k: int,
                  zero: bool = False, global_scale: bool = False,
                  scale_lo: float = 0.005, scale_hi: float = 0.02,
                  e8m0_lo: int = 119, e8m0_hi: int = 123,
                  e4m3_lo: int = 0x18, e4m3_hi: int = 0x38):
    """Random canonical weights of any supported description: codes uniform
    over the format's codes (E4M3 without its NaN codes; INT8 one byte per
    code, all 256), scales uniform in
    [scale_lo, scale_hi] (bf16 / f32) or E8M0 codes in [e8m0_lo, e8m0_hi],
    E4M3 scale codes (NVFP4) uniform in [e4m3_lo, e4m3_hi] (positive, finite),
    zero points uniform over the codes (0..2^b-1), global scales uniform in [0.5, 2]."""
    g = rng(seed)
    e = num_experts
    if scale_gran == "group":
        sn, sg = n, k // group
    elif scale_gran == "block":
        sn, sg = -(-n // group), k // group
    elif scale_gran == "channel":
        sn, sg = n, 1
    else:
        sn, sg = 1, 1
    if weight_dtype == "e4m3":
        c = g.integers(0, 256, size=(e, n, k), dtype=np.uint8)
        codes = np.where((c & 0x7F) == 0x7F, c & 0xFE, c).astype(np.uint8)
    elif weight_dtype == "int8":
        codes = g.integers(0, 256, size=(e, n, k), dtype=np.uint8)
    elif weight_dtype in INT_BITS:
        b = INT_BITS[weight_dtype]
        codes = pack_bits(g.integers(0, 1 << b, size=(e, n, k), dtype=np.uint8), b)
    elif weight_dtype in ("e2m3", "e3m2"):
        codes = pack_bits(g.integers(0, 64, size=(e, n, k), dtype=np.uint8), 6)
    else:
        codes = pack_nibbles(g.integers(0, 16, size=(e, n, k), dtype=np.uint8))
    if scale_dtype == "bf16":
        scales = _uniform_bf16(g, scale_lo, scale_hi, (e, sn, sg))
    elif scale_dtype == "f32":
        scales = g.uniform(scale_lo, scale_hi, size=(e, sn, sg)).astype(np.float32)
    elif scale_dtype == "e4m3":
        scales = g.integers(e4m3_lo, e4m3_hi + 1, size=(e, sn, sg), dtype=np.uint8)
    else:
        scales = g.integers(e8m0_lo, e8m0_hi + 1, size=(e, sn, sg), dtype=np.uint8)
    zmax = 1 << INT_BITS.get(weight_dtype, 4)
    zeros = g.integers(0, zmax, size=(e, sn, sg), dtype=np.uint8) if zero else None
    gsc = g.uniform(0.5, 2.0, size=e).astype(np.float32) if global_scale else None
    return {"codes": codes, "scales": scales, "zeros": zeros, "global_scale": gsc}


def dense_w8a8(seed: int, m: int, n: int, k: int, w_std: float = 0.05):
    """FP8 E4M3 weights with one fp32 scale per output channel.

    Weights are drawn as N(0,1) * w_std in float32, the per-channel scale is
    amax_n / 448 in float32 and the codes are torch's float8_e4m3fn
    conversion of w / scale (clamped to the finite range first).
    Activations are bf16 ~ N(0,1); they are quantized per token on the GPU.
    """
    import torch
    g = rng(seed)
    w = (g.standard_normal((n, k), dtype=np.float32) * np.float32(w_std)).astype(np.float32)
    amax = np.abs(w).max(axis=1).astype(np.float32)
    s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    r = np.clip(w / s[:, None], -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(r).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    x = bf16_normal(g, (m, k))
    return {
        "codes": codes.reshape(1, n, k), "scales": s.reshape(1, n, 1),
        "zeros": None, "x": x, "m": m, "n": n, "k": k, "group": k,
        "num_experts": 1, "weight_dtype": "e4m3",
    }


def moe_weights_mxfp4(seed: int, num_experts: int, n: int, k: int,
                      exp_lo: int = -8, exp_hi: int = -4):
    """MXFP4 weights: E2M1 codes uniform over all 16 codes, one E8M0 scale per
    32 along K with unbiased exponent uniform in [exp_lo, exp_hi]."""
    g = rng(seed)
    codes = np.empty((num_experts, n, k // 2), dtype=np.uint8)
    for e in range(num_experts):  # one expert at a time bounds host memory
        c = g.integers(0, 16, size=(n, k), dtype=np.uint8)
        codes[e] = pack_nibbles(c)
    sc = g.integers(127 + exp_lo, 127 + exp_hi + 1,
                    size=(num_experts, n, k // 32), dtype=np.uint8)
    return {"codes": codes, "scales": sc, "zeros": None,
            "n": n, "k": k, "group": 32, "num_experts": num_experts,
            "weight_dtype": "e2m1"}


def routing(seed: int, t: int, num_experts: int, topk: int,
            zipf_s: float | None = None):
    """Router inputs: logits ~ N(0,1) (+ per-expert bias), softmax in fp64,
    top-k by probability (ties to the lower expert id), weights renormalised
    over the selected experts and stored as float32.

    With ``zipf_s`` the bias of expert e is ``-zipf_s * ln(r_e)`` where r is a
    seeded permutation of 1..E: the Zipf(s) log-weights that skew the load.
    Returns ``(ids int32 [T, topk], weights float32 [T, topk])``.
    """
    g = rng(seed)
    logits = g.standard_normal((t, num_experts), dtype=np.float32).astype(np.float64)
    if zipf_s is not None:
        r = g.permutation(num_experts) + 1
        logits = logits + (-float(zipf_s) * np.log(r.astype(np.float64)))[None, :]
    z = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    # stable sort on (-p, expert id): descending probability, ties -> lower id
    order = np.argsort(-p, axis=1, kind="stable")[:, :topk]
    pt = np.take_along_axis(p, order, axis=1)
    w = (pt / pt.sum(axis=1, keepdims=True)).astype(np.float32)
    return order.astype(np.int32), w
