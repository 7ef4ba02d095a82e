"""Oracle weight dequantization and dense quantized linear layer
(TEST INFRASTRUCTURE ONLY).

The quantization description follows "Announcing Humming: Fast, Flexible
Kernels for Quantized Inference", section "Unified quantization
representation": weight format, scale granularity, scale dtype, zero point
and a second-level scale are independent parameters, and the activations
carry their own format.  Readings where the page is silent:

* zero point: an integer z subtracted from the decoded code before scaling,
  W = (v(q) - z) * S; only unsigned integer codes (UINT1..UINT4) carry one,
  z in [0, 2^b).
* group g of element k is floor(k / G); channel granularity is G = K;
  tensor granularity is one scale per expert.
* the second-level scale is one float32 per expert, multiplied after the
  first-level scale.
* "block" granularity (the block-scaled FP8 W8A8 of section "W8A8 / W4A8 /
  W4A4", whose block shape the page does not give): one scale per
  group_size x group_size block of W (rows n, columns k), block (n // G,
  k // G); scales are [E][ceil(N/G)][K/G].

The layer is C[m, n] = sum_k A[m, k] * W[n, k] (+ bias[n]) evaluated in
float64 from the exactly dequantized operands; the GPU returns bf16(C).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .formats import decode_bf16, decode_scale, decode_weight_codes, decode_e4m3
from .quant import dequant_fp8_group, dequant_fp8_per_token, dequant_mxfp4, dequant_mxfp8


@dataclass
class WeightDesc:
    weight_dtype: str          # "int1".."int4" | "uint1".."uint4" | "int8" | "e2m1" | "e2m3" | "e3m2" | "e4m3"
    scale_gran: str            # "tensor" | "channel" | "group"
    group_size: int            # along K (ignored unless scale_gran == "group")
    scale_dtype: str           # "bf16" | "f32" | "e8m0" | "e4m3" (NVFP4: E2M1 codes, G = 16)
    has_zero: bool
    has_global: bool
    num_experts: int
    n: int
    k: int

    def groups(self) -> int:
        if self.scale_gran in ("group", "block"):
            return self.k // self.group_size
        return 1


def _expand_groups(a, desc: WeightDesc):
    """[E][N or 1][groups] -> [E][N][K] by repeating each group along K."""
    a = np.asarray(a, dtype=np.float64)
    if desc.scale_gran == "block":
        rep = np.repeat(np.repeat(a, desc.group_size, axis=2), desc.group_size, axis=1)[:, :desc.n, :]
        return rep
    if desc.scale_gran == "group":
        rep = np.repeat(a, desc.group_size, axis=2)
    else:
        rep = np.repeat(a, desc.k, axis=2)
    return np.broadcast_to(rep, (desc.num_experts, desc.n, desc.k))


def dequant_weight(desc: WeightDesc, codes, scales, zeros=None, global_scale=None,
                   include_global: bool = True, experts=None):
    """Canonical tensors -> float64 W [E][N][K] (or the listed experts only).

    W[e,n,k] = (v(q[e,n,k]) - z[e,n,g]) * S[e,n,g] * S2[e].
    """
    sel = slice(None) if experts is None else np.asarray(experts)
    codes = np.asarray(codes)[sel]
    sc = np.asarray(scales)[sel]
    sub = WeightDesc(**{**desc.__dict__, "num_experts": codes.shape[0]})
    v = decode_weight_codes(codes, desc.weight_dtype)
    s = _expand_groups(decode_scale(sc, desc.scale_dtype), sub)
    if desc.has_zero:
        z = _expand_groups(np.asarray(zeros)[sel].astype(np.float64), sub)
        w = (v - z) * s
    else:
        w = v * s
    if include_global and desc.has_global:
        g = np.asarray(global_scale, dtype=np.float32)[sel].astype(np.float64)
        w = w * g[:, None, None]
    return w


def activations(act_fmt: str, x=None, q=None, scales=None):
    """Exact float64 activations for each activation format."""
    if act_fmt == "bf16":
        return decode_bf16(x)
    if act_fmt == "fp8_token":
        return dequant_fp8_per_token(q, scales)
    if act_fmt == "mxfp8":
        return dequant_mxfp8(q, scales)
    if act_fmt == "mxfp4":
        return dequant_mxfp4(q, scales)
    if act_fmt == "fp8_group":
        return dequant_fp8_group(q, scales)
    raise ValueError(act_fmt)


def linear(desc: WeightDesc, a, codes, scales, zeros=None, global_scale=None,
           bias_bits=None, expert: int = 0):
    """C = A @ W[expert]^T (+ bias) in float64.  ``a`` is float64 [M, K]."""
    w = dequant_weight(desc, codes, scales, zeros, global_scale, experts=[expert])[0]
    c = np.asarray(a, dtype=np.float64) @ w.T
    if bias_bits is not None:
        c = c + decode_bf16(bias_bits)[None, :]
    return c


def linear_fp8_e4m3(a, w_codes, w_scale):
    """Per-channel FP8 W8A8 written out as the plain definition:
    C[m,n] = sum_k A[m,k] * v(q[n,k]) * s_w[n]."""
    w = decode_e4m3(w_codes) * np.asarray(w_scale, np.float32).astype(np.float64)[:, None]
    return np.asarray(a, dtype=np.float64) @ w.T
