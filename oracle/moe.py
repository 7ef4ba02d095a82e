"""Oracle MoE layer (TEST INFRASTRUCTURE ONLY).

What the pages fix: an MoE layer runs a fused Gateup GEMM and a Down GEMM per
expert ("Announcing Humming: Fast, Flexible Kernels for Quantized Inference",
section "Performance": the MoE figure sums the Gateup and Down GEMM
latencies); tokens are routed by ``topk_ids`` / ``topk_weights``, grouped by
expert (``moe_align_block_size``, ``moe_permute_prepare``) and the expert
outputs are combined by a top-k weighted sum (``moe_fused_mul_sum``,
``moe_unpermute``) -- sections "Implementation breakdown" and "Key source
snippets" of the prhub.com.cn summary of SGLang PR #23754.

Readings where the pages are silent:

* activation between the GEMMs: a = silu(h[:I]) * h[I:], silu(g) = g/(1+e^-g),
  gate = first I rows of the fused weight, up = last I rows; no clamp and a
  routed scaling factor of 1.
* precision at the stage boundary follows the activation format: bf16 (RNE)
  for W4A16, MXFP8 of the float value for W4A8, MXFP4 of it for W4A4; the
  token activations are MXFP8- (W4A8) or MXFP4- (W4A4) quantized.  With FP8
  activations (per token, or per token and 128 along K for block-scaled
  experts -- the W8A8 of section "W8A8 / W4A8 / W4A4") the layer input is
  quantized with that rule, and the SwiGLU output is rounded to bf16 and
  then quantized with the same rule (a per-row amax spans the whole
  intermediate row, so the rule applies to the stored bf16 row).
* align: flat index f = t*topk + j; experts' segments in expert order, each
  padded to a multiple of block_m; inside a segment ascending f (stable);
  padding slots hold the sentinel T*topk.
* reduce: out[t] = sum_j w[t,j] * y[t*topk + j], then bf16.
"""
from __future__ import annotations

import numpy as np

from .formats import decode_bf16, encode_bf16
from .gemm import WeightDesc, dequant_weight
from .quant import (dequant_fp8_group, dequant_fp8_per_token, dequant_mxfp4, dequant_mxfp8, quant_fp8_group,
                    quant_fp8_per_token, quant_mxfp4, quant_mxfp8)


def align_capacity(num_tokens: int, topk: int, num_experts: int, block_m: int) -> int:
    """Upper bound of the padded sorted-id buffer length."""
    return num_tokens * topk + num_experts * (block_m - 1)


def align(ids, num_experts: int, block_m: int):
    """ids int [T, topk] -> (sorted int32 [capacity], offsets int32 [E+1],
    counts int32 [E]).  Entries past offsets[E] also hold the sentinel."""
    ids = np.asarray(ids, dtype=np.int64)
    t, k = ids.shape
    flat = ids.reshape(-1)
    sentinel = t * k
    counts = np.bincount(flat, minlength=num_experts)[:num_experts].astype(np.int64)
    padded = -(-counts // block_m) * block_m
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(padded)
    cap = align_capacity(t, k, num_experts, block_m)
    out = np.full(cap, sentinel, dtype=np.int64)
    order = np.argsort(flat, kind="stable")     # by expert, ties by ascending f
    start = 0
    for e in range(num_experts):
        c = int(counts[e])
        out[offsets[e]:offsets[e] + c] = order[start:start + c]
        start += c
    return out.astype(np.int32), offsets.astype(np.int32), counts.astype(np.int32)


def silu(g):
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu(h, inter: int):
    return silu(h[:, :inter]) * h[:, inter:2 * inter]


def round_bf16(a):
    return decode_bf16(encode_bf16(a))


def qdq_mxfp8(a):
    q, e = quant_mxfp8(a)
    return dequant_mxfp8(q, e)


def qdq_mxfp4(a):
    q, e = quant_mxfp4(a)
    return dequant_mxfp4(q, e)


def qdq_fp8_token(a):
    """Per-token FP8 quantize-dequantize of float32-representable rows
    (bf16 values)."""
    q, s = quant_fp8_per_token(np.asarray(a, np.float64).astype(np.float32))
    return dequant_fp8_per_token(q, s)


def qdq_fp8_group(a):
    q, s = quant_fp8_group(np.asarray(a, np.float64).astype(np.float32))
    return dequant_fp8_group(q, s)


def stage_precision(a, act_fmt: str):
    """The SwiGLU output as the down GEMM sees it."""
    if act_fmt == "bf16":
        return round_bf16(a)
    if act_fmt == "mxfp8":
        return qdq_mxfp8(a)
    if act_fmt == "mxfp4":
        return qdq_mxfp4(a)
    if act_fmt == "fp8_token":
        return qdq_fp8_token(round_bf16(a))
    if act_fmt == "fp8_group":
        return qdq_fp8_group(round_bf16(a))
    raise ValueError(act_fmt)


def moe_forward(desc13: WeightDesc, w13: dict, desc2: WeightDesc, w2: dict,
                x_bits, ids, weights, act_fmt: str, experts=None,
                return_y: bool = False, dequant=None):
    """Full MoE layer in float64.  Returns out (float64 [T, H]) before the
    final bf16 rounding, and optionally y (float64 [T*topk, H]) indexed by
    flat routing index.

    ``w13`` / ``w2``: dicts with canonical ``codes``, ``scales`` and optional
    ``zeros`` / ``global_scale``.  ``act_fmt``: "bf16" (W4A16), "mxfp8"
    (W4A8) or "mxfp4" (W4A4: the layer input and the SwiGLU output are
    quantized to MXFP4 the way MXFP8 is for W4A8).  ``experts``: restrict to these experts (bounded samples).
    ``dequant``: optional e -> (W13[e], W2[e]) giving the dequantized weights
    (a caller's cache of dequant_weight results, for repeated calls).
    """
    ids = np.asarray(ids, dtype=np.int64)
    wts = np.asarray(weights, dtype=np.float32).astype(np.float64)
    t, k = ids.shape
    hdim = desc13.k
    inter = desc2.k
    assert desc13.n == 2 * inter and desc2.n == hdim
    x = decode_bf16(x_bits)
    a_in = quant_input(x, act_fmt)
    out = np.zeros((t, hdim), dtype=np.float64)
    y_all = np.zeros((t * k, hdim), dtype=np.float64) if return_y else None
    flat = ids.reshape(-1)
    ex = range(desc13.num_experts) if experts is None else experts
    for e in ex:
        f = np.nonzero(flat == e)[0]
        if f.size == 0:
            continue
        tok = f // k
        y = expert_mlp(desc13, w13, desc2, w2, a_in[tok], e, act_fmt, dequant)
        if return_y:
            y_all[f] = y
        np.add.at(out, tok, wts.reshape(-1)[f][:, None] * y)
    return (out, y_all) if return_y else out


def quant_input(x, act_fmt: str):
    """The layer input as the GEMM sees it: MXFP8 / MXFP4 quantize-dequantize
    per row and 32 along H, or the bf16 values themselves."""
    if act_fmt == "mxfp8":
        return qdq_mxfp8(x)
    if act_fmt == "mxfp4":
        return qdq_mxfp4(x)
    if act_fmt == "fp8_token":
        return qdq_fp8_token(x)
    if act_fmt == "fp8_group":
        return qdq_fp8_group(x)
    if act_fmt == "bf16":
        return x
    raise ValueError(act_fmt)


def expert_mlp(desc13: WeightDesc, w13: dict, desc2: WeightDesc, w2: dict, a_in, e: int, act_fmt: str,
               dequant=None):
    """One expert on its rows a_in (float64 [R, H], already in the input
    format): h = a_in W13[e]^T, a = SwiGLU(h) at the stage precision,
    y = a W2[e]^T (float64 [R, H])."""
    inter = desc2.k
    if dequant is not None:
        w_gu, w_dn = dequant(e)
        w_gu = np.asarray(w_gu, dtype=np.float64)
        w_dn = np.asarray(w_dn, dtype=np.float64)
    else:
        w_gu = dequant_weight(desc13, w13["codes"], w13["scales"], w13.get("zeros"),
                              w13.get("global_scale"), experts=[e])[0]
        w_dn = None
    h = np.asarray(a_in, dtype=np.float64) @ w_gu.T
    del w_gu
    a = stage_precision(swiglu(h, inter), act_fmt)
    if w_dn is None:
        w_dn = dequant_weight(desc2, w2["codes"], w2["scales"], w2.get("zeros"),
                              w2.get("global_scale"), experts=[e])[0]
    return a @ w_dn.T


def moe_masked(desc13: WeightDesc, w13: dict, desc2: WeightDesc, w2: dict, x_bits, counts, act_fmt: str):
    """The expert layer on the grouped_masked layout, a gemm_type of the MoE
    runner (prhub.com.cn summary of SGLang PR #23754, "Key source
    snippets"), whose arguments alone the pages give.  Reading: x_bits is
    bf16 [E, max_m, H]; expert e's rows are the first counts[e] (clamped to
    [0, max_m]); each runs the expert MLP of the indexed layer and its result
    is that row's down output, without top-k weighting (the combine after
    the layer applies it).  Returns (float64 [E, max_m, H], bool [E, max_m]
    of the rows defined; the others are zero)."""
    x = decode_bf16(x_bits)
    e_count, max_m, hdim = x.shape
    out = np.zeros((e_count, max_m, hdim), dtype=np.float64)
    valid = np.zeros((e_count, max_m), dtype=bool)
    for e in range(e_count):
        c = int(min(max(int(counts[e]), 0), max_m))
        if c == 0:
            continue
        out[e, :c] = expert_mlp(desc13, w13, desc2, w2, quant_input(x[e, :c], act_fmt), e, act_fmt)
        valid[e, :c] = True
    return out, valid


def reduce(y, weights, topk: int):
    """out[t] = sum_j w[t,j] * y[t*topk + j] (float64), y float64 [T*topk, H]."""
    y = np.asarray(y, dtype=np.float64)
    w = np.asarray(weights, dtype=np.float32).astype(np.float64)
    t = w.shape[0]
    return (y.reshape(t, topk, -1) * w[:, :, None]).sum(axis=1)
