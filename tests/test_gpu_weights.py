"""GPU: weight repack -> exact dequantization, bit for bit against the oracle
(hum_prepare_weight + hum_dequant_weight vs oracle.gemm.dequant_weight)."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_packed_amd as hum
import synth
from gpu_util import descs, prepare

pytestmark = pytest.mark.gpu

FORMATS = [
    # wd, gran, gs, sd, zero, glob
    ("int4", "group", 128, "bf16", False, False),
    ("int4", "group", 256, "f32", False, True),
    ("int4", "channel", 0, "f32", False, False),
    ("int4", "tensor", 0, "bf16", False, False),
    ("uint4", "group", 128, "bf16", True, False),
    ("uint4", "group", 0, "bf16", True, False),      # G = K (canonicalised to per-channel)
    ("uint4", "channel", 0, "f32", True, True),
    ("e2m1", "group", 32, "e8m0", False, False),
    ("e4m3", "channel", 0, "f32", False, False),
    ("e4m3", "tensor", 0, "f32", False, True),
    ("e4m3", "block", 128, "f32", False, False),
    ("int3", "group", 128, "bf16", False, False),
    ("uint3", "group", 128, "bf16", True, False),
    ("uint3", "channel", 0, "f32", True, True),
    ("int2", "group", 256, "f32", False, False),
    ("uint2", "group", 128, "bf16", True, False),
    ("int1", "tensor", 0, "bf16", False, False),
    ("uint1", "group", 128, "bf16", True, False),
    ("e2m3", "group", 32, "e8m0", False, False),
    ("e3m2", "group", 32, "e8m0", False, True),
]
SHAPES = [(1, 40, 256), (3, 640, 1024), (2, 16, 128)]


@pytest.mark.parametrize("fmt", FORMATS, ids=lambda f: "-".join(map(str, f)))
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_dequant_bit_exact(fmt, shape):
    wd, gran, gs, sd, zero, glob = fmt
    e, n, k = shape
    if gran == "group" and gs == 0:
        gs = k
    if gran in ("group", "block") and k % gs:
        pytest.skip("group does not divide k")
    act = {"e4m3": "fp8_group" if gran == "block" else "fp8_token"}.get(wd, "bf16")
    hd, od = descs(wd, gran, gs, sd, e, n, k, zero, glob, act)
    w = synth.quant_weights(synth.seed_of(fmt, shape), wd, gran, gs, sd, e, n, k, zero, glob,
                            e8m0_lo=100, e8m0_hi=150)
    print(f"case {fmt} {shape}", flush=True)
    packed = prepare(hd, w, sd)
    got = hum.dequant_weight(hd, packed)
    torch.cuda.synchronize()
    ref = oracle.gemm.dequant_weight(od, w["codes"], w["scales"], w.get("zeros"), w.get("global_scale"),
                                     include_global=False).astype(np.float32)
    g = got.cpu().numpy()
    assert np.array_equal(g.view(np.uint32), ref.view(np.uint32)), \
        f"{int((g.view(np.uint32) != ref.view(np.uint32)).sum())} mismatches"


@pytest.mark.parametrize("gran", ["channel", "tensor"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_dequant_bit_exact_fp8_weights_bf16_act(shape, gran):
    """E4M3 weights packed for bf16 activations (their own fragment order)."""
    e, n, k = shape
    hd, od = descs("e4m3", gran, 0, "f32", e, n, k, act="bf16")
    w = synth.quant_weights(synth.seed_of("w8a16", shape, gran), "e4m3", gran, 0, "f32", e, n, k)
    packed = prepare(hd, w, "f32")
    got = hum.dequant_weight(hd, packed)
    torch.cuda.synchronize()
    ref = oracle.gemm.dequant_weight(od, w["codes"], w["scales"], include_global=False).astype(np.float32)
    g = got.cpu().numpy()
    assert np.array_equal(g.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("gran", ["channel", "tensor"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_dequant_bit_exact_int8(shape, gran):
    """INT8 weights (the FP8-for-bf16 fragment order, every code)."""
    e, n, k = shape
    hd, od = descs("int8", gran, 0, "f32", e, n, k)
    w = synth.quant_weights(synth.seed_of("int8", shape, gran), "int8", gran, 0, "f32", e, n, k)
    packed = prepare(hd, w, "f32")
    got = hum.dequant_weight(hd, packed)
    torch.cuda.synchronize()
    ref = oracle.gemm.dequant_weight(od, w["codes"], w["scales"], include_global=False).astype(np.float32)
    g = got.cpu().numpy()
    assert np.array_equal(g.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_dequant_bit_exact_nvfp4(shape):
    """NVFP4: E2M1 x its E4M3 group scale (16 along K), every scale code
    from subnormal to 448 (exact in f32)."""
    e, n, k = shape
    hd, od = descs("e2m1", "group", 16, "e4m3", e, n, k)
    w = synth.quant_weights(synth.seed_of("nvfp4", shape), "e2m1", "group", 16, "e4m3", e, n, k,
                            e4m3_lo=0x01, e4m3_hi=0x7E)
    packed = prepare(hd, w, "e4m3")
    got = hum.dequant_weight(hd, packed)
    torch.cuda.synchronize()
    ref = oracle.gemm.dequant_weight(od, w["codes"], w["scales"], include_global=False).astype(np.float32)
    g = got.cpu().numpy()
    assert np.array_equal(g.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_dequant_bit_exact_mxint4(shape):
    """MXINT4: every INT4 code times its E8M0 scale per 32."""
    e, n, k = shape
    hd, od = descs("int4", "group", 32, "e8m0", e, n, k)
    w = synth.quant_weights(synth.seed_of("mxint4", shape), "int4", "group", 32, "e8m0", e, n, k)
    packed = prepare(hd, w, "e8m0")
    got = hum.dequant_weight(hd, packed)
    torch.cuda.synchronize()
    ref = oracle.gemm.dequant_weight(od, w["codes"], w["scales"], include_global=False).astype(np.float32)
    g = got.cpu().numpy()
    assert np.array_equal(g.view(np.uint32), ref.view(np.uint32))


def test_group_k_equals_channel_bitwise():
    e, n, k = 1, 96, 512
    w = synth.quant_weights(5, "uint4", "group", k, "bf16", e, n, k, zero=True)
    hd_g, _ = descs("uint4", "group", k, "bf16", e, n, k, zero=True)
    hd_c, _ = descs("uint4", "channel", 0, "bf16", e, n, k, zero=True)
    pg = prepare(hd_g, w, "bf16")
    pc = prepare(hd_c, w, "bf16")
    assert hum.packed_weight_bytes(hd_g) == hum.packed_weight_bytes(hd_c)
    assert torch.equal(hum.dequant_weight(hd_g, pg), hum.dequant_weight(hd_c, pc))
    x = torch.randn(7, k, device="cuda").to(torch.bfloat16)
    assert torch.equal(hum.linear(hd_g, pg, x), hum.linear(hd_c, pc, x))
