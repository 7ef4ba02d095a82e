"""CPU checks of the binding's argument validation and of host-side
refusals that must happen before any launch: wrong dtypes or shapes are a
ValueError (the kernels size their memory accesses from the description,
not from the tensors), and configurations the library cannot finish are
refused by the C ABI with nothing enqueued."""
import ctypes

import pytest
import torch

import quantized_gemm_packed_amd as hum


@pytest.fixture(scope="module")
def lib():
    return hum.load_library()


def _d(**kw):
    base = dict(weight_dtype="int4", scale_gran="group", group_size=128, scale_dtype="bf16", n=64, k=256)
    base.update(kw)
    n, k = base.pop("n"), base.pop("k")
    return hum.make_desc(base.pop("weight_dtype"), base.pop("scale_gran"), base.pop("group_size"),
                         base.pop("scale_dtype"), n, k, **base)


def test_linear_rejects_wrong_activation_dtype_and_shape(lib):
    d = _d()
    pk = torch.zeros(hum.packed_weight_bytes(d), dtype=torch.uint8)
    with pytest.raises(ValueError, match="bfloat16"):
        hum.linear(d, pk, torch.zeros(4, 256, dtype=torch.float32))
    with pytest.raises(ValueError, match="shape"):
        hum.linear(d, pk, torch.zeros(4, 128, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out"):
        hum.linear(d, pk, torch.zeros(4, 256, dtype=torch.bfloat16), out=torch.zeros(4, 32, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="bias"):
        hum.linear(d, pk, torch.zeros(4, 256, dtype=torch.bfloat16), bias=torch.zeros(64, dtype=torch.float32))
    with pytest.raises(ValueError, match="packed"):
        hum.linear(d, pk.view(torch.int8), torch.zeros(4, 256, dtype=torch.bfloat16))


def test_linear_rejects_wrong_prequantized_layout(lib):
    d = _d(weight_dtype="e4m3", scale_gran="channel", group_size=0, scale_dtype="f32", act_fmt="fp8_token")
    pk = torch.zeros(hum.packed_weight_bytes(d), dtype=torch.uint8)
    q = torch.zeros(4, 256, dtype=torch.uint8)
    with pytest.raises(ValueError, match="a_scales"):
        hum.linear(d, pk, q, a_scales=torch.zeros(4, 2, dtype=torch.float32))
    with pytest.raises(ValueError, match="pre-quantized"):
        hum.linear(d, pk, torch.zeros(4, 256, dtype=torch.bfloat16), a_scales=torch.zeros(4, dtype=torch.float32))
    d4 = _d(weight_dtype="e2m1", group_size=32, scale_dtype="e8m0", act_fmt="mxfp4")
    pk4 = torch.zeros(hum.packed_weight_bytes(d4), dtype=torch.uint8)
    with pytest.raises(ValueError, match="shape"):   # E2M1 codes are k/2 bytes per row
        hum.linear(d4, pk4, torch.zeros(4, 256, dtype=torch.uint8), a_scales=torch.zeros(4, 8, dtype=torch.uint8))


def test_moe_rejects_int64_ids_and_wrong_weights(lib):
    w13 = _d(weight_dtype="e2m1", group_size=32, scale_dtype="e8m0", n=256, k=256, num_experts=4)
    w2 = _d(weight_dtype="e2m1", group_size=32, scale_dtype="e8m0", n=256, k=128, num_experts=4)
    p13 = torch.zeros(hum.packed_weight_bytes(w13), dtype=torch.uint8)
    p2 = torch.zeros(hum.packed_weight_bytes(w2), dtype=torch.uint8)
    x = torch.zeros(3, 256, dtype=torch.bfloat16)
    ids64 = torch.zeros(3, 2, dtype=torch.int64)         # what torch.topk returns
    w = torch.zeros(3, 2, dtype=torch.float32)
    with pytest.raises(ValueError, match="topk_ids"):
        hum.moe_gemm(w13, p13, w2, p2, x, ids64, w)
    ids = ids64.to(torch.int32)
    with pytest.raises(ValueError, match="topk_weights"):
        hum.moe_gemm(w13, p13, w2, p2, x, ids, w.to(torch.bfloat16))
    with pytest.raises(ValueError, match="x"):
        hum.moe_gemm(w13, p13, w2, p2, torch.zeros(3, 128, dtype=torch.bfloat16), ids, w)
    with pytest.raises(ValueError, match="out"):
        hum.moe_gemm(w13, p13, w2, p2, x, ids, w, out=torch.zeros(3, 256, dtype=torch.float32))
    with pytest.raises(ValueError, match="topk_ids"):
        hum.moe_align(ids64, 4, 16)
    with pytest.raises(ValueError, match="y"):
        hum.moe_reduce(torch.zeros(5, 256, dtype=torch.bfloat16), w)


def test_prepare_rejects_wrong_sizes(lib):
    d = _d(has_zero=True, weight_dtype="uint4")
    codes = torch.zeros(64, 128, dtype=torch.uint8)
    scales = torch.zeros(64, 2, dtype=torch.int16)
    zeros = torch.zeros(64, 2, dtype=torch.uint8)
    with pytest.raises(ValueError, match="codes"):
        hum.prepare_weight(d, codes[:32], scales, zeros)
    with pytest.raises(ValueError, match="scales"):
        hum.prepare_weight(d, codes, scales.to(torch.float32), zeros)
    with pytest.raises(ValueError, match="zeros"):
        hum.prepare_weight(d, codes, scales, zeros[:, :1])


def test_w4a4_moe_split_k_refused_before_launch(lib):
    """W4A4 MoE GEMMs have no split-K reduce: a forced split must be refused
    by the argument checks (NULL buffers prove nothing was launched)."""
    w13 = _d(weight_dtype="e2m1", group_size=32, scale_dtype="e8m0", n=256, k=256, num_experts=4, act_fmt="mxfp4")
    w2 = _d(weight_dtype="e2m1", group_size=32, scale_dtype="e8m0", n=256, k=128, num_experts=4, act_fmt="mxfp4")
    c = hum.TileConfig()
    c.kind, c.wave_m, c.wave_n, c.waves_n, c.waves_k, c.split_k, c.block_m, c.stages = 0, 1, 4, 4, 1, 2, 16, 2
    p = ctypes.c_void_p(16)   # never dereferenced: the call must fail first
    st = lib.hum_moe_gemm_ex(ctypes.byref(w13), p, ctypes.byref(w2), p, 4, 2, p, p, p, p, p, 1 << 30,
                             ctypes.byref(c), None)
    assert st == 2 and b"split-K" in lib.hum_last_error()


@pytest.mark.parametrize("h", [5120, 7168])
@pytest.mark.parametrize("act", ["bf16", "mxfp8"])
def test_moe_selection_fits_lds_for_wide_hidden(lib, h, act):
    """The decode-kernel MoE configuration stages every activation row of its
    K range in LDS: for hidden sizes above 4096 the selector must raise
    split-K (or fall back to tiles) so that the plan fits the 159 KB limit."""
    e, inter, topk = 128, 1024, 8
    w13 = hum.make_desc("e2m1", "group", 32, "e8m0", 2 * inter, h, num_experts=e, act_fmt=act)
    w2 = hum.make_desc("e2m1", "group", 32, "e8m0", h, inter, num_experts=e, act_fmt=act)
    for t in range(1, 17):
        assert hum.moe_workspace_bytes(w13, w2, t, topk) > 0
        for gate_up, k in ((True, h), (False, inter)):
            c = hum.moe_select_config(w13, w2, t, topk, gate_up=gate_up)
            if c.kind == hum.KERNEL_STREAM:
                rows = min(t * topk, 16)
                kb = k // 128
                per = -(-kb // c.split_k)
                per = -(-per // c.waves_k) * c.waves_k
                row_bytes = 256 if act == "bf16" else 132
                assert rows * per * row_bytes <= 159 * 1024, (t, gate_up, c)
