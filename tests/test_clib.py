"""CPU checks of the C ABI library: it loads, exports every function
include/hum.h declares, and its host-side validation / sizing / selector
paths answer without touching a GPU."""
import ctypes

import numpy as np
import pytest

import quantized_gemm_packed_amd as hum


@pytest.fixture(scope="module")
def lib():
    return hum.load_library()


def test_exports_every_header_function(lib):
    names = hum.header_functions()
    assert len(names) >= 15
    raw = ctypes.CDLL(hum.lib_path())
    missing = [n for n in names if not hasattr(raw, n)]
    assert not missing, missing
    assert set(names) <= set(hum._SIGS), set(names) - set(hum._SIGS)


def test_packed_size_dense_int4(lib):
    d = hum.make_desc("uint4", "group", 128, "bf16", 8192, 8192, has_zero=True)
    nb = hum.packed_weight_bytes(d)
    codes = 8192 * 8192 // 2
    scales = 8192 * 64 * 2
    zeros = 8192 * 64 // 2
    # per column and K-block, the offset term as a bf16 hi / lo pair (K-blocks
    # padded to 32)
    offsets = 8192 * 64 * 4
    assert codes + scales + zeros + offsets <= nb <= codes + scales + zeros + offsets + 4096


@pytest.mark.parametrize("wd,bits", [("int3", 3), ("uint3", 3), ("int2", 2), ("uint2", 2), ("int1", 1), ("uint1", 1)])
def test_packed_size_low_bit_integers(lib, wd, bits):
    """b-bit codes take 4b bytes per lane and K-block (N = K = 8192, G = 128,
    bf16 scales, zero points for the unsigned codes)."""
    zero = wd.startswith("u")
    d = hum.make_desc(wd, "group", 128, "bf16", 8192, 8192, has_zero=zero)
    nb = hum.packed_weight_bytes(d)
    codes = 8192 * 8192 * bits // 8
    scales = 8192 * 64 * 2
    zeros = 8192 * 64 // 2 if zero else 0
    offsets = 8192 * 64 * 4
    assert codes + scales + zeros + offsets <= nb <= codes + scales + zeros + offsets + 4096


def test_packed_size_ragged_n_pads_to_16(lib):
    d = hum.make_desc("int4", "group", 128, "bf16", 40, 256)
    assert hum.packed_weight_bytes(d) >= 48 * 256 // 2


@pytest.mark.parametrize("bad", [
    dict(weight_dtype="int4", scale_gran="group", group_size=64, scale_dtype="bf16"),   # G % 128
    dict(weight_dtype="int4", scale_gran="group", group_size=128, scale_dtype="bf16", has_zero=True),
    dict(weight_dtype="e2m1", scale_gran="group", group_size=128, scale_dtype="e8m0"),
    dict(weight_dtype="e4m3", scale_gran="channel", group_size=0, scale_dtype="f32", act_fmt="mxfp8"),
    dict(weight_dtype="e4m3", scale_gran="group", group_size=128, scale_dtype="f32", act_fmt="fp8_token"),
    dict(weight_dtype="int8", scale_gran="group", group_size=128, scale_dtype="f32"),
    dict(weight_dtype="e2m1", scale_gran="group", group_size=32, scale_dtype="e4m3"),
    dict(weight_dtype="int4", scale_gran="group", group_size=128, scale_dtype="e8m0"),
    dict(weight_dtype="uint4", scale_gran="group", group_size=32, scale_dtype="e8m0"),
    dict(weight_dtype="e2m1", scale_gran="group", group_size=16, scale_dtype="e4m3", act_fmt="mxfp8"),
    dict(weight_dtype="int8", scale_gran="channel", group_size=0, scale_dtype="bf16"),
    dict(weight_dtype="int8", scale_gran="channel", group_size=0, scale_dtype="f32", act_fmt="fp8_token"),
    dict(weight_dtype="int3", scale_gran="group", group_size=128, scale_dtype="bf16", has_zero=True),
    dict(weight_dtype="int2", scale_gran="group", group_size=32, scale_dtype="e8m0"),
    dict(weight_dtype="uint3", scale_gran="group", group_size=128, scale_dtype="bf16", act_fmt="mxfp8"),
    dict(weight_dtype="int1", scale_gran="group", group_size=64, scale_dtype="bf16"),
])
def test_unsupported_descriptions_rejected(lib, bad):
    kw = dict(n=256, k=1024)
    kw.update(bad)
    d = hum.make_desc(kw.pop("weight_dtype"), kw.pop("scale_gran"), kw.pop("group_size"), kw.pop("scale_dtype"),
                      **kw)
    assert lib.hum_packed_weight_bytes(ctypes.byref(d)) == 0
    assert lib.hum_last_error()


def test_k_not_multiple_of_128_rejected(lib):
    d = hum.make_desc("int4", "channel", 0, "bf16", 64, 200)
    assert lib.hum_packed_weight_bytes(ctypes.byref(d)) == 0
    assert b"multiple of 128" in lib.hum_last_error()


def test_null_pointers_rejected_before_launch(lib):
    d = hum.make_desc("int4", "group", 128, "bf16", 64, 256)
    st = lib.hum_prepare_weight(ctypes.byref(d), None, None, None, None, None, 0, None)
    assert st == 1
    st = lib.hum_linear(ctypes.byref(d), None, 4, None, None, None, None, None, 0, None)
    assert st == 1


def test_small_packed_buffer_is_workspace_error(lib):
    d = hum.make_desc("int4", "group", 128, "bf16", 64, 256)
    st = lib.hum_prepare_weight(ctypes.byref(d), ctypes.c_void_p(16), ctypes.c_void_p(16), None, None,
                                ctypes.c_void_p(16), 10, None)
    assert st == 3


def test_selector_is_deterministic_and_covers_m_range(lib):
    d = hum.make_desc("uint4", "group", 128, "bf16", 8192, 8192, has_zero=True)
    seen = set()
    for m in (1, 4, 16, 64, 256, 1024, 4096):
        c1 = hum.select_config(d, m).as_tuple()
        c2 = hum.select_config(d, m).as_tuple()
        assert c1 == c2
        kind, wave_m, wave_n, waves_n, waves_k, split_k, block_m, stages, stream_k = c1
        assert split_k >= 1 and block_m == 16 * wave_m
        assert kind == (1 if m <= 4 else (2 if m >= 256 else 0))   # decode, 16x16 tiles, 32x32 tiles
        assert 16 * wave_m >= min(m, 32)
        seen.add(c1)
    assert len(seen) >= 3


@pytest.mark.parametrize("fmt", [
    ("uint4", "group", 128, "bf16", dict(has_zero=True), 8192, 8192),
    ("e4m3", "channel", 0, "f32", dict(act_fmt="fp8_token"), 7168, 2048),
    ("e4m3", "channel", 0, "f32", dict(), 7168, 2048),
    ("e2m1", "group", 32, "e8m0", dict(act_fmt="mxfp8"), 7168, 2048),
])
def test_batch_invariant_selection(lib, fmt):
    """Every M gets a tile-kernel configuration without split-K; the tile
    shape may still follow M."""
    wd, gran, gs, sd, kw, n, k = fmt
    d = hum.make_desc(wd, gran, gs, sd, n, k, **kw)
    for m in (0, 1, 4, 16, 17, 64, 256, 1024, 4096):
        c = hum.select_config(d, m, batch_invariant=True)
        assert c.kind == hum.KERNEL_TILE and c.split_k == 1 and c.block_m == 16 * c.wave_m, (m, c)
    bad = hum.TileConfig()
    assert lib.hum_select_config_ex(ctypes.byref(d), 4, 2, ctypes.byref(bad)) != 0
    assert b"flags" in lib.hum_last_error()


def test_autotune_argument_errors(lib):
    """Rejected before any device work."""
    d = hum.make_desc("int4", "group", 128, "bf16", 256, 1024)
    best = hum.TileConfig()
    us = ctypes.c_float()
    f = lib.hum_autotune_linear
    assert f(ctypes.byref(d), None, 4, None, None, None, None, None, 0, 10, 0, ctypes.byref(best), ctypes.byref(us),
             None) == 1
    p = ctypes.c_void_p(16)
    assert f(ctypes.byref(d), p, 4, p, None, None, p, None, 0, 0, 0, ctypes.byref(best), None, None) == 1
    assert f(ctypes.byref(d), p, 4, p, None, None, p, None, 0, 10, 4, ctypes.byref(best), None, None) == 1
    assert b"flags" in lib.hum_last_error()
    assert f(ctypes.byref(d), p, 0, p, None, None, p, None, 0, 10, 0, ctypes.byref(best), None, None) == 1
    assert f(ctypes.byref(d), p, 4, p, None, None, p, None, 0, 10, 0, None, None, None) == 1


def test_moe_expert_formats(lib):
    """The MoE layer takes every expert format of the description with a
    MoE path; w13 and w2 must share one."""
    ok = [("e2m1", "group", 32, "e8m0", "bf16"), ("e2m1", "group", 32, "e8m0", "mxfp8"),
          ("e2m1", "group", 32, "e8m0", "mxfp4"), ("e2m1", "group", 16, "e4m3", "bf16"),
          ("int4", "group", 32, "e8m0", "bf16"), ("e4m3", "channel", 0, "f32", "bf16"),
          ("e4m3", "channel", 0, "f32", "fp8_token"), ("e4m3", "block", 128, "f32", "fp8_group"),
          ("int8", "channel", 0, "f32", "bf16")]
    for wd, gr, gs, sd, act in ok:
        w13 = hum.make_desc(wd, gr, gs, sd, 512, 256, num_experts=4, act_fmt=act)
        w2 = hum.make_desc(wd, gr, gs, sd, 256, 256, num_experts=4, act_fmt=act)
        assert lib.hum_moe_workspace_bytes(ctypes.byref(w13), ctypes.byref(w2), 8, 2) > 0, (wd, act, lib.hum_last_error())
    w13 = hum.make_desc("e2m1", "group", 32, "e8m0", 512, 256, num_experts=4)
    w2 = hum.make_desc("e2m1", "group", 16, "e4m3", 256, 256, num_experts=4)
    assert lib.hum_moe_workspace_bytes(ctypes.byref(w13), ctypes.byref(w2), 8, 2) == 0
    assert b"differ" in lib.hum_last_error()


def test_moe_batch_invariant_selection(lib):
    w13 = hum.make_desc("e2m1", "group", 32, "e8m0", 2048, 4096, num_experts=128, act_fmt="mxfp8")
    w2 = hum.make_desc("e2m1", "group", 32, "e8m0", 4096, 1024, num_experts=128, act_fmt="mxfp8")
    kinds = set()
    for t in (0, 1, 16, 64, 1024, 8192):
        kinds.add(hum.moe_select_config(w13, w2, t, 8).kind)
        kinds.add(hum.moe_select_config(w13, w2, t, 8, gate_up=True).kind)
        c = hum.moe_select_config(w13, w2, t, 8, batch_invariant=True)
        assert c.kind == hum.KERNEL_TILE and c.split_k == 1, (t, c)
        assert hum.moe_workspace_bytes(w13, w2, max(t, 1), 8, c) > 0
    assert hum.KERNEL_STREAM in kinds    # the default does use the decode kernel (gate_up at decode sizes)


def test_workspace_sizes(lib):
    d = hum.make_desc("e4m3", "channel", 0, "f32", 7168, 2048, act_fmt="fp8_token")
    assert hum.linear_workspace_bytes(d, 128) >= 128 * 2048 + 128 * 4
    w13 = hum.make_desc("e2m1", "group", 32, "e8m0", 2048, 4096, num_experts=128)
    w2 = hum.make_desc("e2m1", "group", 32, "e8m0", 4096, 1024, num_experts=128)
    nb = hum.moe_workspace_bytes(w13, w2, 64, 8)
    assert nb >= 64 * 8 * 4096 * 2


def test_k_beyond_limit_rejected(lib):
    ok = hum.make_desc("int4", "group", 128, "bf16", 64, 1 << 21)
    assert lib.hum_packed_weight_bytes(ctypes.byref(ok)) > 0
    d = hum.make_desc("int4", "group", 128, "bf16", 64, (1 << 21) + 128)
    assert lib.hum_packed_weight_bytes(ctypes.byref(d)) == 0
    assert b"too large" in lib.hum_last_error()


def test_group_index_by_fp32_reciprocal_is_exact():
    """The GEMM kernels find the scale group of K-block kb as
    floor((kb + 1/2) * fl(1 / d)) in fp32 (d = K-blocks per group).  Check it
    against integer division for every kb < 2^14 (k <= 2^21) and every d."""
    kb = np.arange(1 << 14, dtype=np.float32) + np.float32(0.5)
    kbi = np.arange(1 << 14, dtype=np.int64)
    for d in range(1, (1 << 14) + 1):
        inv = np.float32(1.0) / np.float32(d)
        q = np.floor(kb * inv).astype(np.int64)   # fp32 product, rounded to nearest
        assert np.array_equal(q, kbi // d), d


def _sk(kind, wm, wn, stages, split, groups):
    c = hum.TileConfig()
    c.kind, c.wave_m, c.wave_n, c.waves_n, c.waves_k = kind, wm, wn, 1 if kind == 1 else 4, 8 if kind == 1 else 1
    c.stages, c.split_k, c.block_m, c.stream_k = stages, split, 16 * wm, groups
    return c


@pytest.mark.parametrize("cfg,why", [
    (dict(kind=0, wm=2, wn=2, stages=3, split=2, groups=64), "with split-K"),
    (dict(kind=1, wm=1, wn=1, stages=0, split=1, groups=64), "on the decode kernel"),
    (dict(kind=0, wm=2, wn=2, stages=3, split=1, groups=-1), "negative"),
    (dict(kind=0, wm=1, wn=4, stages=2, split=1, groups=64), "no such instance"),
])
def test_stream_k_configs_refused_before_launch(lib, cfg, why):
    """Stream-K configurations the library does not run are refused with
    HUM_ERR_UNSUPPORTED before anything is enqueued (null device pointers
    would fault if a kernel were launched)."""
    d = hum.make_desc("uint4", "group", 128, "bf16", 512, 1024, has_zero=True)
    c = _sk(**cfg)
    st = lib.hum_linear_ex(ctypes.byref(d), ctypes.c_void_p(256), 64, ctypes.c_void_p(256), None, None,
                           ctypes.c_void_p(256), ctypes.c_void_p(256), 1 << 30, ctypes.byref(c), None)
    assert st == 2, why


def test_stream_k_workspace_has_counter_header_and_slots(lib):
    """The workspace of a Stream-K call: the 64 KiB counter header, then two
    fp32 partial-tile slots per workgroup (after the INT row sums' offset
    region is added, the size only grows)."""
    d = hum.make_desc("uint4", "group", 128, "bf16", 512, 1024, has_zero=True)
    base = _sk(0, 2, 2, 3, 1, 0)
    sk = _sk(0, 2, 2, 3, 1, 64)
    b0 = hum.linear_workspace_bytes(d, 64, cfg=base)
    b1 = hum.linear_workspace_bytes(d, 64, cfg=sk)
    assert b1 - b0 >= 2 * 64 * 32 * 128 * 4
    assert b0 >= 64 << 10
