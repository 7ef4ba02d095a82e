"""Python binding of libhum (MI355X / gfx950 quantized GEMM).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libhum.so``; PyTorch provides device memory and the current
stream.  The names mirror the C ABI in ``include/hum.h``.  If the library is
not built, every entry point raises -- there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass

__all__ = [
    "HumError", "WeightDesc", "TileConfig", "lib_path", "load_library",
    "BF16", "F32", "INT4", "UINT4", "E2M1", "E4M3", "E8M0", "INT8",
    "INT3", "UINT3", "INT2", "UINT2", "INT1", "UINT1", "E2M3", "E3M2",
    "SCALE_TENSOR", "SCALE_CHANNEL", "SCALE_GROUP", "SCALE_BLOCK",
    "ACT_BF16", "ACT_FP8_TOKEN", "ACT_MXFP8", "ACT_MXFP4", "ACT_FP8_GROUP",
    "packed_weight_bytes", "prepare_weight", "dequant_weight", "quant_act",
    "select_config", "linear_workspace_bytes", "linear", "moe_workspace_bytes",
    "moe_gemm", "moe_align", "moe_reduce", "Workspace", "header_functions",
]

BF16, F32, INT4, UINT4, E2M1, E4M3, E8M0, INT8, INT3, UINT3, INT2, UINT2, INT1, UINT1, E2M3, E3M2 = range(16)
# bits per code of the packed-integer weight dtypes (LSB-first bit stream along K)
_BITS = {INT4: 4, UINT4: 4, E2M1: 4, INT3: 3, UINT3: 3, INT2: 2, UINT2: 2, INT1: 1, UINT1: 1, E2M3: 6, E3M2: 6}
KERNEL_TILE, KERNEL_STREAM, KERNEL_TILE32 = range(3)
SCALE_TENSOR, SCALE_CHANNEL, SCALE_GROUP, SCALE_BLOCK = range(4)
ACT_BF16, ACT_FP8_TOKEN, ACT_MXFP8, ACT_MXFP4, ACT_FP8_GROUP = range(5)

_HERE = os.path.dirname(os.path.abspath(__file__))
_HEADER = os.path.join(os.path.dirname(_HERE), "include", "hum.h")


def lib_path() -> str:
    return os.path.join(_HERE, "libhum.so")


class HumError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"hum status {status}: {msg}")
        self.status = status


class WeightDesc(ctypes.Structure):
    _fields_ = [
        ("weight_dtype", ctypes.c_int32), ("scale_gran", ctypes.c_int32),
        ("group_size", ctypes.c_int32), ("scale_dtype", ctypes.c_int32),
        ("has_zero_point", ctypes.c_int32), ("has_global_scale", ctypes.c_int32),
        ("act_fmt", ctypes.c_int32), ("num_experts", ctypes.c_int32),
        ("n", ctypes.c_int64), ("k", ctypes.c_int64),
    ]

    def __repr__(self):
        return ("WeightDesc(" + ", ".join(f"{f}={getattr(self, f)}" for f, _ in self._fields_) + ")")


class TileConfig(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("wave_m", ctypes.c_int32), ("wave_n", ctypes.c_int32), ("waves_n", ctypes.c_int32),
        ("waves_k", ctypes.c_int32), ("split_k", ctypes.c_int32), ("block_m", ctypes.c_int32),
        ("stages", ctypes.c_int32), ("stream_k", ctypes.c_int32),
    ]

    def as_tuple(self):
        return tuple(getattr(self, f) for f, _ in self._fields_)

    def __repr__(self):
        return "TileConfig(" + ", ".join(f"{f}={getattr(self, f)}" for f, _ in self._fields_) + ")"


_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t
_DP = ctypes.POINTER(WeightDesc)
_CP = ctypes.POINTER(TileConfig)

_SIGS = {
    "hum_last_error": (ctypes.c_char_p, []),
    "hum_packed_weight_bytes": (_SZ, [_DP]),
    "hum_select_config_ex": (_I32, [_DP, _I64, ctypes.c_uint32, _CP]),
    "hum_autotune_moe": (_I32, [_DP, _P, _DP, _P, _I64, _I32, _P, _P, _P, _P, _P, _SZ, _I32, ctypes.c_uint32, _CP,
                                ctypes.POINTER(ctypes.c_float), _P]),
    "hum_moe_gemm_masked": (_I32, [_DP, _P, _DP, _P, _I64, _I64, _P, _P, _P, _P, _SZ, _CP, _P]),
    "hum_moe_masked_workspace_bytes": (_SZ, [_DP, _DP, _I64, _I64, _CP]),
    "hum_autotune_linear": (_I32, [_DP, _P, _I64, _P, _P, _P, _P, _P, _SZ, _I32, ctypes.c_uint32, _CP,
                                   ctypes.POINTER(ctypes.c_float), _P]),
    "hum_moe_select_config": (_I32, [_DP, _DP, _I64, _I32, ctypes.c_uint32, _CP]),
    "hum_prepare_weight": (_I32, [_DP, _P, _P, _P, _P, _P, _SZ, _P]),
    "hum_dequant_weight": (_I32, [_DP, _P, _P, _P]),
    "hum_quant_act": (_I32, [_I32, _I64, _I64, _P, _I64, _P, _P, _P]),
    "hum_linear_workspace_bytes": (_SZ, [_DP, _I64]),
    "hum_linear_workspace_bytes_ex": (_SZ, [_DP, _I64, _CP]),
    "hum_linear": (_I32, [_DP, _P, _I64, _P, _P, _P, _P, _P, _SZ, _P]),
    "hum_linear_ex": (_I32, [_DP, _P, _I64, _P, _P, _P, _P, _P, _SZ, _CP, _P]),
    "hum_linear_noalloc": (_I32, [_DP, _P, _I64, _P, _P, _P, _P, _P]),
    "hum_prepare_workspace": (_I32, [_P, _SZ, _P]),
    "hum_select_config": (_I32, [_DP, _I64, _CP]),
    "hum_moe_workspace_bytes": (_SZ, [_DP, _DP, _I64, _I32]),
    "hum_moe_workspace_bytes_ex": (_SZ, [_DP, _DP, _I64, _I32, _CP]),
    "hum_moe_gemm": (_I32, [_DP, _P, _DP, _P, _I64, _I32, _P, _P, _P, _P, _P, _SZ, _P]),
    "hum_moe_gemm_ex": (_I32, [_DP, _P, _DP, _P, _I64, _I32, _P, _P, _P, _P, _P, _SZ, _CP, _P]),
    "hum_moe_align": (_I32, [_P, _I64, _I32, _I32, _I32, _P, _P, _P, _P]),
    "hum_moe_align_ex": (_I32, [_P, _I64, _I32, _I32, _I32, _P, _P, _P, _P, _SZ, _P]),
    "hum_moe_align_workspace_bytes": (_SZ, [_I64, _I32, _I32]),
    "hum_moe_reduce": (_I32, [_P, _P, _I64, _I32, _I64, _P, _P]),
    "hum_peak_probe": (_I32, [_I32, _I64, _P, _P, ctypes.POINTER(ctypes.c_double), _P]),
    "hum_moe_grouped_gemm_workspace_bytes": (_SZ, [_DP, _I32, _I32, _I64, _I32, _I64, _I32, _CP]),
    "hum_moe_grouped_gemm": (_I32, [_DP, _P, _I32, _I32, _I64, _I32, _P, _P, _P, _I64, _P, _I32, _P, _P, _P, _CP,
                                    _P, _SZ, _P]),
}


def header_functions() -> list[str]:
    """Names of the functions include/hum.h declares."""
    txt = open(_HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(hum_\w+)\s*\(", txt)))


def load_library():
    """Load libhum.so (raises if it is missing: the library has no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() "
                           "(quantized_gemm_packed_amd.build.build_library())")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise HumError(status, load_library().hum_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device=None):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _gpu(t, name):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _want(t, name, dtype, shape=None, numel=None):
    """Checks a tensor argument's dtype and shape (or element count) before
    anything is handed to the library: the kernels size their reads and
    writes from the description, not from the tensor."""
    if t is None:
        return
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() != int(numel):
        raise ValueError(f"{name} must hold {int(numel)} elements, got {t.numel()}")


def _same_device(*ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError(f"tensors on different devices: {sorted(str(d) for d in devs)}")


def _act_shapes(desc, m):
    """(codes dtype, codes shape, scales dtype, scales shape) of pre-quantized
    activations of `m` rows in desc's activation format."""
    import torch
    k = desc.k
    fmt = desc.act_fmt
    if fmt == ACT_FP8_TOKEN:
        return torch.uint8, (m, k), torch.float32, (m,)
    if fmt == ACT_MXFP8:
        return torch.uint8, (m, k), torch.uint8, (m, k // 32)
    if fmt == ACT_MXFP4:
        return torch.uint8, (m, k // 2), torch.uint8, (m, k // 32)
    if fmt == ACT_FP8_GROUP:
        return torch.uint8, (m, k), torch.float32, (m, k // 128)
    raise ValueError("bf16 activations take no a_scales")


def _check_linear_args(desc, packed, a, a_scales, bias, out):
    import torch
    if a is None or a.dim() != 2:
        raise ValueError("a must be a 2-D tensor [m, k]")
    m = a.shape[0]
    _want(packed, "packed", torch.uint8)
    if a_scales is None:
        _want(a, "a", torch.bfloat16, (m, desc.k))
    else:
        cd, cs, sd, ss = _act_shapes(desc, m)
        _want(a, "a (pre-quantized codes)", cd, cs)
        _want(a_scales, "a_scales", sd, ss)
    _want(bias, "bias", torch.bfloat16, (desc.n,))
    _want(out, "out", torch.bfloat16, (m, desc.n))
    _same_device(packed, a, a_scales, bias, out)


_DT = {"int4": INT4, "uint4": UINT4, "e2m1": E2M1, "e4m3": E4M3, "int8": INT8, "int3": INT3, "uint3": UINT3,
       "int2": INT2, "uint2": UINT2, "int1": INT1, "uint1": UINT1, "e2m3": E2M3, "e3m2": E3M2}
_GR = {"tensor": SCALE_TENSOR, "channel": SCALE_CHANNEL, "group": SCALE_GROUP, "block": SCALE_BLOCK}
_SD = {"bf16": BF16, "f32": F32, "e8m0": E8M0, "e4m3": E4M3}
_AF = {"bf16": ACT_BF16, "fp8_token": ACT_FP8_TOKEN, "mxfp8": ACT_MXFP8, "mxfp4": ACT_MXFP4,
       "fp8_group": ACT_FP8_GROUP}


def make_desc(weight_dtype, scale_gran, group_size, scale_dtype, n, k, num_experts=1,
              has_zero=False, has_global=False, act_fmt="bf16") -> WeightDesc:
    """Build a WeightDesc from names ("int4", "group", "bf16", ...)."""
    d = WeightDesc()
    d.weight_dtype = _DT.get(weight_dtype, weight_dtype)
    d.scale_gran = _GR.get(scale_gran, scale_gran)
    d.group_size = int(group_size)
    d.scale_dtype = _SD.get(scale_dtype, scale_dtype)
    d.has_zero_point = int(bool(has_zero))
    d.has_global_scale = int(bool(has_global))
    d.act_fmt = _AF.get(act_fmt, act_fmt)
    d.num_experts = int(num_experts)
    d.n = int(n)
    d.k = int(k)
    return d


__all__.append("make_desc")


def packed_weight_bytes(desc: WeightDesc) -> int:
    b = load_library().hum_packed_weight_bytes(ctypes.byref(desc))
    if b == 0:
        raise HumError(2, load_library().hum_last_error().decode())
    return b


def prepare_weight(desc: WeightDesc, codes, scales, zeros=None, global_scale=None, packed=None):
    """Canonical device tensors -> packed uint8 device tensor."""
    import torch
    e, n, k = desc.num_experts, desc.n, desc.k
    bits = _BITS.get(desc.weight_dtype, 8)
    _want(codes, "codes", torch.uint8, numel=e * n * k * bits // 8)
    if desc.scale_gran == SCALE_TENSOR:
        nsc = e
    elif desc.scale_gran == SCALE_CHANNEL:
        nsc = e * n
    elif desc.scale_gran == SCALE_BLOCK:
        g = max(desc.group_size, 1)
        nsc = e * (-(-n // g)) * (k // g)
    else:
        nsc = e * n * (k // max(desc.group_size, 1))
    sdt = {BF16: (torch.int16, torch.bfloat16, torch.uint16), F32: (torch.float32,),
           E8M0: (torch.uint8,), E4M3: (torch.uint8,)}.get(desc.scale_dtype, ())
    if scales is None or scales.dtype not in sdt:
        raise ValueError(f"scales must be one of {sdt} for scale dtype {desc.scale_dtype}")
    _want(scales, "scales", scales.dtype, numel=nsc)
    if desc.has_zero_point:
        _want(zeros, "zeros", torch.uint8, numel=nsc)
    if desc.has_global_scale:
        _want(global_scale, "global_scale", torch.float32, numel=e)
    _same_device(codes, scales, zeros, global_scale)
    for t, nm in ((codes, "codes"), (scales, "scales"), (zeros, "zeros"), (global_scale, "global_scale")):
        _gpu(t, nm)
    nb = packed_weight_bytes(desc)
    if packed is None:
        packed = torch.empty(nb, dtype=torch.uint8, device=codes.device)
    _want(packed, "packed", torch.uint8)
    _gpu(packed, "packed")
    _check(load_library().hum_prepare_weight(ctypes.byref(desc), _ptr(codes), _ptr(scales), _ptr(zeros),
                                             _ptr(global_scale), _ptr(packed), packed.numel(),
                                             _stream(codes.device)))
    return packed


def dequant_weight(desc: WeightDesc, packed):
    import torch
    _gpu(packed, "packed")
    out = torch.empty((desc.num_experts, desc.n, desc.k), dtype=torch.float32, device=packed.device)
    _check(load_library().hum_dequant_weight(ctypes.byref(desc), _ptr(packed), _ptr(out), _stream(packed.device)))
    return out


def quant_act(act_fmt, x):
    """bf16 x [m, k] -> (codes, scales): E4M3 codes uint8 [m, k], or for
    MXFP4 E2M1 codes two per byte uint8 [m, k/2] (even k in the low nibble)."""
    import torch
    if x is None or x.dim() != 2:
        raise ValueError("x must be a 2-D tensor [m, k]")
    _want(x, "x", torch.bfloat16)
    _gpu(x, "x")
    fmt = _AF.get(act_fmt, act_fmt)
    m, k = x.shape
    q = torch.empty((m, k // 2 if fmt == ACT_MXFP4 else k), dtype=torch.uint8, device=x.device)
    if fmt == ACT_FP8_TOKEN:
        s = torch.empty((m,), dtype=torch.float32, device=x.device)
    elif fmt == ACT_FP8_GROUP:
        s = torch.empty((m, k // 128), dtype=torch.float32, device=x.device)
    else:
        s = torch.empty((m, k // 32), dtype=torch.uint8, device=x.device)
    _check(load_library().hum_quant_act(fmt, m, k, _ptr(x), k, _ptr(q), _ptr(s), _stream(x.device)))
    return q, s


SELECT_BATCH_INVARIANT = 1


def select_config(desc: WeightDesc, m: int, batch_invariant: bool = False) -> TileConfig:
    c = TileConfig()
    if batch_invariant:
        _check(load_library().hum_select_config_ex(ctypes.byref(desc), int(m), SELECT_BATCH_INVARIANT,
                                                   ctypes.byref(c)))
    else:
        _check(load_library().hum_select_config(ctypes.byref(desc), int(m), ctypes.byref(c)))
    return c


SELECT_MOE_GATE_UP = 2


def moe_select_config(w13: WeightDesc, w2: WeightDesc, t: int, topk: int, batch_invariant: bool = False,
                      gate_up: bool = False) -> TileConfig:
    """The MoE selector's configuration: the down GEMM's, or with gate_up the
    gate_up GEMM's."""
    c = TileConfig()
    flags = (SELECT_BATCH_INVARIANT if batch_invariant else 0) | (SELECT_MOE_GATE_UP if gate_up else 0)
    _check(load_library().hum_moe_select_config(ctypes.byref(w13), ctypes.byref(w2), int(t), int(topk),
                                                flags, ctypes.byref(c)))
    return c


def linear_workspace_bytes(desc: WeightDesc, m: int, cfg: TileConfig | None = None) -> int:
    lib = load_library()
    if cfg is None:
        return lib.hum_linear_workspace_bytes(ctypes.byref(desc), int(m))
    return lib.hum_linear_workspace_bytes_ex(ctypes.byref(desc), int(m), ctypes.byref(cfg))


class Workspace:
    """A device buffer that grows on demand (its contents need no
    initialisation).  One buffer serves any sequence of calls on one stream;
    calls that may overlap in time (on different streams) need different
    workspaces."""

    def __init__(self, device):
        self.device = device
        self.buf = None

    def get(self, nbytes: int):
        import torch
        if nbytes == 0:
            return None
        if self.buf is None or self.buf.numel() < nbytes:
            if self.buf is not None:
                # the old buffer may still be read by work queued on the
                # current stream: keep the allocator from reusing it early
                self.buf.record_stream(torch.cuda.current_stream(self.device))
            self.buf = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=self.device)
        return self.buf


_WS: dict = {}


def _workspace(device):
    """The binding's own workspace for calls on `device`'s current stream:
    one per (device, stream), so calls on two streams never share scratch."""
    import torch
    d = torch.device(device)
    idx = d.index if d.index is not None else torch.cuda.current_device()
    key = (idx, torch.cuda.current_stream(idx).cuda_stream)
    if key not in _WS:
        _WS[key] = Workspace(torch.device("cuda", idx))
    return _WS[key]


def linear(desc: WeightDesc, packed, a, a_scales=None, bias=None, out=None, cfg: TileConfig | None = None,
           workspace=None, batch_invariant: bool = False):
    """bf16 out [m, n] = A @ W^T (+ bias).  batch_invariant: every row's
    result independent of m (the library's invariant configuration)."""
    import torch
    _check_linear_args(desc, packed, a, a_scales, bias, out)
    for t, nm in ((packed, "packed"), (a, "a"), (a_scales, "a_scales"), (bias, "bias"), (out, "out")):
        _gpu(t, nm)
    m = a.shape[0]
    if batch_invariant and cfg is None:
        cfg = select_config(desc, m, batch_invariant=True)
    if out is None:
        out = torch.empty((m, desc.n), dtype=torch.bfloat16, device=a.device)
    need = linear_workspace_bytes(desc, m, cfg)
    ws = workspace if workspace is not None else _workspace(a.device).get(need)
    wsb = 0 if ws is None else ws.numel()
    lib = load_library()
    _check(lib.hum_linear_ex(ctypes.byref(desc), _ptr(packed), m, _ptr(a), _ptr(a_scales), _ptr(bias), _ptr(out),
                             _ptr(ws), wsb, None if cfg is None else ctypes.byref(cfg), _stream(a.device)))
    return out


def linear_noalloc(desc: WeightDesc, packed, a, out, a_scales=None, bias=None):
    """hum_linear_noalloc: the library's static scratch array instead of a
    workspace; `out` (bf16 [m, n]) must be given, so nothing is allocated."""
    _check_linear_args(desc, packed, a, a_scales, bias, out)
    if out is None:
        raise ValueError("out must be given (the no-allocation call allocates nothing)")
    for t, nm in ((packed, "packed"), (a, "a"), (a_scales, "a_scales"), (bias, "bias"), (out, "out")):
        _gpu(t, nm)
    _check(load_library().hum_linear_noalloc(ctypes.byref(desc), _ptr(packed), a.shape[0], _ptr(a), _ptr(a_scales),
                                             _ptr(bias), _ptr(out), _stream(a.device)))
    return out


def autotune_linear(desc: WeightDesc, packed, a, a_scales=None, bias=None, out=None, workspace=None,
                    iters: int = 10, batch_invariant: bool = False):
    """Time every compiled configuration on these buffers (on the device) ->
    (fastest TileConfig, its µs per call).  `out`, if given, ends holding
    the winner's result.  The workspace defaults to the largest any
    candidate needs (a tile configuration with split-K 16)."""
    import torch
    _check_linear_args(desc, packed, a, a_scales, bias, out)
    for t, nm in ((packed, "packed"), (a, "a"), (a_scales, "a_scales"), (bias, "bias"), (out, "out")):
        _gpu(t, nm)
    m = a.shape[0]
    if out is None:
        out = torch.empty((m, desc.n), dtype=torch.bfloat16, device=a.device)
    if workspace is None:
        big = select_config(desc, max(m, 17))
        big.split_k = 16
        workspace = _workspace(a.device).get(linear_workspace_bytes(desc, m, big))
    wsb = 0 if workspace is None else workspace.numel()
    best = TileConfig()
    us = ctypes.c_float()
    _check(load_library().hum_autotune_linear(ctypes.byref(desc), _ptr(packed), m, _ptr(a), _ptr(a_scales),
                                              _ptr(bias), _ptr(out), _ptr(workspace), wsb, int(iters),
                                              SELECT_BATCH_INVARIANT if batch_invariant else 0,
                                              ctypes.byref(best), ctypes.byref(us), _stream(a.device)))
    return best, us.value


def _check_moe_args(w13, packed_w13, packed_w2, x, topk_ids, topk_weights, out):
    import torch
    if topk_ids is None or topk_ids.dim() != 2:
        raise ValueError("topk_ids must be a 2-D tensor [T, topk]")
    t, k = topk_ids.shape
    _want(topk_ids, "topk_ids", torch.int32)
    _want(topk_weights, "topk_weights", torch.float32, (t, k))
    _want(x, "x", torch.bfloat16, (t, w13.k))
    _want(out, "out", torch.bfloat16, (t, w13.k))
    _want(packed_w13, "packed_w13", torch.uint8)
    _want(packed_w2, "packed_w2", torch.uint8)
    _same_device(packed_w13, packed_w2, x, topk_ids, topk_weights, out)


def moe_workspace_bytes(w13: WeightDesc, w2: WeightDesc, t: int, topk: int, cfg: TileConfig | None = None) -> int:
    lib = load_library()
    if cfg is None:
        return lib.hum_moe_workspace_bytes(ctypes.byref(w13), ctypes.byref(w2), int(t), int(topk))
    return lib.hum_moe_workspace_bytes_ex(ctypes.byref(w13), ctypes.byref(w2), int(t), int(topk), ctypes.byref(cfg))


def moe_gemm(w13: WeightDesc, packed_w13, w2: WeightDesc, packed_w2, x, topk_ids, topk_weights, out=None,
             cfg: TileConfig | None = None, workspace=None, batch_invariant: bool = False):
    """bf16 out [T, H] of the MoE expert layer.  batch_invariant: every
    token's result independent of the other tokens of the call."""
    import torch
    _check_moe_args(w13, packed_w13, packed_w2, x, topk_ids, topk_weights, out)
    for t, nm in ((packed_w13, "packed_w13"), (packed_w2, "packed_w2"), (x, "x"), (topk_ids, "topk_ids"),
                  (topk_weights, "topk_weights"), (out, "out")):
        _gpu(t, nm)
    t_count, topk = topk_ids.shape
    if batch_invariant and cfg is None:
        cfg = moe_select_config(w13, w2, t_count, topk, batch_invariant=True)
    if out is None:
        out = torch.empty((t_count, w13.k), dtype=torch.bfloat16, device=x.device)
    need = moe_workspace_bytes(w13, w2, t_count, topk, cfg)
    if need == 0 and t_count > 0:
        raise HumError(2, load_library().hum_last_error().decode())
    ws = workspace if workspace is not None else _workspace(x.device).get(need)
    wsb = 0 if ws is None else ws.numel()
    _check(load_library().hum_moe_gemm_ex(ctypes.byref(w13), _ptr(packed_w13), ctypes.byref(w2), _ptr(packed_w2),
                                          t_count, topk, _ptr(x), _ptr(topk_ids), _ptr(topk_weights), _ptr(out),
                                          _ptr(ws), wsb, None if cfg is None else ctypes.byref(cfg),
                                          _stream(x.device)))
    return out


def autotune_moe(w13: WeightDesc, packed_w13, w2: WeightDesc, packed_w2, x, topk_ids, topk_weights, out=None,
                 workspace=None, iters: int = 5, batch_invariant: bool = False):
    """Time every compiled MoE configuration on these buffers (on the device)
    -> (fastest TileConfig, its µs per layer call).  `out`, if given, ends
    holding the winner's result.  The workspace defaults to what the largest
    expert block (128 rows) needs."""
    import torch
    _check_moe_args(w13, packed_w13, packed_w2, x, topk_ids, topk_weights, out)
    for t, nm in ((packed_w13, "packed_w13"), (packed_w2, "packed_w2"), (x, "x"), (topk_ids, "topk_ids"),
                  (topk_weights, "topk_weights"), (out, "out")):
        _gpu(t, nm)
    t_count, topk = topk_ids.shape
    if out is None:
        out = torch.empty((t_count, w13.k), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        big = TileConfig()
        big.kind, big.wave_m, big.wave_n, big.waves_n, big.waves_k, big.split_k, big.block_m = 0, 8, 4, 4, 1, 1, 128
        workspace = _workspace(x.device).get(moe_workspace_bytes(w13, w2, t_count, topk, big))
    best = TileConfig()
    us = ctypes.c_float()
    _check(load_library().hum_autotune_moe(ctypes.byref(w13), _ptr(packed_w13), ctypes.byref(w2), _ptr(packed_w2),
                                           t_count, topk, _ptr(x), _ptr(topk_ids), _ptr(topk_weights), _ptr(out),
                                           _ptr(workspace), workspace.numel(), int(iters),
                                           SELECT_BATCH_INVARIANT if batch_invariant else 0, ctypes.byref(best),
                                           ctypes.byref(us), _stream(x.device)))
    return best, us.value


def moe_masked_workspace_bytes(w13: WeightDesc, w2: WeightDesc, max_m: int, expected_m: int,
                               cfg: TileConfig | None = None) -> int:
    lib = load_library()
    b = lib.hum_moe_masked_workspace_bytes(ctypes.byref(w13), ctypes.byref(w2), int(max_m), int(expected_m),
                                           None if cfg is None else ctypes.byref(cfg))
    if b == 0:
        raise HumError(1, lib.hum_last_error().decode())
    return b


def moe_gemm_masked(w13: WeightDesc, packed_w13, w2: WeightDesc, packed_w2, x, expert_num_tokens, expected_m: int,
                    out=None, cfg: TileConfig | None = None, workspace=None):
    """grouped_masked layout: x bf16 [E, max_m, H], expert_num_tokens int32
    [E] (device) -> bf16 [E, max_m, H]; rows past an expert's count are left
    as they were in `out`."""
    import torch
    if x is None or x.dim() != 3:
        raise ValueError("x must be a 3-D tensor [E, max_m, H]")
    e, max_m, h = x.shape
    _want(x, "x", torch.bfloat16, (w13.num_experts, max_m, w13.k))
    _want(expert_num_tokens, "expert_num_tokens", torch.int32, (w13.num_experts,))
    _want(out, "out", torch.bfloat16, (w13.num_experts, max_m, w13.k))
    _want(packed_w13, "packed_w13", torch.uint8)
    _want(packed_w2, "packed_w2", torch.uint8)
    _same_device(packed_w13, packed_w2, x, expert_num_tokens, out)
    for t, nm in ((packed_w13, "packed_w13"), (packed_w2, "packed_w2"), (x, "x"),
                  (expert_num_tokens, "expert_num_tokens"), (out, "out")):
        _gpu(t, nm)
    if out is None:
        out = torch.zeros((e, max_m, h), dtype=torch.bfloat16, device=x.device)
    lib = load_library()
    need = moe_masked_workspace_bytes(w13, w2, max_m, expected_m, cfg)
    ws = workspace if workspace is not None else _workspace(x.device).get(need)
    wsb = 0 if ws is None else ws.numel()
    _check(lib.hum_moe_gemm_masked(ctypes.byref(w13), _ptr(packed_w13), ctypes.byref(w2), _ptr(packed_w2), max_m,
                                   int(expected_m), _ptr(x), _ptr(expert_num_tokens), _ptr(out), _ptr(ws), wsb,
                                   None if cfg is None else ctypes.byref(cfg), _stream(x.device)))
    return out


def moe_align(topk_ids, num_experts: int, block_m: int, multi_workgroup: bool = False):
    """-> (sorted int32 [T*topk + E*(block_m-1)], offsets int32 [E+1], counts int32 [E]).
    multi_workgroup: give the sort scratch so that large tables are shared by
    many workgroups (the layer's own path); the result is the same."""
    import torch
    if topk_ids is None or topk_ids.dim() != 2:
        raise ValueError("topk_ids must be a 2-D tensor [T, topk]")
    _want(topk_ids, "topk_ids", torch.int32)
    _gpu(topk_ids, "topk_ids")
    t, k = topk_ids.shape
    cap = t * k + num_experts * (block_m - 1)
    dev = topk_ids.device
    srt = torch.empty(cap, dtype=torch.int32, device=dev)
    off = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
    cnt = torch.empty(num_experts, dtype=torch.int32, device=dev)
    if multi_workgroup:
        lib = load_library()
        nb = lib.hum_moe_align_workspace_bytes(t, k, num_experts)
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
        _check(lib.hum_moe_align_ex(_ptr(topk_ids), t, k, num_experts, block_m, _ptr(srt), _ptr(off), _ptr(cnt),
                                    _ptr(ws), nb, _stream(dev)))
        return srt, off, cnt
    _check(load_library().hum_moe_align(_ptr(topk_ids), t, k, num_experts, block_m, _ptr(srt), _ptr(off), _ptr(cnt),
                                        _stream(dev)))
    return srt, off, cnt


def moe_reduce(y, topk_weights):
    """y bf16 [T*topk, H], w f32 [T, topk] -> bf16 [T, H]."""
    import torch
    if topk_weights is None or topk_weights.dim() != 2 or y is None or y.dim() != 2:
        raise ValueError("y must be [T*topk, H] and topk_weights [T, topk]")
    t, k = topk_weights.shape
    h = y.shape[1]
    _want(topk_weights, "topk_weights", torch.float32)
    _want(y, "y", torch.bfloat16, (t * k, h))
    _same_device(y, topk_weights)
    _gpu(y, "y")
    _gpu(topk_weights, "topk_weights")
    out = torch.empty((t, h), dtype=torch.bfloat16, device=y.device)
    _check(load_library().hum_moe_reduce(_ptr(y), _ptr(topk_weights), t, k, h, _ptr(out), _stream(y.device)))
    return out


MOE_A_GATHER, MOE_A_SORTED = range(2)
MOE_EPI_NONE, MOE_EPI_SCATTER, MOE_EPI_SWIGLU_BF16, MOE_EPI_SWIGLU_MXFP8, MOE_EPI_SWIGLU_MXFP4 = range(5)
_MOE_EPI = {"none": MOE_EPI_NONE, "scatter": MOE_EPI_SCATTER, "swiglu_bf16": MOE_EPI_SWIGLU_BF16,
            "swiglu_mxfp8": MOE_EPI_SWIGLU_MXFP8, "swiglu_mxfp4": MOE_EPI_SWIGLU_MXFP4}


def moe_grouped_gemm(w: WeightDesc, packed, a, sorted_ids, offsets, block_m: int, num_tokens: int, topk: int,
                     a_mode: str = "gather", epilogue: str = "none", a_scales=None, cfg: TileConfig | None = None,
                     keep_swiglu_f32: bool = False, workspace=None):
    """One grouped GEMM stage over rows sorted by expert (hum_moe_grouped_gemm).
    Returns out, or (out, out_scales) for the MX SwiGLU epilogues, plus the
    fp32 SwiGLU values last when keep_swiglu_f32."""
    import torch
    if sorted_ids is None or sorted_ids.dim() != 1:
        raise ValueError("sorted_ids must be a 1-D int32 tensor")
    _want(sorted_ids, "sorted_ids", torch.int32)
    _want(offsets, "offsets", torch.int32, (w.num_experts + 1,))
    _want(packed, "packed", torch.uint8)
    mode = {"gather": MOE_A_GATHER, "sorted": MOE_A_SORTED}[a_mode]
    epi = _MOE_EPI[epilogue]
    slen = sorted_ids.shape[0]
    rows = num_tokens if mode == MOE_A_GATHER else slen
    if w.act_fmt == ACT_BF16:
        _want(a, "a", torch.bfloat16, (rows, w.k))
    else:
        cd, cs, sd, ss = _act_shapes(w, rows)
        _want(a, "a", cd, cs)
        _want(a_scales, "a_scales", sd, ss)
    _same_device(packed, a, a_scales, sorted_ids, offsets)
    for t, nm in ((packed, "packed"), (a, "a"), (a_scales, "a_scales"), (sorted_ids, "sorted_ids"),
                  (offsets, "offsets")):
        _gpu(t, nm)
    dev = a.device
    n = w.n
    out_s = None
    if epi == MOE_EPI_NONE:
        out = torch.empty((slen, n), dtype=torch.bfloat16, device=dev)
    elif epi == MOE_EPI_SCATTER:
        out = torch.empty((num_tokens * topk, n), dtype=torch.bfloat16, device=dev)
    elif epi == MOE_EPI_SWIGLU_BF16:
        out = torch.empty((slen, n // 2), dtype=torch.bfloat16, device=dev)
    elif epi == MOE_EPI_SWIGLU_MXFP8:
        out = torch.empty((slen, n // 2), dtype=torch.uint8, device=dev)
        out_s = torch.empty((slen, n // 64), dtype=torch.uint8, device=dev)
    else:
        out = torch.empty((slen, n // 4), dtype=torch.uint8, device=dev)
        out_s = torch.empty((slen, n // 64), dtype=torch.uint8, device=dev)
    f32 = torch.empty((slen, n // 2), dtype=torch.float32, device=dev) if keep_swiglu_f32 else None
    lib = load_library()
    cp = None if cfg is None else ctypes.byref(cfg)
    need = lib.hum_moe_grouped_gemm_workspace_bytes(ctypes.byref(w), mode, epi, num_tokens, topk, slen, block_m, cp)
    if need == 0:
        raise HumError(2, lib.hum_last_error().decode())
    ws = workspace if workspace is not None else _workspace(dev).get(need)
    _check(lib.hum_moe_grouped_gemm(ctypes.byref(w), _ptr(packed), mode, epi, num_tokens, topk, _ptr(a),
                                    _ptr(a_scales), _ptr(sorted_ids), slen, _ptr(offsets), block_m, _ptr(out),
                                    _ptr(out_s), _ptr(f32), cp, _ptr(ws), ws.numel(), _stream(dev)))
    res = (out,) if out_s is None else (out, out_s)
    if keep_swiglu_f32:
        res = res + (f32,)
    return res[0] if len(res) == 1 else res


(PEAK_HBM_READ, PEAK_MFMA_BF16, PEAK_MFMA_FP8, PEAK_MFMA_FP4, PEAK_MFMA_FP8_FP4, PEAK_MFMA32_BF16, PEAK_MFMA32_FP8,
 PEAK_MFMA32_FP4, PEAK_MFMA32_FP8_FP4) = range(9)


def peak_probe(kind: int, n: int, buf=None, sink=None):
    """Enqueue one device peak probe (measurement only) -> (sink, work):
    bytes read for PEAK_HBM_READ, flops for the matrix-instruction loops."""
    import torch
    if sink is None:
        sink = torch.empty(2048 * 256, dtype=torch.float32, device="cuda")
    work = ctypes.c_double()
    _check(load_library().hum_peak_probe(int(kind), int(n), _ptr(buf), _ptr(sink), ctypes.byref(work),
                                         _stream(sink.device)))
    return sink, work.value


@dataclass
class _Version:
    arch: str = "gfx950"


version = _Version()
