"""GPU: the no-allocation entry point hum_linear_noalloc (its workspace is
the library's static device scratch array) called through the C ABI,
against hum_linear with a caller workspace -- two calls in a row, the
second with fewer rows, so the second runs over what the first left in the
array.  The two entry points run the same kernels with the same
configuration, so their outputs must agree bit for bit."""
import ctypes

import numpy as np
import pytest
import torch

import quantized_gemm_packed_amd as hum
import synth
from gpu_util import bf16_bits_of, descs, dev, prepare

pytestmark = pytest.mark.gpu


def _noalloc(lib, d, packed, a, a_scales, out):
    st = lib.hum_linear_noalloc(ctypes.byref(d), ctypes.c_void_p(packed.data_ptr()), a.shape[0],
                                ctypes.c_void_p(a.data_ptr()),
                                None if a_scales is None else ctypes.c_void_p(a_scales.data_ptr()), None,
                                ctypes.c_void_p(out.data_ptr()),
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lib.hum_last_error()


CASES = [
    # (name, weight desc args, n, k, (m1, m2)): Stream-K tiles, whose tile
    # counters live in the array's header, then the decode kernel with
    # split-K partials; per-token FP8 activations quantized into the
    # scratch; INT tiles with row sums, Stream-K at both sizes
    ("uint4_zp_g128_decode", ("uint4", "group", 128, "bf16"), dict(zero=True), 4096, 4096, (16, 5)),
    ("fp8_token", ("e4m3", "channel", 0, "f32"), dict(act="fp8_token"), 2048, 2048, (64, 3)),
    ("uint4_zp_g128_tile", ("uint4", "group", 128, "bf16"), dict(zero=True), 2048, 4096, (200, 33)),
]


@pytest.mark.parametrize("name,wargs,kw,n,k,ms", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_linear_two_calls(name, wargs, kw, n, k, ms):
    lib = hum.load_library()
    wd, gran, gs, sd = wargs
    hd, _ = descs(wd, gran, gs, sd, 1, n, k, **kw)
    if wd == "e4m3":
        w = synth.dense_w8a8(synth.seed_for(90), 1, n, k)
    else:
        w = synth.dense_w4a16(synth.seed_for(91), 1, n, k, group=gs, asym=True)
    packed = prepare(hd, w, sd)
    g = synth.rng(92)
    for m in ms:
        print(f"case noalloc {name} m={m}", flush=True)
        x = dev(synth.bf16_normal(g, (m, k)))
        ref = hum.linear(hd, packed, x)
        out = torch.full((m, n), 7.0, dtype=torch.bfloat16, device="cuda")
        _noalloc(lib, hd, packed, x, None, out)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits_of(out), bf16_bits_of(ref)), f"{name} m={m}"


def test_noalloc_refuses_oversized_call():
    lib = hum.load_library()
    hd, _ = descs("e4m3", "channel", 0, "f32", 1, 512, 8192, act="fp8_token")
    m = 8192                       # 64 MiB of quantized activations > the array
    p = ctypes.c_void_p(16)        # never dereferenced: refused before any launch
    st = lib.hum_linear_noalloc(ctypes.byref(hd), p, m, p, None, None, p, None)
    assert st == 3 and b"scratch" in lib.hum_last_error()
