"""GPU: parity at the full benchmark sizes, in the launch configuration the
bench times (selector choices), on outputs the oracle computes one sample at
a time: sampled rows x sampled columns for the dense layers, sampled tokens
for the MoE layers (a token's output depends only on its own row)."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_packed_amd as hum
import synth
from gpu_util import assert_tol, dev, prepare, descs

pytestmark = pytest.mark.gpu


def _sample(rng, n, count):
    return np.sort(rng.choice(n, size=min(count, n), replace=False))


@pytest.fixture(scope="module")
def dense_w4a16_full():
    n = k = 8192
    case = synth.dense_w4a16(synth.seed_for(2), 1, n, k, group=128, asym=True)
    hd, od = descs("uint4", "group", 128, "bf16", 1, n, k, zero=True)
    return case, hd, od, prepare(hd, case, "bf16")


@pytest.mark.parametrize("m", [1, 64, 4096])
def test_dense_w4a16_full_size(dense_w4a16_full, m):
    case, hd, od, packed = dense_w4a16_full
    n = k = 8192
    xb = synth.bf16_normal(synth.rng(synth.seed_for(2, 1)), (m, k))
    print(f"case dense w4a16 m={m}", flush=True)
    out = hum.linear(hd, packed, dev(xb))
    torch.cuda.synchronize()
    g = synth.rng(9000 + m)
    rows, cols = _sample(g, m, 16), _sample(g, n, 256)
    sub = oracle.gemm.WeightDesc("uint4", "group", 128, "bf16", True, False, 1, len(cols), k)
    ref = oracle.gemm.linear(sub, oracle.formats.decode_bf16(xb[rows]), case["codes"][:, cols],
                             case["scales"][:, cols], case["zeros"][:, cols])
    got = out[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()]
    assert_tol(got, ref, f"m={m}")


@pytest.mark.parametrize("m", [1, 128, 4096])
def test_dense_w8a8_full_size(m):
    n, k = 7168, 2048
    case = synth.dense_w8a8(synth.seed_for(3), 1, n, k)
    hd, od = descs("e4m3", "channel", 0, "f32", 1, n, k, act="fp8_token")
    packed = prepare(hd, case, "f32")
    xb = synth.bf16_normal(synth.rng(synth.seed_for(3, 1)), (m, k))
    out = hum.linear(hd, packed, dev(xb))
    torch.cuda.synchronize()
    g = synth.rng(9100 + m)
    rows, cols = _sample(g, m, 32), _sample(g, n, 512)
    q, s = oracle.quant.quant_fp8_per_token(oracle.formats.decode_bf16(xb[rows]).astype(np.float32))
    ref = oracle.gemm.linear_fp8_e4m3(oracle.quant.dequant_fp8_per_token(q, s), case["codes"][0, cols],
                                      case["scales"][0, cols, 0])
    got = out[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()]
    assert_tol(got, ref, f"m={m}")


@pytest.fixture(scope="module")
def moe_full():
    e, h, inter = 128, 4096, 1024
    w13 = synth.moe_weights_mxfp4(synth.seed_for(4), e, 2 * inter, h)
    w2 = synth.moe_weights_mxfp4(synth.seed_for(4, 1), e, h, inter)
    packs = {}
    for act in ("bf16", "mxfp8"):
        d13, o13 = descs("e2m1", "group", 32, "e8m0", e, 2 * inter, h, act=act)
        d2, o2 = descs("e2m1", "group", 32, "e8m0", e, h, inter, act=act)
        packs[act] = (d13, o13, d2, o2)
    d13, _, d2, _ = packs["bf16"]
    p13, p2 = prepare(d13, w13, "e8m0"), prepare(d2, w2, "e8m0")
    return w13, w2, packs, p13, p2


@pytest.mark.parametrize("act,t,zipf", [("bf16", 1, None), ("bf16", 4096, None), ("mxfp8", 1, 1.1),
                                        ("mxfp8", 8192, 1.1)])
def test_moe_full_size(moe_full, act, t, zipf):
    w13, w2, packs, p13, p2 = moe_full
    d13, o13, d2, o2 = packs[act]
    cfgno = 4 if act == "bf16" else 5
    ids, wts = synth.routing(synth.seed_for(cfgno, t), t, 128, 8, zipf_s=zipf)
    xb = synth.bf16_normal(synth.rng(synth.seed_for(cfgno, 100 + t)), (t, 4096))
    print(f"case moe act={act} t={t}", flush=True)
    out = hum.moe_gemm(d13, p13, d2, p2, dev(xb), dev(ids), dev(wts))
    torch.cuda.synchronize()
    toks = _sample(synth.rng(9200 + t), t, 2)
    ref = oracle.moe.moe_forward(o13, w13, o2, w2, xb[toks], ids[toks], wts[toks], act)
    got = out[torch.from_numpy(toks).cuda()]
    assert_tol(got, ref, f"act={act} t={t}")
