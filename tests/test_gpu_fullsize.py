"""GPU: parity at the full benchmark sizes, in the launch configuration the
bench times (selector choices).  Dense layers: the whole output of every
sweep size against the oracle.  MoE layers: at least 256 tokens of every
sweep size (all of them when fewer), among them every token routed into the
first block of the most loaded expert and a token of an expert that
receives a single row (a token's output depends only on its own routing)."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_packed_amd as hum
import synth
from gpu_util import assert_tol, dev, prepare, descs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dense_w4a16_full():
    n = k = 8192
    case = synth.dense_w4a16(synth.seed_for(2), 1, n, k, group=128, asym=True)
    hd, od = descs("uint4", "group", 128, "bf16", 1, n, k, zero=True)
    return case, hd, od, prepare(hd, case, "bf16")


def test_dense_w4a16_tiny_full():
    """M = 16, N = 512, K = 1024, INT4 symmetric, group 128: whole output."""
    case = synth.dense_w4a16(synth.seed_for(1), 16, 512, 1024, group=128)
    hd, od = descs("int4", "group", 128, "bf16", 1, 512, 1024)
    out = hum.linear(hd, prepare(hd, case, "bf16"), dev(case["x"]))
    torch.cuda.synchronize()
    ref = oracle.gemm.linear(od, oracle.formats.decode_bf16(case["x"]), case["codes"], case["scales"])
    assert_tol(out, ref, "tiny")


@pytest.mark.parametrize("m", synth.DENSE_SWEEP_M)
def test_dense_w4a16_full_size(dense_w4a16_full, m):
    case, hd, od, packed = dense_w4a16_full
    k = 8192
    xb = synth.bf16_normal(synth.rng(synth.seed_for(2, 1)), (m, k))
    print(f"case dense w4a16 full m={m}", flush=True)
    out = hum.linear(hd, packed, dev(xb))
    torch.cuda.synchronize()
    ref = oracle.gemm.linear(od, oracle.formats.decode_bf16(xb), case["codes"], case["scales"], case["zeros"])
    assert_tol(out, ref, f"m={m}")


@pytest.mark.parametrize("m", synth.FP8_SWEEP_M)
def test_dense_w8a8_full_size(m):
    n, k = 7168, 2048
    case = synth.dense_w8a8(synth.seed_for(3), 1, n, k)
    hd, od = descs("e4m3", "channel", 0, "f32", 1, n, k, act="fp8_token")
    packed = prepare(hd, case, "f32")
    xb = synth.bf16_normal(synth.rng(synth.seed_for(3, 1)), (m, k))
    print(f"case dense w8a8 full m={m}", flush=True)
    out = hum.linear(hd, packed, dev(xb))
    torch.cuda.synchronize()
    q, s = oracle.quant.quant_fp8_per_token(oracle.formats.decode_bf16(xb).astype(np.float32))
    ref = oracle.gemm.linear_fp8_e4m3(oracle.quant.dequant_fp8_per_token(q, s), case["codes"][0],
                                      case["scales"][0, :, 0])
    assert_tol(out, ref, f"m={m}")


class _Dequant:
    """Per-expert dequantized weights, computed once by the oracle and kept
    in float32 (MXFP4 values are E2M1 x 2^e with e in [-8, -4]: exact in
    float32), shared by every MoE case of the module."""

    def __init__(self, o13, w13, o2, w2):
        self.args = (o13, w13, o2, w2)
        self.cache = {}

    def __call__(self, e):
        if e not in self.cache:
            o13, w13, o2, w2 = self.args
            gu = oracle.gemm.dequant_weight(o13, w13["codes"], w13["scales"], experts=[e])[0]
            dn = oracle.gemm.dequant_weight(o2, w2["codes"], w2["scales"], experts=[e])[0]
            g32, d32 = gu.astype(np.float32), dn.astype(np.float32)
            assert np.array_equal(g32, gu) and np.array_equal(d32, dn)
            self.cache[e] = (g32, d32)
        return self.cache[e]


@pytest.fixture(scope="module")
def moe_full():
    e, h, inter = 128, 4096, 1024
    w13 = synth.moe_weights_mxfp4(synth.seed_for(4), e, 2 * inter, h)
    w2 = synth.moe_weights_mxfp4(synth.seed_for(4, 1), e, h, inter)
    packs = {}
    for act in ("bf16", "mxfp8", "mxfp4"):
        d13, o13 = descs("e2m1", "group", 32, "e8m0", e, 2 * inter, h, act=act)
        d2, o2 = descs("e2m1", "group", 32, "e8m0", e, h, inter, act=act)
        packs[act] = (d13, o13, d2, o2)
    d13, o13, d2, o2 = packs["bf16"]
    p13, p2 = prepare(d13, w13, "e8m0"), prepare(d2, w2, "e8m0")
    return w13, w2, packs, p13, p2, _Dequant(o13, w13, o2, w2)


def _tokens(ids, t, bm, count, seed):
    """count tokens (all when t <= count): every token routed into the first
    bm-row block of the most loaded expert, one token of a single-row expert
    (if any), the rest drawn at random."""
    if t <= count:
        return np.arange(t)
    flat = ids.reshape(-1)
    cnt = np.bincount(flat, minlength=128)
    heavy = int(cnt.argmax())
    slots = np.nonzero(flat == heavy)[0][:bm]          # stable order = the block's slots
    pick = set((slots // ids.shape[1]).tolist())
    ones = np.nonzero(cnt == 1)[0]
    if len(ones):
        pick.add(int(np.nonzero(flat == ones[0])[0][0] // ids.shape[1]))
    g = synth.rng(seed)
    rest = g.permutation(t)
    for tt in rest:
        if len(pick) >= count:
            break
        pick.add(int(tt))
    return np.array(sorted(pick))


CASES = ([("bf16", t, None) for t in synth.MOE_W4A16_T] + [("mxfp8", t, 1.1) for t in synth.MOE_W4A8_T] +
         [("mxfp4", 1, 1.1), ("mxfp4", 8192, 1.1)])


@pytest.mark.parametrize("act,t,zipf", CASES)
def test_moe_full_size(moe_full, act, t, zipf):
    w13, w2, packs, p13, p2, deq = moe_full
    d13, o13, d2, o2 = packs[act]
    cfgno = 4 if act == "bf16" else 5
    ids, wts = synth.routing(synth.seed_for(cfgno, t), t, 128, 8, zipf_s=zipf)
    xb = synth.bf16_normal(synth.rng(synth.seed_for(cfgno, 100 + t)), (t, 4096))
    bm = hum.moe_select_config(d13, d2, t, 8).block_m
    print(f"case moe full act={act} t={t} block_m={bm}", flush=True)
    out = hum.moe_gemm(d13, p13, d2, p2, dev(xb), dev(ids), dev(wts))
    torch.cuda.synchronize()
    toks = _tokens(ids, t, bm, 256, 9200 + t)
    ref = oracle.moe.moe_forward(o13, w13, o2, w2, xb[toks], ids[toks], wts[toks], act, dequant=deq)
    got = out[torch.from_numpy(toks).cuda()]
    assert_tol(got, ref, f"act={act} t={t} tokens={len(toks)}")
