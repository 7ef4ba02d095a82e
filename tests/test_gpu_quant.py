"""GPU: activation quantizers (hum_quant_act) bit for bit against the oracle:
per-token FP8 codes + f32 scales, MXFP8 codes + E8M0 scales."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_packed_amd as hum
import synth
from gpu_util import dev

pytestmark = pytest.mark.gpu


def _inputs(seed, m, k):
    g = synth.rng(seed)
    x = g.standard_normal((m, k)).astype(np.float32)
    x[0] = 0.0                                   # all-zero row
    if m > 2:
        x[1] *= 1e30                             # huge values
        x[2] *= 1e-30                            # tiny values
    if m > 3:
        x[3, :32] = 0.0                          # one zero MX block
        x[3, 40] = -0.0
    return synth.bf16_bits(x)


@pytest.mark.parametrize("m,k", [(1, 128), (6, 2048), (37, 4096), (130, 1024)])
def test_fp8_token_codes_bit_exact(m, k):
    xb = _inputs(100 + m, m, k)
    q, s = hum.quant_act("fp8_token", dev(xb))
    torch.cuda.synchronize()
    rq, rs = oracle.quant.quant_fp8_per_token(oracle.formats.decode_bf16(xb).astype(np.float32))
    assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), rq)


@pytest.mark.parametrize("m,k", [(1, 128), (6, 2048), (37, 4096), (130, 1024)])
def test_mxfp8_codes_bit_exact(m, k):
    xb = _inputs(200 + m, m, k)
    q, s = hum.quant_act("mxfp8", dev(xb))
    torch.cuda.synchronize()
    rq, rs = oracle.quant.quant_mxfp8(oracle.formats.decode_bf16(xb))
    assert np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(q.cpu().numpy(), rq)


@pytest.mark.parametrize("m,k", [(1, 128), (6, 2048), (37, 4096), (130, 1024)])
def test_fp8_group_codes_bit_exact(m, k):
    xb = _inputs(400 + m, m, k)
    if m > 1:
        xb[1, 128:256] = 0                                # an all-zero group
    q, s = hum.quant_act("fp8_group", dev(xb))
    torch.cuda.synchronize()
    rq, rs = oracle.quant.quant_fp8_group(oracle.formats.decode_bf16(xb).astype(np.float32))
    assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), rq)


@pytest.mark.parametrize("m,k", [(1, 128), (6, 2048), (37, 4096), (130, 1024)])
def test_mxfp4_codes_bit_exact(m, k):
    xb = _inputs(300 + m, m, k)
    q, s = hum.quant_act("mxfp4", dev(xb))
    torch.cuda.synchronize()
    rq, rs = oracle.quant.quant_mxfp4(oracle.formats.decode_bf16(xb))
    assert np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(q.cpu().numpy(), rq)


def test_mxfp4_ties_saturation_and_signed_zero():
    """Blocks built so that x / X hits every E2M1 rounding midpoint, values
    above 6 and negative values that round to zero."""
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 5.5, 7.0, 7.9]
    row = np.zeros(64, np.float64)
    row[:len(mids)] = mids
    row[16:16 + len(mids)] = [-v for v in mids]
    row[30] = -0.1
    row[31] = -0.0
    row[32:64] = np.linspace(-3.0, 3.0, 32)
    row[40] = 6.0                                  # amax 6: X = 2^0 for both blocks
    xb = oracle.formats.encode_bf16(row[None, :])
    q, s = hum.quant_act("mxfp4", dev(xb))
    torch.cuda.synchronize()
    rq, rs = oracle.quant.quant_mxfp4(oracle.formats.decode_bf16(xb))
    assert np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(q.cpu().numpy(), rq)


def test_fp8_representable_round_trip():
    g = synth.rng(7)
    codes = g.integers(0, 0x7E, size=(16, 256), dtype=np.uint8) | (g.integers(0, 2, (16, 256), dtype=np.uint8) << 7)
    codes[:, 3] = 0x7E
    x = oracle.formats.decode_e4m3(codes) * np.ldexp(1.0, g.integers(-6, 3, size=16))[:, None]
    xb = oracle.formats.encode_bf16(x)
    q, s = hum.quant_act("fp8_token", dev(xb))
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), codes)
