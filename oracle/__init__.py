"""CPU oracle for the quantized dense / MoE GEMM path.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
NumPy float64 statement of what the GPU library computes.  Only the tests,
the smoke check and the bench's CPU-baseline leg may import it; the library
(``quantized_gemm_packed_amd``) never does, and this package imports nothing
from the library.  The two share no code; only the seeded input generators
in ``synth`` serve both.

Structure (quantize -> dequantize exactly -> fp64 matmul) is the
quantize/dequantize reference against which fused kernels were checked in
the "H100, W4A8 and group-32" section of the aireiter.com benchmark review
of vLLM Humming.  The formats themselves are only named on the pages
("Announcing Humming: Fast, Flexible Kernels for Quantized Inference",
sections "Background", "Unified quantization representation", "Quantization
support"); their bit-level definitions are taken from the public OCP FP8 and
OCP Microscaling (MX) v1.0 specifications that those names refer to.

Modules:
  formats  decode / encode of INT4, UINT4, E2M1, E4M3 (FN), E8M0, BF16
  quant    per-token FP8 and MXFP8 activation quantizers
  gemm     weight dequantization and the dense linear layer
  moe      routing align, per-expert GEMMs with SwiGLU, weighted reduce

Every function here is pinned by a CPU test against something other than
itself (brute force, library routines, closed forms, invariants); see the
``tests/test_oracle_*.py`` files.
"""
from . import formats, quant, gemm, moe  # noqa: F401
