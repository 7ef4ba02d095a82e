"""Builds libhum.so (all HIP kernels + the C ABI) for gfx950 with hipcc.

The library is built in-tree, next to this file, so it travels with the
source tree.  Every translation unit is compiled with packed-FP32 code
generation disabled (hipcc still emits plain FP32 VALU code).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libhum.so")
BUILD_DIR = os.path.join(HERE, "_build")
# The GEMM kernel instances are spread over several translation units so
# that they compile in parallel.
GEMM_SOURCES = ["gemm.hip", "inst_dense_a.hip", "inst_dense_b.hip", "inst_dense_c.hip", "inst_dense_d.hip",
                "inst_dense_sk.hip", "inst_moe_a.hip", "inst_moe_b.hip", "inst_moe_c.hip"]
SOURCES = ["api.hip", "repack.hip", "act_moe.hip", "peaks.hip", *GEMM_SOURCES]
ARCH = os.environ.get("HUM_OFFLOAD_ARCH", "gfx950")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-I", os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    raise RuntimeError("hipcc not found")


# Per-source flags.  The GEMM kernels keep MFMA results in ordinary VGPRs:
# the INT path scales every K-block's MFMA result on the VALU, which reads
# VGPRs only (AGPR results would cost one v_accvgpr_read per element).
EXTRA = {src: ["-mllvm", "-amdgpu-mfma-vgpr-form"] for src in GEMM_SOURCES}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-6000:]}")
    return obj


def build_library(verbose: bool = True) -> str:
    """Compile every source and link libhum.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = min(len(SOURCES), max(1, int(os.environ.get("MAX_JOBS", "8"))))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-6000:]}")
    # every symbol of the library's own namespace must be defined (a kernel
    # whose host stub the compiler dropped shows up here, not at load time)
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [ln.split()[-1] for ln in nm.stdout.splitlines() if "3hum" in ln]
    if nm.returncode != 0 or missing:
        raise RuntimeError(f"{tmp}: undefined library symbols: {missing[:5]}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build_library()
