"""Build the gfx950 HIP library ``libfp4amd.so`` in-tree with hipcc.

Every HIP source under ``csrc/`` is compiled for gfx950 only. Packed-FP32
instruction selection is disabled, FP32 denormals are kept and floating-point
contraction is off, so that the quantization decisions written as explicit
fused multiply-adds are the only contractions in the code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfp4amd.so")
SOURCES = ["api.hip", "quant.hip", "gemm.hip", "gemm_tile.hip", "gemm_w4a16.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=off",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found; the FP4 library needs ROCm's hipcc to build")


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + HIPCC_FLAGS + ["-I", os.path.join(HERE, "..", "include"), "-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 target feature; that warning is expected
    noise = [l for l in (res.stderr or "").splitlines() if "packed-fp32-ops" not in l]
    if res.returncode != 0:
        sys.stderr.write("\n".join(noise) + "\n")
        raise RuntimeError("hipcc failed building %s" % LIB)
    if verbose and noise:
        sys.stderr.write("\n".join(noise) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
