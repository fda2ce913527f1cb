"""Host-side AddressSanitizer and UndefinedBehaviorSanitizer runs (CPU only).

The oracle (plain C) and the host side of the HIP library (argument checks,
sizes, layouts, workspace arithmetic; the GPU code is built as usual) are
rebuilt with ASan + UBSan and exercised by the CPU tests that cover them: the
oracle pins and the C-ABI checks, each in a child process with the matching
sanitizer runtime preloaded (gcc's for the oracle, the ROCm compiler's for the
library). Negative controls with a planted heap overflow, built the same way,
must abort, so a run that passes had the sanitizers armed."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}

pytestmark = pytest.mark.slow

OVERFLOW_C = r"""
#include <stdlib.h>
int planted_overflow(int n) { int *p = (int *)malloc(4 * sizeof(int)); p[n] = 1; int r = p[0]; free(p); return r; }
"""

RUNNER = r"""
import sys
sys.path.insert(0, {root!r})
import {module} as m
setattr(m, {attr!r}, {lib!r})
if {control!r}:
    import ctypes
    ctypes.CDLL({control!r}).planted_overflow(9)
import pytest
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", {tests!r}]))
"""


def _run(tmp, module, attr, lib, tests, runtime, control=""):
    script = os.path.join(tmp, "run_%s.py" % module)
    with open(script, "w") as fh:
        fh.write(RUNNER.format(root=ROOT, module=module, attr=attr, lib=lib, tests=tests,
                               control=control))
    env = dict(os.environ, LD_PRELOAD=runtime, **SAN_ENV)
    return subprocess.run([sys.executable, script], env=env, capture_output=True, text=True,
                          timeout=900)


def _gcc_runtime():
    return subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True, check=True).stdout.strip()


def test_oracle_under_asan_ubsan(tmp_path):
    tmp = str(tmp_path)
    lib = os.path.join(tmp, "liborc_san.so")
    flags = ["-O1", "-g", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    subprocess.run(["gcc"] + flags + ["-o", lib, os.path.join(ROOT, "oracle", "fp4_oracle.c"), "-lm"],
                   check=True)
    ctl_src = os.path.join(tmp, "overflow.c")
    with open(ctl_src, "w") as fh:
        fh.write(OVERFLOW_C)
    ctl = os.path.join(tmp, "liboverflow_gcc.so")
    subprocess.run(["gcc"] + flags + ["-o", ctl, ctl_src], check=True)
    rt = _gcc_runtime()
    pins = os.path.join(ROOT, "tests", "test_oracle_pins.py")
    bad = _run(tmp, "oracle", "_LIB_PATH", lib, pins, rt, control=ctl)
    assert bad.returncode != 0 and ("AddressSanitizer" in bad.stderr or "runtime error" in bad.stderr), \
        "sanitizer not armed"
    res = _run(tmp, "oracle", "_LIB_PATH", lib, pins, rt)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs ROCm's hipcc")
def test_library_host_code_under_asan_ubsan(tmp_path):
    tmp = str(tmp_path)
    rts = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rts:
        pytest.skip("the ROCm compiler's ASan runtime is not installed")
    csrc = os.path.join(ROOT, "block_scaled_fp4_quantize_amd", "csrc")
    srcs = [os.path.join(csrc, f) for f in ("api.hip", "quant.hip", "gemm.hip", "gemm_tile.hip",
                                            "gemm_w4a16.hip")]
    host_san = ["-Xarch_host", "-fsanitize=address",
                "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all",
                "-Xarch_host", "-fno-omit-frame-pointer"]
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=off"]
    lib = os.path.join(tmp, "libfp4amd_san.so")
    subprocess.run([HIPCC] + common + host_san + ["-I", os.path.join(ROOT, "include"), "-o", lib]
                   + srcs, check=True, capture_output=True)
    ctl_src = os.path.join(tmp, "overflow.cpp")
    with open(ctl_src, "w") as fh:
        fh.write('extern "C" ' + OVERFLOW_C.replace("(int *)malloc", "(int *)malloc"))
    ctl = os.path.join(tmp, "liboverflow_clang.so")
    subprocess.run([HIPCC] + ["-O1", "-fPIC", "-shared"] + host_san + ["-o", ctl, ctl_src],
                   check=True, capture_output=True)
    abi = os.path.join(ROOT, "tests", "test_abi.py")
    bad = _run(tmp, "block_scaled_fp4_quantize_amd", "LIB_PATH", lib, abi, rts[-1], control=ctl)
    assert bad.returncode != 0 and ("AddressSanitizer" in bad.stderr or "runtime error" in bad.stderr), \
        "sanitizer not armed"
    res = _run(tmp, "block_scaled_fp4_quantize_amd", "LIB_PATH", lib, abi, rts[-1])
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]
