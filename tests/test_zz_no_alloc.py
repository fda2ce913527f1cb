"""The allocation-free linear (fp4_linear_noalloc) against fp4_linear.

Both run the same kernels; the allocation-free one keeps its workspace in the
library's device array. Each case runs two calls in a row through the C ABI,
the second with a smaller input, and compares every output with fp4_linear's
bit for bit (and with the oracle's product within the GEMM tolerance)."""
import ctypes

import numpy as np
import pytest
import torch

import block_scaled_fp4_quantize_amd as fp4
import oracle
import synth
from tests.gpu_helpers import F, assert_gemm_close, bf16_out_to_f64, to_dev

pytestmark = pytest.mark.gpu


def _noalloc(x, wq, out, static=None):
    """fp4_linear_noalloc straight through ctypes (the C ABI)."""
    L = fp4.lib()
    st = L.fp4_linear_noalloc(ctypes.c_void_p(x.data_ptr()), x.shape[0], ctypes.byref(wq.desc),
                              None if static is None else ctypes.c_void_p(static.data_ptr()),
                              ctypes.c_void_p(out.data_ptr()),
                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


# (m, k, n) pairs: first call, then a smaller one. NVFP4 dynamic at M = 32
# takes the quantizer whose maximum exchange keeps words in the array; M = 300
# the tile GEMM; M = 2 the fused single launch (no workspace use); M = 97 and
# 65 on large weights the mid-size GEMM (three slices of K with their partial
# sums in the array, then one slice).
PAIRS = [((32, 5120, 2048), (8, 2880, 512)),
         ((300, 2880, 1024), (40, 1024, 640)),
         ((16, 4096, 4096), (2, 2880, 520)),
         ((97, 17504, 4100), (65, 5120, 17408))]


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
@pytest.mark.parametrize("pair", PAIRS, ids=["decode", "tile", "fused", "mid"])
@pytest.mark.parametrize("static", [False, True])
def test_noalloc_matches_linear(fmt, pair, static):
    if static and fmt == "mxfp4":
        pytest.skip("MXFP4 has no per-tensor scale")
    f = F[fmt]
    for i, (m, k, n) in enumerate(pair):
        print(f"[noalloc] fmt={fmt} static={static} call {i}: m={m} k={k} n={n}", flush=True)
        a = synth.normal((m, k), 1.0, 90 + i, m * 7 + k)
        w = synth.normal((n, k), 0.02, 91 + i, n * 5 + k)
        wq = fp4.fp4_quantize_weight(to_dev(w), f)
        if pair == PAIRS[3]:
            assert fp4.fp4_linear_mid_splits(f, m, n, k) == (3 if i == 0 else 1)
        x = to_dev(a)
        st_val = float(np.float32(0.0125))
        st = torch.tensor([st_val], dtype=torch.float32, device="cuda") if static else None
        want = fp4.fp4_linear(x, wq, static_scale=st)
        got = torch.full_like(want, float("nan"))
        assert _noalloc(x, wq, got, st) == 0, fp4.lib().fp4_last_error()
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"call {i}: differs from fp4_linear"
        mode = oracle.STATIC if static else oracle.DYNAMIC
        qa = oracle.quantize(f, a, mode=mode, static_scale=st_val if static else None)
        c_ref, l_ref = oracle.gemm(qa, oracle.quantize(f, w))
        assert_gemm_close(bf16_out_to_f64(got), c_ref, l_ref, f"noalloc call {i}")


def test_noalloc_rejects_calls_past_its_array():
    """A call that needs more workspace than the array holds is rejected on the
    host, before anything is launched (M = 4096, K = 8192: ~19 MB)."""
    m, k, n = 4096, 8192, 256
    assert fp4.fp4_linear_workspace_bytes(fp4.NVFP4, m, n, k) > fp4.NOALLOC_SCRATCH_BYTES
    w = synth.normal((n, k), 0.02, 95, 1)
    wq = fp4.fp4_quantize_weight(to_dev(w), fp4.NVFP4)
    x = torch.zeros(m, k, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(m, n, dtype=torch.bfloat16, device="cuda")
    assert _noalloc(x, wq, out) == 4                     # FP4_ERR_WORKSPACE
    assert b"device array" in fp4.lib().fp4_last_error()
