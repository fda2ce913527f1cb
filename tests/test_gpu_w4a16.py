"""GPU parity of the weight-only linear (W4A16): bf16 activations times the
FP4 weight cache, against the oracle's binary64 weight-only product, within
|err| <= 1e-5 * sum|x w^| + one bf16 ulp."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_quantize_amd as fp4
import oracle
import synth
from tests.gpu_helpers import F, assert_gemm_close, bf16_out_to_f64, to_dev

pytestmark = pytest.mark.gpu

FMTS = ["nvfp4", "mxfp4"]


def _case(fmt, a, w, what, sample=None):
    m, k = a.shape
    n = w.shape[0]
    print(f"[w4a16] {what} fmt={fmt} m={m} n={n} k={k}", flush=True)
    f = F[fmt]
    qw = oracle.quantize(f, w)
    wq = fp4.fp4_quantize_weight(to_dev(w), f)
    y = bf16_out_to_f64(fp4.fp4_linear_w4a16(to_dev(a), wq))
    if sample is None:
        c_ref, l_ref = oracle.gemm_w4a16(a, qw)
        assert_gemm_close(y, c_ref, l_ref, what)
    else:
        rng = np.random.default_rng(m + n + k)
        rows, cols = rng.integers(0, m, sample), rng.integers(0, n, sample)
        rows[:4], cols[:4] = [0, 0, m - 1, m - 1], [0, n - 1, 0, n - 1]
        c_ref, l_ref = oracle.gemm_w4a16_sampled(a, qw, rows, cols)
        assert_gemm_close(y[rows, cols], c_ref, l_ref, what)
    return y


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m,k,n", [
    (1, 256, 256), (5, 2880, 520), (16, 1056, 100), (17, 4160, 64), (32, 5120, 1000),
    (1, 48, 33), (3, 16, 17),           # K below one fragment; NVFP4 K tail of 16
    (33, 512, 17), (300, 1024, 700), (520, 4160, 1000), (129, 2880, 4096),
    (8, 256, 16400), (20, 512, 8200), (24, 1024, 4100),  # 4 / 2 tiles per workgroup, odd counts
])
def test_w4a16_shapes(fmt, m, k, n):
    if fmt == "mxfp4" and k % 32:
        pytest.skip("MXFP4 needs K % 32 == 0")
    a = synth.normal((m, k), 1.0, 61, m * 13 + k)
    w = synth.normal((n, k), 0.02, 61, n * 7 + k)
    _case(fmt, a, w, f"shape {m}x{k}x{n}")


@pytest.mark.parametrize("fmt", FMTS)
def test_w4a16_outliers_and_zero_rows(fmt):
    a = synth.student_t((40, 2048), 3.0, 4.0, 62, 1, plant=3616.0, n_plant=16)
    w = synth.normal((300, 2048), 0.02, 62, 2)
    a[3] = 0
    w[7] = 0
    w[:, 512:544] = 0
    _case(fmt, a, w, "outliers + zero rows")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("wscale", [2.0 ** -120, 2.0 ** -60, 2.0 ** 60, 2.0 ** 100])
def test_w4a16_extreme_weight_scales(fmt, wscale):
    """Tiny weights (MXFP4 block exponents down to the 2^-127 scale, which
    takes the FP32 route) and large ones."""
    rng = np.random.default_rng(63)
    a = synth.normal((8, 1024), 1.0, 63, 1)
    w = synth.bf16_bits((rng.standard_normal((64, 1024)) * wscale).astype(np.float32))
    _case(fmt, a, w, f"weights x{wscale:g}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m", [1, 8, 32])
@pytest.mark.parametrize("k,n", [(5120, 5120), (5120, 17408), (17408, 5120)])
def test_w4a16_decode_shapes_full(fmt, m, k, n):
    """The decode configurations the benchmark runs, sampled outputs."""
    a, w = synth.decode_inputs(m, k, n, seed=0)
    _case(fmt, a, w, "decode", sample=2048)


@pytest.mark.parametrize("fmt", FMTS)
def test_w4a16_prefill_shape_sampled(fmt):
    a, w = synth.prefill_inputs("gate", seed=0)
    _case(fmt, a, w, "prefill gate", sample=2048)


@pytest.mark.parametrize("fmt", FMTS)
def test_w4a16_deterministic_graph_and_pitch(fmt):
    """Bit-identical repeats, graph replays, and an output row pitch wider than N."""
    f = F[fmt]
    for m in (8, 200):
        a = synth.normal((m, 1024), 1.0, 64, m)
        w = synth.normal((520, 1024), 0.02, 64, 2)
        wq = fp4.fp4_quantize_weight(to_dev(w), f)
        x = to_dev(a)
        e1 = fp4.fp4_linear_w4a16(x, wq).clone()
        e2 = fp4.fp4_linear_w4a16(x, wq).clone()
        torch.cuda.synchronize()
        assert torch.equal(e1, e2)
        big = torch.full((m, 527), 3.0, dtype=torch.bfloat16, device="cuda")
        fp4.fp4_linear_w4a16(x, wq, out=big[:, :520])
        torch.cuda.synchronize()
        assert torch.equal(big[:, :520], e1) and torch.all(big[:, 520:] == 3.0)
        out = torch.empty(m, 520, dtype=torch.bfloat16, device="cuda")
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fp4.fp4_linear_w4a16(x, wq, out=out)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fp4.fp4_linear_w4a16(x, wq, out=out)
        for rep in range(3):
            out.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, e1), f"replay {rep}"
            assert torch.equal(fp4.fp4_linear_w4a16(x, wq), e1)
