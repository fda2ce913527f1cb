"""GPU parity of the mid-size GEMM (33-128 activation rows, four weight tiles per
workgroup, K split over workgroups with an ordered FP32 combine) against the
oracle: |C_gpu - C_ref| <= 1e-5 * sum|a_k w_k| + 1 bf16 ulp of C_ref, through
fp4_linear and through fp4_gemm on tiled activations, and against the skinny
kernel it replaces (same tolerance, both against the oracle)."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_quantize_amd as fp4
import oracle
import synth
from tests.gpu_helpers import F, assert_gemm_close, bf16_out_to_f64, mid_rule, to_dev

pytestmark = pytest.mark.gpu

FMTS = ["nvfp4", "mxfp4"]


@pytest.fixture(autouse=True)
def _mid_on():
    prev = fp4.fp4_set_mid_gemm(True)
    yield
    fp4.fp4_set_mid_gemm(prev)


def _splits(m, n, k, fmt=fp4.NVFP4):
    """K slices of fp4_linear's mid-size GEMM (0: another kernel runs)."""
    return fp4.fp4_linear_mid_splits(fmt, m, n, k)


def _sample(m, n, seed, count=2048):
    rng = np.random.default_rng(seed)
    return rng.integers(0, m, count), rng.integers(0, n, count)


def test_mid_full_oracle():
    """33 rows (four activation groups, one real row in the last), 513 weight
    tiles (the last workgroup holds one, N not a multiple of 16), one slice:
    every output against the oracle, both formats."""
    m, n, k = 33, 8200, 4096
    for fmt in FMTS:
        assert _splits(m, n, k, F[fmt]) == 1
        print(f"[mid-full] fmt={fmt} m={m} n={n} k={k} splits={_splits(m, n, k)}", flush=True)
        f = F[fmt]
        a = synth.normal((m, k), 1.0, 21, 1)
        w = synth.normal((n, k), 0.02, 21, 2)
        qa_ref, qw_ref = oracle.quantize(f, a), oracle.quantize(f, w)
        c_ref, l_ref = oracle.gemm(qa_ref, qw_ref)
        wq = fp4.fp4_quantize_weight(to_dev(w), f)
        x = to_dev(a)
        y = fp4.fp4_linear(x, wq)
        assert_gemm_close(bf16_out_to_f64(y), c_ref, l_ref, "mid linear")
        fp4.fp4_set_mid_gemm(False)
        y0 = fp4.fp4_linear(x, wq)
        fp4.fp4_set_mid_gemm(True)
        assert_gemm_close(bf16_out_to_f64(y0), c_ref, l_ref, "skinny linear")


# (m, n, k): eight and four activation groups with ragged rows, ragged weight
# tiles and K (not a multiple of 128), one slice and three; the decode shapes
# at 64 and 65 rows
SHAPES = [(97, 4100, 17504), (128, 8200, 8224), (64, 5120, 17408), (65, 17408, 5120),
          (128, 4112, 16448), (120, 16400, 4224)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m,n,k", SHAPES)
def test_mid_sampled(fmt, m, n, k):
    """fp4_linear and fp4_gemm on tiled activations (the same launches, so
    bit-equal) and the skinny kernel, 2048 sampled outputs against the
    oracle's k-ordered sums."""
    print(f"[mid] fmt={fmt} m={m} n={n} k={k} splits={_splits(m, n, k)}", flush=True)
    assert _splits(m, n, k, F[fmt]) >= 1
    f = F[fmt]
    a = synth.normal((m, k), 1.0, 22, m * 131 + k)
    w = synth.normal((n, k), 0.02, 22, n * 7 + k)
    qa_ref, qw_ref = oracle.quantize(f, a), oracle.quantize(f, w)
    rows, cols = _sample(m, n, m + n + k)
    c_ref, l_ref = oracle.gemm_sampled(qa_ref, qw_ref, rows, cols)
    wq = fp4.fp4_quantize_weight(to_dev(w), f)
    x = to_dev(a)
    y = fp4.fp4_linear(x, wq)
    assert_gemm_close(bf16_out_to_f64(y)[rows, cols], c_ref, l_ref, "mid linear")
    qt = fp4.fp4_quantize_act(x, f, layout=fp4.TILED)
    c = fp4.fp4_gemm(qt, wq)
    torch.cuda.synchronize()
    assert torch.equal(c, y)
    fp4.fp4_set_mid_gemm(False)
    y0 = fp4.fp4_linear(x, wq)
    assert_gemm_close(bf16_out_to_f64(y0)[rows, cols], c_ref, l_ref, "skinny linear")


@pytest.mark.parametrize("fmt", FMTS)
def test_mid_launch_counts(fmt):
    f = F[fmt]
    m, n, k = 128, 5120, 17408
    assert _splits(m, n, k) == 3
    assert fp4.fp4_linear_launches(f, m, n, k) == 3
    fp4.fp4_set_mid_gemm(False)
    assert fp4.fp4_linear_launches(f, m, n, k) == 2
    fp4.fp4_set_mid_gemm(True)
    # one slice: no combining launch
    assert _splits(128, 17408, 5120) == 1
    assert fp4.fp4_linear_launches(f, 128, 17408, 5120) == 2


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m,n,k", [(128, 5760, 2880), (64, 5120, 5120), (48, 2880, 4096)])
def test_small_shapes_keep_the_skinny_kernel(fmt, m, n, k):
    """Below the mid-size kernel's bound the switch changes nothing: bit-equal."""
    f = F[fmt]
    assert _splits(m, n, k, f) == 0
    x = to_dev(synth.normal((m, k), 1.0, 24, 1))
    wq = fp4.fp4_quantize_weight(to_dev(synth.normal((n, k), 0.02, 24, 2)), f)
    y = fp4.fp4_linear(x, wq)
    fp4.fp4_set_mid_gemm(False)
    y0 = fp4.fp4_linear(x, wq)
    torch.cuda.synchronize()
    assert torch.equal(y, y0)


@pytest.mark.parametrize("fmt", FMTS)
def test_mid_graph_replay_matches_eager(fmt):
    """Three slices: every replay of a captured fp4_linear (with eager work
    and synchronizations in between) equals the eager result bit for bit."""
    m, n, k = 97, 4100, 17504
    assert _splits(m, n, k) == 3
    f = F[fmt]
    x = to_dev(synth.normal((m, k), 1.0, 25, 1))
    wq = fp4.fp4_quantize_weight(to_dev(synth.normal((n, k), 0.02, 25, 2)), f)
    ws = torch.zeros(fp4.fp4_linear_workspace_bytes(f, m, n, k), dtype=torch.uint8, device="cuda")
    out = torch.empty(m, n, dtype=torch.bfloat16, device="cuda")
    eager = fp4.fp4_linear(x, wq, out=torch.empty_like(out), workspace=ws).clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fp4.fp4_linear(x, wq, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fp4.fp4_linear(x, wq, out=out, workspace=ws)
    for rep in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from eager"
        other = fp4.fp4_linear(x, wq)
        torch.cuda.synchronize()
        assert torch.equal(other, eager)


def test_mid_gemm_small_workspace_falls_back():
    """fp4_gemm on tiled activations without room for the partial sums runs
    on the skinny kernel (still within tolerance)."""
    m, n, k = 64, 5120, 17408
    assert _splits(m, n, k) == 3
    f = fp4.NVFP4
    a = synth.normal((m, k), 1.0, 23, 1)
    w = synth.normal((n, k), 0.02, 23, 2)
    qa_ref, qw_ref = oracle.quantize(f, a), oracle.quantize(f, w)
    wq = fp4.fp4_quantize_weight(to_dev(w), f)
    qt = fp4.fp4_quantize_act(to_dev(a), f, layout=fp4.TILED)
    tiny = torch.zeros(16, dtype=torch.uint8, device="cuda")
    c = fp4.fp4_gemm(qt, wq, workspace=tiny)
    full = fp4.fp4_gemm(qt, wq)
    rows, cols = _sample(m, n, 5)
    c_ref, l_ref = oracle.gemm_sampled(qa_ref, qw_ref, rows, cols)
    assert_gemm_close(bf16_out_to_f64(c)[rows, cols], c_ref, l_ref, "skinny fallback")
    assert_gemm_close(bf16_out_to_f64(full)[rows, cols], c_ref, l_ref, "mid")


def _mid_sweep_shapes():
    """Seeded (M, N, K) that the mid-size kernel takes: 33-128 rows, ragged
    N, K a multiple of 32, 64-100 M weight values."""
    g = np.random.default_rng(20261205)
    shapes = []
    while len(shapes) < 6:
        m = int(g.integers(33, 129))
        n = int(g.integers(3000, 17500))
        k = int(g.integers(64_000_000 // n, 100_000_000 // n)) // 32 * 32
        if mid_rule(m, n, k):
            shapes.append((m, n, k))
    return shapes


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m,n,k", _mid_sweep_shapes())
def test_mid_seeded_sweep(fmt, m, n, k):
    """The library's slice count equals the restated rule; 2048 sampled
    outputs of fp4_linear within the oracle's tolerance."""
    f = F[fmt]
    s = mid_rule(m, n, k)
    print(f"[mid-sweep] fmt={fmt} m={m} n={n} k={k} splits={s}", flush=True)
    assert _splits(m, n, k, f) == s
    a = synth.student_t((m, k), 3.0, 1.0, 29, m * 13 + k)
    w = synth.normal((n, k), 0.02, 29, n * 7 + k)
    qa_ref, qw_ref = oracle.quantize(f, a), oracle.quantize(f, w)
    rows, cols = _sample(m, n, m * 3 + k)
    c_ref, l_ref = oracle.gemm_sampled(qa_ref, qw_ref, rows, cols)
    y = fp4.fp4_linear(to_dev(a), fp4.fp4_quantize_weight(to_dev(w), f))
    assert_gemm_close(bf16_out_to_f64(y)[rows, cols], c_ref, l_ref, f"mid sweep {m}x{n}x{k}")
