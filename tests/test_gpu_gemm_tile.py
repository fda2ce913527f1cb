"""GPU parity of the LDS-staged GEMM for large M (both operands fragment-tiled).

fp4_gemm takes this kernel when M > 128 and the activations are in the tiled
layout (the layout fp4_linear quantizes into). The cases cover each workgroup
tile (256x256 and 128x128, chosen by the output's shape), ragged M and
N, and K loops of 1, 2, 3, 4, 5 and 33 steps of 128 (the ring's prologue and
the unrolled loop's tails). Full-size prefill and square shapes are checked on
sampled outputs against the oracle's k-ordered binary64 sums.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp4_quantize_amd as fp4
import oracle
import synth
from tests.gpu_helpers import F, assert_gemm_close, bf16_out_to_f64, to_dev

pytestmark = pytest.mark.gpu

FMTS = ["nvfp4", "mxfp4"]


def tile_config(m, n):
    """The workgroup tile the library picks for an M x N output (256 CUs)."""
    return 88 if -(-m // 256) * -(-n // 256) >= 256 else 44


def _tiled_case(fmt, a_bits, w_bits, what):
    m, k = a_bits.shape
    n = w_bits.shape[0]
    print(f"[tile] {what} fmt={fmt} m={m} n={n} k={k} cfg={tile_config(m, n)}", flush=True)
    f = F[fmt]
    qa_ref, qw_ref = oracle.quantize(f, a_bits), oracle.quantize(f, w_bits)
    c_ref, l_ref = oracle.gemm(qa_ref, qw_ref)
    wq = fp4.fp4_quantize_weight(to_dev(w_bits), f)
    x = to_dev(a_bits)
    qa = fp4.fp4_quantize_act(x, f, layout=fp4.TILED)
    c = bf16_out_to_f64(fp4.fp4_gemm(qa, wq))
    assert_gemm_close(c, c_ref, l_ref, what + " gemm (tiled A)")
    y = bf16_out_to_f64(fp4.fp4_linear(x, wq))
    assert_gemm_close(y, c_ref, l_ref, what + " linear")
    return c


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m,n,k", [
    (4096, 4096, 256),      # 256 x 256 tiles, 2 K steps
    (4100, 4104, 384),      # 256 x 256 tiles, ragged M and N, 3 K steps
    (4096, 3072, 640),      # 128 x 128 tiles, 5 K steps
    (4111, 2056, 128),      # 128 x 128 tiles, ragged, 1 K step
    (520, 1000, 4160),      # 128 x 128 tiles, 33 K steps (K tail 64)
    (129, 17, 512),         # two partial 128 x 128 tiles, 4 K steps
])
def test_tile_configs(fmt, m, n, k):
    a = synth.normal((m, k), 1.0, 21, m * 31 + k)
    w = synth.normal((n, k), 0.02, 21, n * 17 + k)
    _tiled_case(fmt, a, w, f"tile cfg {tile_config(m, n)}")


@pytest.mark.parametrize("m,n,k", [
    (8200, 4104, 1024),     # 33 x 17 tiles of 256 x 256, ragged M and N
    (2056, 40960, 512),     # 9 x 160 tiles: several per CU
])
def test_mxfp4_tiles_closed_form(m, n, k):
    """Every output of a large MXFP4 tile GEMM against a closed form: A row
    i = 2^(i mod 7 - 3), W row j = 2^(j mod 5 - 2) quantize exactly (each
    block is one power of two: code 4, E8M0 2^(p - 2)), so C[i, j] =
    K * 2^(i mod 7 - 3 + j mod 5 - 2) exactly; a tile written to the wrong
    place, a row or column shifted or a K step dropped changes outputs.
    Eager and over graph replays."""
    print(f"[tile-closed] m={m} n={n} k={k}", flush=True)
    ea = (torch.arange(m, device="cuda") % 7 - 3).float()
    ew = (torch.arange(n, device="cuda") % 5 - 2).float()
    x = torch.pow(2.0, ea).unsqueeze(1).expand(m, k).to(torch.bfloat16).contiguous()
    w = torch.pow(2.0, ew).unsqueeze(1).expand(n, k).to(torch.bfloat16).contiguous()
    want = (float(k) * torch.pow(2.0, ea.unsqueeze(1) + ew.unsqueeze(0))).to(torch.bfloat16)
    wq = fp4.fp4_quantize_weight(w, fp4.MXFP4)
    qa = fp4.fp4_quantize_act(x, fp4.MXFP4, layout=fp4.TILED)
    out = torch.empty(m, n, dtype=torch.bfloat16, device="cuda")
    fp4.fp4_gemm(qa, wq, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out, want), f"{(out != want).sum().item()} outputs differ"
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fp4.fp4_gemm(qa, wq, out=out)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(2):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {rep}: {(out != want).sum().item()} outputs differ"


@pytest.mark.parametrize("fmt", FMTS)
def test_tile_outliers_and_zero_rows(fmt):
    """Planted +-3616 outliers and whole zero rows/blocks in A and W."""
    m, n, k = 300, 700, 1024
    a = synth.student_t((m, k), 3.0, 4.0, 22, 1, plant=3616.0, n_plant=8)
    w = synth.normal((n, k), 0.02, 22, 2)
    a[5] = 0
    a[:, 64:96] = 0
    w[13] = 0
    _tiled_case(fmt, a, w, "outliers + zero rows")


@pytest.mark.parametrize("fmt", FMTS)
def test_tile_all_ones_closed_form(fmt):
    """Every value 1.0 through the tiled path: C = K exactly."""
    m, n, k = 260, 300, 2048
    a = np.full((m, k), 0x3F80, np.uint16)
    w = np.full((n, k), 0x3F80, np.uint16)
    c = _tiled_case(fmt, a, w, "all ones")
    assert np.all(c == k)


@pytest.mark.parametrize("fmt", FMTS)
def test_tile_unaligned_output_pitch(fmt):
    """An output row pitch that is not a multiple of 4 elements takes the
    element-wise stores; the result is the same as with a dense output."""
    m, n, k = 100, 130, 512
    f = F[fmt]
    a = synth.normal((m, k), 1.0, 23, 1)
    w = synth.normal((n, k), 0.02, 23, 2)
    wq = fp4.fp4_quantize_weight(to_dev(w), f)
    qa = fp4.fp4_quantize_act(to_dev(a), f, layout=fp4.TILED)
    dense = fp4.fp4_gemm(qa, wq)
    big = torch.full((m, n + 3), 7.0, dtype=torch.bfloat16, device="cuda")
    view = big[:, :n]
    fp4.fp4_gemm(qa, wq, out=view)
    torch.cuda.synchronize()
    assert torch.equal(view, dense)
    assert torch.all(big[:, n:] == 7.0), "stores past N"


@pytest.fixture
def nv_tile_lds():
    """The NVFP4 256 x 256 tiles with the conversion in LDS for one test."""
    prev = fp4.fp4_set_nvfp4_tile_mode(fp4.NV_TILE_LDS)
    yield
    fp4.fp4_set_nvfp4_tile_mode(prev)


@pytest.mark.parametrize("m,n,k", [
    (4096, 4096, 256),      # 2 K steps (one pass of the two-stage ring)
    (4100, 4104, 384),      # ragged M and N, 3 K steps (odd stage count)
    (4096, 4352, 128),      # 1 K step
    (4224, 4096, 1152),     # 9 K steps
    (4096, 4100, 2944),     # 23 K steps, K tail of 64 (K = 2880)
])
def test_nvfp4_tile_lds_conversion(nv_tile_lds, m, n, k):
    """The NVFP4 tile with every fragment converted once per workgroup into
    LDS matches the oracle, and matches the in-register conversion bit for bit
    (both sum the same exact f16 products in the same order)."""
    kk = 2880 if k == 2944 else k
    a = synth.student_t((m, kk), 3.0, 4.0, 25, m + kk, plant=3616.0, n_plant=4)
    w = synth.normal((n, kk), 0.02, 25, n * 3 + kk)
    c_lds = _tiled_case("nvfp4", a, w, "nvfp4 tile, conversion in LDS")
    prev = fp4.fp4_set_nvfp4_tile_mode(fp4.NV_TILE_REGISTERS)
    try:
        wq = fp4.fp4_quantize_weight(to_dev(w), fp4.NVFP4)
        qa = fp4.fp4_quantize_act(to_dev(a), fp4.NVFP4, layout=fp4.TILED)
        c_reg = bf16_out_to_f64(fp4.fp4_gemm(qa, wq))
    finally:
        fp4.fp4_set_nvfp4_tile_mode(prev)
    assert np.array_equal(c_lds, c_reg)


def test_nvfp4_tile_lds_square_8192_sampled(nv_tile_lds):
    a, w = synth.square_inputs(8192, seed=0)
    _sampled_full("nvfp4", a, w, "square 8192, conversion in LDS")


@pytest.mark.parametrize("fmt", FMTS)
def test_tile_deterministic_and_graph(fmt):
    """Two eager calls agree bit for bit, and so does every replay of a graph
    holding the call (with eager work between replays)."""
    m, n, k = 1024, 2048, 1024
    f = F[fmt]
    a = synth.normal((m, k), 1.0, 24, 1)
    w = synth.normal((n, k), 0.02, 24, 2)
    wq = fp4.fp4_quantize_weight(to_dev(w), f)
    x = to_dev(a)
    ws = torch.zeros(fp4.fp4_linear_workspace_bytes(f, m, n, k), dtype=torch.uint8, device="cuda")
    e1 = fp4.fp4_linear(x, wq, workspace=ws).clone()
    e2 = fp4.fp4_linear(x, wq, workspace=ws).clone()
    torch.cuda.synchronize()
    assert torch.equal(e1, e2)
    out = torch.empty(m, n, dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fp4.fp4_linear(x, wq, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fp4.fp4_linear(x, wq, out=out, workspace=ws)
    for rep in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, e1), f"replay {rep} differs"
        assert torch.equal(fp4.fp4_linear(x, wq), e1)


def _sampled_full(fmt, a, w, what, nsamp=4096, seed=0):
    m, k = a.shape
    n = w.shape[0]
    print(f"[tile-full] {what} fmt={fmt} m={m} n={n} k={k}", flush=True)
    f = F[fmt]
    qa_ref, qw_ref = oracle.quantize(f, a), oracle.quantize(f, w)
    wq = fp4.fp4_quantize_weight(to_dev(w), f)
    y = fp4.fp4_linear(to_dev(a), wq)
    rng = np.random.default_rng(seed + m + n + k)
    rows = rng.integers(0, m, nsamp)
    cols = rng.integers(0, n, nsamp)
    # include the corners of the output
    rows[:4] = [0, 0, m - 1, m - 1]
    cols[:4] = [0, n - 1, 0, n - 1]
    c_ref, l_ref = oracle.gemm_sampled(qa_ref, qw_ref, rows, cols)
    yv = bf16_out_to_f64(y)[rows, cols]
    assert_gemm_close(yv, c_ref, l_ref, what)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("layer", list(synth.PREFILL_LAYERS))
def test_prefill_full_size_sampled(fmt, layer):
    """Llama-style 3B block prefill GEMMs (M = 4096, t(3)*4 activations with
    planted 3616 outliers), as the benchmark runs them."""
    a, w = synth.prefill_inputs(layer, seed=0)
    _sampled_full(fmt, a, w, f"prefill {layer}")


@pytest.mark.parametrize("fmt", FMTS)
def test_square_4096_sampled(fmt):
    """M = N = K = 4096 (the smallest square configuration), operands ~N(0, 1)."""
    a, w = synth.square_inputs(4096, seed=0)
    _sampled_full(fmt, a, w, "square 4096")


@pytest.mark.parametrize("fmt", FMTS)
def test_square_8192_sampled(fmt):
    """M = N = K = 8192, operands ~N(0, 1)."""
    a, w = synth.square_inputs(8192, seed=0)
    _sampled_full(fmt, a, w, "square 8192")


_SQ16 = {}


@pytest.mark.parametrize("fmt", FMTS)
def test_square_16384_sampled(fmt):
    """M = N = K = 16384 (the largest square configuration), operands ~N(0, 1);
    the inputs are drawn once for both formats."""
    if "ab" not in _SQ16:
        _SQ16["ab"] = synth.square_inputs(16384, seed=0)
    a, w = _SQ16["ab"]
    _sampled_full(fmt, a, w, "square 16384", nsamp=2048)
    if fmt == FMTS[-1]:
        _SQ16.clear()


# ------------------------------------------- single-launch linear for large M

@pytest.fixture
def large_fusion():
    """fp4_linear with large-M quantization inside the GEMM launch (off by
    default), restored afterwards."""
    prev = fp4.fp4_set_large_linear_fusion(True)
    yield
    fp4.fp4_set_large_linear_fusion(prev)


@pytest.mark.parametrize("fmt,m,n,k,rotate", [
    ("nvfp4", 4096, 4096, 256, False),     # 256 x 256 tiles, 16 panels
    ("nvfp4", 4100, 4104, 384, False),     # ragged M and N
    ("nvfp4", 300, 520, 2880, False),      # 128 x 128 tiles, K tail of 64
    ("nvfp4", 4096, 3072, 3072, True),     # rotated
    ("mxfp4", 4096, 4096, 1152, False),
    ("mxfp4", 129, 1000, 4160, False),     # two panels, 33 K steps
    ("mxfp4", 4224, 4096, 640, True),
])
def test_fused_large_linear(fmt, m, n, k, rotate, large_fusion):
    """fp4_linear at M > 128 as one launch (the first workgroups quantize each
    row panel of activations, split along K; the tiles wait for their panel):
    within the tolerance of the oracle, and bit for bit the quantize + GEMM
    result (the same codes and the same kernel arithmetic)."""
    print(f"[fused-large] fmt={fmt} m={m} n={n} k={k} rotate={rotate}", flush=True)
    f = F[fmt] | (fp4.ROTATE if rotate else 0)
    a = synth.student_t((m, k), 3.0, 4.0, 26, m + 7 * k, plant=3616.0, n_plant=4)
    w = synth.normal((n, k), 0.02, 26, n * 5 + k)
    st_val = float(np.float32(1.5))
    st = torch.tensor([st_val], dtype=torch.float32, device="cuda") if fmt == "nvfp4" else None
    mode = oracle.STATIC if fmt == "nvfp4" else oracle.DYNAMIC
    qa_ref = oracle.quantize(F[fmt], a, mode=mode, static_scale=st_val if st is not None else None,
                             rotate=rotate)
    qw_ref = oracle.quantize(F[fmt], w, rotate=rotate)
    c_ref, l_ref = oracle.gemm(qa_ref, qw_ref)
    assert fp4.fp4_linear_launches(f, m, n, k, st is not None) == 1
    wq = fp4.fp4_quantize_weight(to_dev(w), f)
    x = to_dev(a)
    ws = torch.zeros(fp4.fp4_linear_workspace_bytes(f, m, n, k), dtype=torch.uint8, device="cuda")
    y = fp4.fp4_linear(x, wq, static_scale=st, workspace=ws)
    y2 = fp4.fp4_linear(x, wq, static_scale=st, workspace=ws)     # the panel words reset
    assert_gemm_close(bf16_out_to_f64(y), c_ref, l_ref, "fused large linear")
    prev = fp4.fp4_set_large_linear_fusion(False)
    try:
        assert fp4.fp4_linear_launches(f, m, n, k, st is not None) >= 2
        y3 = fp4.fp4_linear(x, wq, static_scale=st)
    finally:
        fp4.fp4_set_large_linear_fusion(prev)
    assert fp4.fp4_linear_launches(f, m, n, k, st is not None) == 1
    # other activations through the same workspace: the panels written by this
    # call, not the lines the previous call left in any cache, are what the
    # tiles read
    x2 = to_dev(synth.normal((m, k), 2.0, 26, m + 11 * k))
    y4 = fp4.fp4_linear(x2, wq, static_scale=st, workspace=ws)
    fp4.fp4_set_large_linear_fusion(False)
    try:
        y5 = fp4.fp4_linear(x2, wq, static_scale=st)
    finally:
        fp4.fp4_set_large_linear_fusion(True)
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(y, y3)
    assert torch.equal(y4, y5) and not torch.equal(y4, y)
    assert fp4.fp4_workspace_flags(ws) == 0


def test_fused_large_linear_give_up_is_visible(large_fusion):
    """Tiles that give up waiting for their activation panel (forced from the
    host: zero polls) output NaN and set the workspace flag; a re-zeroed
    workspace then serves a correct call."""
    m, n, k = 4096, 4096, 512
    a = synth.normal((m, k), 1.0, 27, 1)
    w = synth.normal((n, k), 0.02, 27, 2)
    wq = fp4.fp4_quantize_weight(to_dev(w), fp4.MXFP4)
    x = to_dev(a)
    ws = torch.zeros(fp4.fp4_linear_workspace_bytes(fp4.MXFP4, m, n, k), dtype=torch.uint8, device="cuda")
    prev = fp4.fp4_set_exchange_spin_limit(0)
    try:
        y = fp4.fp4_linear(x, wq, workspace=ws)
        torch.cuda.synchronize()
    finally:
        fp4.fp4_set_exchange_spin_limit(prev)
    assert torch.isnan(y.float()).all()
    assert fp4.fp4_workspace_flags(ws) == fp4.WS_EXCHANGE_TIMEOUT
    ws.zero_()
    c_ref, l_ref = oracle.gemm(oracle.quantize(oracle.MXFP4, a), oracle.quantize(oracle.MXFP4, w))
    y2 = fp4.fp4_linear(x, wq, workspace=ws)
    assert_gemm_close(bf16_out_to_f64(y2), c_ref, l_ref, "after a give-up")
    assert fp4.fp4_workspace_flags(ws) == 0
