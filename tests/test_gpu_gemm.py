"""GPU GEMM / linear parity: |C_gpu - C_ref| <= 1e-5 * sum|a_k w_k| + 1 bf16 ulp of C_ref."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_quantize_amd as fp4
import oracle
import synth
from tests.gpu_helpers import F, assert_canonical_equal, assert_gemm_close, bf16_out_to_f64, to_dev

pytestmark = pytest.mark.gpu

FMTS = ["nvfp4", "mxfp4"]


def _gemm_case(fmt, a_bits, w_bits, what, use_linear=True):
    m, k = a_bits.shape
    n = w_bits.shape[0]
    print(f"[gemm] {what} fmt={fmt} m={m} n={n} k={k}", flush=True)
    f = F[fmt]
    qa_ref, qw_ref = oracle.quantize(f, a_bits), oracle.quantize(f, w_bits)
    c_ref, l_ref = oracle.gemm(qa_ref, qw_ref)
    wq = fp4.fp4_quantize_weight(to_dev(w_bits), f)
    x = to_dev(a_bits)
    qa = fp4.fp4_quantize_act(x, f)
    assert_canonical_equal(qa, qa_ref, f, what=what + " (A codes)")
    c = bf16_out_to_f64(fp4.fp4_gemm(qa, wq))
    assert_gemm_close(c, c_ref, l_ref, what + " gemm")
    if m > 128:   # without the re-tiling workspace: the direct-load kernel
        tiny = torch.zeros(16, dtype=torch.uint8, device="cuda")
        c2 = bf16_out_to_f64(fp4.fp4_gemm(qa, wq, workspace=tiny))
        assert_gemm_close(c2, c_ref, l_ref, what + " gemm, no workspace")
    if use_linear:
        y = bf16_out_to_f64(fp4.fp4_linear(x, wq))
        assert_gemm_close(y, c_ref, l_ref, what + " linear")
    return c


@pytest.mark.parametrize("fmt", FMTS)
def test_single_gemm_config(fmt):
    a, w = synth.single_gemm_inputs(0)
    _gemm_case(fmt, a, w, "A[16,256] x W[256,256]")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m,n,k", [(1, 64, 128), (8, 272, 2880), (17, 100, 512), (32, 1040, 1024),
                                   (5, 520, 5120), (2, 48, 17408),
                                   # four and eight activation groups of 16 (M up to 128)
                                   (48, 300, 1024), (64, 1040, 2880), (65, 100, 512),
                                   (100, 520, 4160), (128, 257, 640), (128, 48, 17408),
                                   # two weight tiles per workgroup (>= 512 tiles), odd count
                                   (5, 8200, 256), (20, 8200, 512), (32, 8192, 128),
                                   # two tiles per workgroup at 256-511 tiles: odd and ragged
                                   # tile counts, fewer K fragments than waves
                                   (3, 4112, 640), (16, 4100, 2880), (1, 8176, 128),
                                   (24, 4112, 640), (17, 4100, 5120), (32, 4096, 96)])
def test_decode_path(fmt, m, n, k):
    a = synth.normal((m, k), 1.0, 3, m * 31 + k)
    w = synth.normal((n, k), 0.02, 3, n * 17 + k)
    _gemm_case(fmt, a, w, "decode")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m,n,k", [(33, 136, 256), (300, 520, 2880), (129, 257, 640),
                                   (256, 384, 3072)])
def test_prefill_path(fmt, m, n, k):
    a = synth.normal((m, k), 1.0, 4, m * 31 + k)
    w = synth.normal((n, k), 0.02, 4, n * 17 + k)
    _gemm_case(fmt, a, w, "prefill")


def test_prefill_planted_outliers():
    a, w = synth.prefill_inputs("k", seed=0, m=256)
    _gemm_case("nvfp4", a, w[:512], "prefill t3 + 3616 plants")


@pytest.mark.parametrize("fmt", FMTS)
def test_all_ones_closed_form(fmt):
    """Every value 1.0: C = K exactly (alpha folds the tensor scales)."""
    m, n, k = 40, 48, 1024
    a = np.full((m, k), 0x3F80, np.uint16)   # bf16 1.0
    w = np.full((n, k), 0x3F80, np.uint16)
    c = _gemm_case(fmt, a, w, "all ones")
    assert np.all(c == k)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m", [1, 8, 32])
@pytest.mark.parametrize("k,n", synth.DECODE_SHAPES)
def test_decode_full_size_sampled(fmt, m, k, n):
    """Decode shapes at full size, in the launch configuration the benchmark times;
    4096 sampled outputs against the oracle's k-ordered sums."""
    print(f"[decode-full] fmt={fmt} m={m} k={k} n={n}", flush=True)
    f = F[fmt]
    a, w = synth.decode_inputs(m, k, n, seed=0)
    qa_ref, qw_ref = oracle.quantize(f, a), oracle.quantize(f, w)
    wq = fp4.fp4_quantize_weight(to_dev(w), f)
    x = to_dev(a)
    y = fp4.fp4_linear(x, wq)
    y2 = fp4.fp4_linear(x, wq)
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "results differ between runs"
    rng = np.random.default_rng(m * 7 + n)
    rows = rng.integers(0, m, 4096)
    cols = rng.integers(0, n, 4096)
    c_ref, l_ref = oracle.gemm_sampled(qa_ref, qw_ref, rows, cols)
    yv = bf16_out_to_f64(y)[rows, cols]
    assert_gemm_close(yv, c_ref, l_ref, f"decode full {m}x{n}x{k}")
    # the activation codes of the linear path equal the oracle's
    qa = fp4.fp4_quantize_act(x, f)
    assert_canonical_equal(qa, qa_ref, f, what="decode activation")
    # weight codes, compared through the canonical export
    assert_canonical_equal(fp4.fp4_export_canonical(wq), qw_ref, f, what="decode weight")


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_deterministic(fmt):
    a = synth.normal((200, 1024), 1.0, 6, 1)
    w = synth.normal((300, 1024), 0.02, 6, 2)
    wq = fp4.fp4_quantize_weight(to_dev(w), F[fmt])
    x = to_dev(a)
    y1, y2 = fp4.fp4_linear(x, wq), fp4.fp4_linear(x, wq)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m", [8, 32, 64])
def test_graph_replay_matches_eager(fmt, m):
    """fp4_linear captured in a HIP graph: every replay (with eager work and
    synchronizations in between) equals the eager result bit for bit."""
    k, n = 1024, 2048
    a = synth.normal((m, k), 1.0, 8, m)
    w = synth.normal((n, k), 0.02, 8, n)
    wq = fp4.fp4_quantize_weight(to_dev(w), F[fmt])
    x = to_dev(a)
    ws = torch.zeros(fp4.fp4_linear_workspace_bytes(F[fmt], m, n, k), dtype=torch.uint8, device="cuda")
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
        other = fp4.fp4_linear(x, wq)       # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(other, eager)


@pytest.mark.parametrize("fmt", FMTS)
def test_skinny_gemm_with_one_byte_workspace(fmt):
    """The skinny GEMM (one workgroup per weight tile over the whole K) needs
    no workspace: fp4_gemm with a one-byte workspace matches the oracle."""
    m, n, k = 8, 320, 17408
    f = F[fmt]
    a = synth.normal((m, k), 1.0, 12, 1)
    w = synth.normal((n, k), 0.02, 12, 2)
    qa_ref, qw_ref = oracle.quantize(f, a), oracle.quantize(f, w)
    c_ref, l_ref = oracle.gemm(qa_ref, qw_ref)
    wq = fp4.fp4_quantize_weight(to_dev(w), f)
    qa = fp4.fp4_quantize_act(to_dev(a), f)
    tiny = torch.zeros(1, dtype=torch.uint8, device="cuda")
    c = bf16_out_to_f64(fp4.fp4_gemm(qa, wq, workspace=tiny))
    assert_gemm_close(c, c_ref, l_ref, "skinny GEMM, one-byte workspace")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m", [1, 32])
def test_workspace_reused_across_calls(fmt, m):
    """One zeroed linear workspace (the quantizer's exchange words and the tiled
    activations) serves many calls in sequence."""
    n, k = 640, 5120
    f = F[fmt]
    w = synth.normal((n, k), 0.02, 13, 1)
    qw_ref = oracle.quantize(f, w)
    wq = fp4.fp4_quantize_weight(to_dev(w), f)
    ws = torch.zeros(fp4.fp4_linear_workspace_bytes(f, m, n, k), dtype=torch.uint8, device="cuda")
    for call in range(3):
        a = synth.normal((m, k), 1.0 + call, 13, 10 + call)
        c_ref, l_ref = oracle.gemm(oracle.quantize(f, a), qw_ref)
        y = bf16_out_to_f64(fp4.fp4_linear(to_dev(a), wq, workspace=ws))
        assert_gemm_close(y, c_ref, l_ref, f"call {call}")
    torch.cuda.synchronize()


@pytest.mark.parametrize("m,k", [(1, 17408), (8, 5120), (16, 4096), (17, 2880), (64, 1024)])
def test_linear_static_scale(m, k):
    """fp4_linear with a caller-given per-tensor scale (saturating block scales),
    on both the fused single-launch path and the quantize-then-GEMM path."""
    n = 272
    a, w = synth.prefill_inputs("k", seed=2, m=m)
    a = a[:, :k] if a.shape[1] >= k else synth.student_t((m, k), 3.0, 4.0, 2, 77, plant=3616.0, n_plant=2)
    w = synth.normal((n, k), 0.02, 2, 78)
    st = float(np.float32(0.25))
    qa_ref = oracle.quantize_nvfp4(a, mode=oracle.STATIC, static_scale=st)
    qw_ref = oracle.quantize_nvfp4(w)
    c_ref, l_ref = oracle.gemm(qa_ref, qw_ref)
    wq = fp4.fp4_quantize_weight(to_dev(w), 0)
    y = bf16_out_to_f64(fp4.fp4_linear(to_dev(np.ascontiguousarray(a)), wq,
                                       static_scale=torch.tensor([st], dtype=torch.float32, device="cuda")))
    assert_gemm_close(y, c_ref, l_ref, f"static-scale linear {m}x{k}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m", [1, 8, 32, 300])
def test_extreme_tensor_scales(fmt, m):
    """Operands scaled by 2^-60 and 2^-70: the NVFP4 output scale S_tA * S_tW
    is below FP32's range (~2^-155) while the outputs themselves are around
    2^-130 (bf16 subnormals); every path (fused, decode, tiled) must keep them."""
    k, n = 1024, 272
    a = synth.normal((m, k), 1.0, 31, m)
    w = synth.normal((n, k), 0.02, 31, 1000 + m)
    a = synth.bf16_bits(synth.bf16_to_f32(a) * np.float32(2.0 ** -60))
    w = synth.bf16_bits(synth.bf16_to_f32(w) * np.float32(2.0 ** -70))
    f = F[fmt]
    qa_ref, qw_ref = oracle.quantize(f, a), oracle.quantize(f, w)
    c_ref, l_ref = oracle.gemm(qa_ref, qw_ref)
    assert np.abs(c_ref).max() > 2.0 ** -133, "outputs must not all sit below the tolerance floor"
    wq = fp4.fp4_quantize_weight(to_dev(w), f)
    y = bf16_out_to_f64(fp4.fp4_linear(to_dev(a), wq))
    assert_gemm_close(y, c_ref, l_ref, f"tiny scales m={m}")


_FWD_CACHE = {}


def _forward_weight(fmt, j):
    """Layer 0's weight j of the 24-layer forward: oracle quantization and the
    GPU weight cache, kept across the parametrized cases."""
    key = (fmt, j)
    if key not in _FWD_CACHE:
        w = synth.forward_weight(0, j)
        _FWD_CACHE[key] = (oracle.quantize(F[fmt], w), fp4.fp4_quantize_weight(to_dev(w), F[fmt]))
    return _FWD_CACHE[key]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m", synth.FORWARD_M)
def test_forward_layer_sampled(fmt, m):
    """The 12 linear shapes of one layer of the synthetic 24-layer forward
    (Q, K, V, O, up/down pairs) at the forward's batch sizes, through
    fp4_linear as the benchmark calls it; 512 sampled outputs per call
    against the oracle's k-ordered binary64 sums."""
    for j, (name, k, n) in enumerate(synth.FORWARD_LAYER):
        print(f"[forward] fmt={fmt} m={m} {name} {k}->{n}", flush=True)
        qw_ref, wq = _forward_weight(fmt, j)
        a = synth.forward_act(0, j, m)
        qa_ref = oracle.quantize(F[fmt], a)
        y = bf16_out_to_f64(fp4.fp4_linear(to_dev(a), wq))
        rng = np.random.default_rng(m * 100 + j)
        rows, cols = rng.integers(0, m, 512), rng.integers(0, n, 512)
        c_ref, l_ref = oracle.gemm_sampled(qa_ref, qw_ref, rows, cols)
        assert_gemm_close(y[rows, cols], c_ref, l_ref, f"forward {name} m={m}")


def _linear_sweep_shapes():
    """Seeded (M, N, K) on every GEMM path: the fused skinny linear (small
    M * K), the skinny GEMM with 1, 2, 4 and 8 row groups, the 128 x 128 and
    256 x 256 tiles; ragged M, N and K (K a multiple of 32)."""
    g = np.random.default_rng(20261204)
    shapes = []
    for lo, hi in ((1, 17), (17, 33), (33, 129), (129, 700), (700, 1400)):
        for _ in range(2):
            m = int(g.integers(lo, hi))
            n = int(g.integers(1, 160)) * 8 + int(g.integers(0, 8))
            k = int(g.integers(1, 96)) * 32
            shapes.append((m, n, k))
    return shapes


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m,n,k", _linear_sweep_shapes())
def test_seeded_linear_sweep(fmt, m, n, k):
    """fp4_quantize_act + fp4_gemm and fp4_linear on seeded shapes over every
    GEMM path, within the oracle's tolerance at every output."""
    a = synth.student_t((m, k), 3.0, 1.0, 28, m * 13 + k)
    w = synth.normal((n, k), 0.02, 28, n * 7 + k)
    _gemm_case(fmt, a, w, "seeded sweep")


@pytest.fixture
def no_decode_fusion():
    """fp4_linear with 1-32 rows as quantize + GEMM where the fused skinny
    linear does not apply (the producer form switched off), restored after."""
    prev = fp4.fp4_set_decode_linear_fusion(False)
    yield
    fp4.fp4_set_decode_linear_fusion(prev)


@pytest.mark.parametrize("m,k,n,launches", [(2, 5120, 5120, 1), (3, 5120, 5120, 2),
                                            (2, 8192, 4096, 1), (2, 8192, 4112, 2),
                                            (1, 16384, 8192, 1), (1, 16384, 8208, 2)])
def test_nvfp4_fused_bound(m, k, n, launches, no_decode_fusion):
    """NVFP4 fp4_linear on both sides of the fused path's M * K_pad * tiles
    bounds (4M for two or more rows, 8M for one), with the producer form of
    the skinny linear switched off: the fused single launch and quantize +
    GEMM agree with the oracle alike."""
    assert fp4.fp4_linear_launches("nvfp4", m, n, k) == launches
    a = synth.normal((m, k), 1.0, 11, m * 7 + k)
    w = synth.normal((n, k), 0.02, 11, n * 5 + k)
    _gemm_case("nvfp4", a, w, f"fused bound ({launches} launch(es))")


def test_linear_workspace_shared_across_shapes():
    """One zero-filled workspace, sized for the largest call, serves NVFP4
    dynamic-scale linears of different K, M and paths in sequence (the
    quantizer's exchange words sit at a fixed offset of the workspace)."""
    cases = [(8, 2880, 512), (8, 5760, 2880), (1, 4096, 2880), (32, 2880, 5760), (8, 2880, 4096),
             (128, 5760, 2880), (8, 4096, 2880), (2, 2880, 512)]
    size = max(fp4.fp4_linear_workspace_bytes(0, m, n, k) for (m, k, n) in cases)
    ws = torch.zeros(size, dtype=torch.uint8, device="cuda")
    for rep in range(2):
        for i, (m, k, n) in enumerate(cases):
            print(f"[shared-ws] rep={rep} m={m} k={k} n={n}", flush=True)
            a = synth.normal((m, k), 1.0 + i, 41, 10 * rep + i)
            w = synth.normal((n, k), 0.02, 41, 100 + i)
            qa_ref, qw_ref = oracle.quantize_nvfp4(a), oracle.quantize_nvfp4(w)
            c_ref, l_ref = oracle.gemm(qa_ref, qw_ref)
            wq = fp4.fp4_quantize_weight(to_dev(w), 0)
            y = bf16_out_to_f64(fp4.fp4_linear(to_dev(a), wq, workspace=ws))
            assert_gemm_close(y, c_ref, l_ref, f"shared workspace call {rep}/{i} {m}x{k}x{n}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m,n,k", [(1, 272, 640), (8, 520, 2880), (20, 8200, 512), (33, 100, 256),
                                   (4, 4112, 640), (30, 4100, 512),
                                   # M > 128: re-tiled into the workspace
                                   (200, 272, 640), (300, 100, 2880)])
def test_decode_canonical_wide_pitch(fmt, m, n, k):
    """fp4_gemm on canonical activations whose rows are wider than they need
    to be (codes pitch + 80 bytes, scales pitch + 24): the skinny kernels and
    the re-tiling copy must read only each row's own bytes, whatever lies
    between the rows."""
    print(f"[gemm] canonical wide pitch fmt={fmt} m={m} n={n} k={k}", flush=True)
    f = F[fmt]
    a = synth.normal((m, k), 1.0, 7, m * 29 + k)
    w = synth.normal((n, k), 0.02, 7, n * 13 + k)
    qa_ref, qw_ref = oracle.quantize(f, a), oracle.quantize(f, w)
    c_ref, l_ref = oracle.gemm(qa_ref, qw_ref)
    wq = fp4.fp4_quantize_weight(to_dev(w), f)
    qa = fp4.fp4_quantize_act(to_dev(a), f)
    cp, sp = qa.desc.codes_pitch, qa.desc.scales_pitch
    # copy the rows into wider buffers whose gaps hold bytes that would wreck
    # the result if read (0xFF: NaN E8M0 scales, -6 codes)
    codes = torch.full((m, cp + 80), 0xFF, dtype=torch.uint8, device=qa.codes.device)
    scales = torch.full((m, sp + 24), 0xFF, dtype=torch.uint8, device=qa.codes.device)
    codes[:, :cp] = qa.codes_2d()
    scales[:, :sp] = qa.scales_2d()
    wide = fp4.Fp4Tensor.__new__(fp4.Fp4Tensor)
    wide.fmt, wide.layout, wide.rows, wide.k = qa.fmt, qa.layout, qa.rows, qa.k
    wide.codes, wide.scales, wide.tensor_scale = codes, scales, qa.tensor_scale
    wide.desc = fp4.fp4_tensor()
    wide.desc.fmt, wide.desc.layout, wide.desc.rows, wide.desc.cols = qa.desc.fmt, qa.desc.layout, m, k
    wide.desc.codes_pitch, wide.desc.scales_pitch = cp + 80, sp + 24
    wide.desc.codes, wide.desc.scales = codes.data_ptr(), scales.data_ptr()
    wide.desc.tensor_scale = qa.tensor_scale.data_ptr()
    c = bf16_out_to_f64(fp4.fp4_gemm(wide, wq))
    assert_gemm_close(c, c_ref, l_ref, "decode canonical wide pitch")


@pytest.mark.parametrize("fmt,m,n,k", [("nvfp4", 1, 16, 16), ("nvfp4", 3, 40, 48), ("mxfp4", 1, 16, 32),
                                       ("mxfp4", 5, 48, 96), ("nvfp4", 17, 33, 16), ("mxfp4", 33, 20, 32)])
def test_one_block_deep(fmt, m, n, k):
    """K of one or a few blocks (a single, mostly padded fragment along K)."""
    a = synth.normal((m, k), 1.0, 13, m * 7 + k)
    w = synth.normal((n, k), 0.02, 13, n * 5 + k)
    _gemm_case(fmt, a, w, "one-block K")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m,k,n", [(1, 5120, 272), (8, 2880, 520), (32, 1024, 1040), (200, 512, 300)])
def test_zero_activations_give_zero_output(fmt, m, k, n):
    """All-zero activations: every block scale is zero (NVFP4 takes S_t = 1),
    every code +0, and every output a zero, on each linear path."""
    print(f"[gemm] zero activations fmt={fmt} m={m} k={k} n={n}", flush=True)
    f = F[fmt]
    w = synth.normal((n, k), 0.02, 14, n + k)
    wq = fp4.fp4_quantize_weight(to_dev(w), f)
    x = torch.zeros(m, k, dtype=torch.bfloat16, device="cuda")
    y = fp4.fp4_linear(x, wq)
    qa = fp4.fp4_quantize_act(x, f)
    c = fp4.fp4_gemm(qa, wq)
    torch.cuda.synchronize()
    for out, what in ((y, "linear"), (c, "gemm")):
        bits = out.view(torch.int16).cpu().numpy()
        assert ((bits & 0x7FFF) == 0).all(), f"{what}: nonzero output for zero activations"
    assert (qa.codes_2d().cpu().numpy()[:, : k // 2] == 0).all()
    assert (qa.scales_2d().cpu().numpy()[:, : k // oracle.BLOCK[f]] == 0).all()


# ------------------------------------------------ single-launch decode linear

# (shapes past the fused skinny linear's bounds: more than 16 rows, or M * K_pad
# or M * K_pad * tiles above them)
_DEC1_CASES = [(12, 5200, 5120), (8, 1040, 17408), (19, 1000, 4160), (32, 5120, 5120),
               (17, 8200, 512),      # two weight tiles per workgroup
               (16, 4112, 4224),     # NVFP4: 16-wave workgroups with two tiles
               (1, 8200, 640),       # one row, 513 tiles (NVFP4: the fused skinny linear)
               (1, 8208, 16384),     # NVFP4: one row past the fused bound, >= 512 tiles
               (32, 48, 128),        # fewer K fragments than waves
               (32, 48, 65536)]      # 1024 fragments: 128 producers, the most


@pytest.fixture
def decode_fusion():
    """fp4_linear with 1-32 rows as one launch with producer workgroups (off by
    default), restored afterwards."""
    prev = fp4.fp4_set_decode_linear_fusion(True)
    yield
    fp4.fp4_set_decode_linear_fusion(prev)


@pytest.mark.parametrize("fmt,static", [("nvfp4", False), ("nvfp4", True), ("mxfp4", False),
                                        ("mxfp4+oas", False)])
@pytest.mark.parametrize("m,n,k", _DEC1_CASES)
def test_decode_single_launch(fmt, static, m, n, k, decode_fusion):
    """fp4_linear with 1-32 rows as one launch of the skinny GEMM whose first
    workgroups quantize the activations (NVFP4 dynamic: exchanging their
    maxima first): 2048 sampled outputs within the oracle's tolerance, the
    whole output bit for bit the two-launch result, and a second call with
    other activations through the same workspace reading that call's codes."""
    print(f"[decode-1launch] fmt={fmt} static={static} m={m} n={n} k={k}", flush=True)
    f = fp4._fmt(fmt)
    ofmt = F[fmt.split("+")[0]]
    oas = "oas" in fmt
    st_val = float(np.float32(0.75))
    st = torch.tensor([st_val], dtype=torch.float32, device="cuda") if static else None
    a = synth.student_t((m, k), 3.0, 2.0, 51, m * 13 + k, plant=3616.0, n_plant=2)
    a2 = synth.normal((m, k), 3.0, 51, m * 17 + k)
    w = synth.normal((n, k), 0.02, 51, n * 7 + k)
    assert fp4.fp4_linear_launches(f, m, n, k, static) == 1
    wq = fp4.fp4_quantize_weight(to_dev(w), f)
    x, x2 = to_dev(a), to_dev(a2)
    ws = torch.zeros(fp4.fp4_linear_workspace_bytes(f, m, n, k), dtype=torch.uint8, device="cuda")
    y = fp4.fp4_linear(x, wq, static_scale=st, workspace=ws)
    y2 = fp4.fp4_linear(x2, wq, static_scale=st, workspace=ws)
    fp4.fp4_set_decode_linear_fusion(False)
    try:
        y_two = fp4.fp4_linear(x, wq, static_scale=st)
        y2_two = fp4.fp4_linear(x2, wq, static_scale=st)
    finally:
        fp4.fp4_set_decode_linear_fusion(True)
    torch.cuda.synchronize()
    assert torch.equal(y, y_two), "single launch differs from quantize + GEMM"
    assert torch.equal(y2, y2_two), "second call through the same workspace"
    assert fp4.fp4_workspace_flags(ws) == 0
    mode = oracle.STATIC if static else oracle.DYNAMIC
    qa_ref = oracle.quantize(ofmt, a, mode=mode, static_scale=st_val if static else None, oas=oas)
    qw_ref = oracle.quantize(ofmt, w, oas=oas)
    rng = np.random.default_rng(m * 3 + n)
    rows, cols = rng.integers(0, m, 2048), rng.integers(0, n, 2048)
    c_ref, l_ref = oracle.gemm_sampled(qa_ref, qw_ref, rows, cols)
    assert_gemm_close(bf16_out_to_f64(y)[rows, cols], c_ref, l_ref, f"single-launch decode {m}x{n}x{k}")


@pytest.mark.parametrize("fmt", FMTS)
def test_decode_single_launch_give_up_is_visible(fmt, decode_fusion):
    """The GEMM workgroups' wait for the producers (and, NVFP4, the producers'
    maximum exchange) forced to give up from the host (zero polls): every
    output NaN, the workspace flag set; re-zeroed, the workspace serves a
    correct call."""
    m, n, k = 32, 5120, 5120
    print(f"[decode-1launch] give-up fmt={fmt}", flush=True)
    a = synth.normal((m, k), 1.0, 52, 1)
    w = synth.normal((n, k), 0.02, 52, 2)
    assert fp4.fp4_linear_launches(F[fmt], m, n, k) == 1
    wq = fp4.fp4_quantize_weight(to_dev(w), F[fmt])
    x = to_dev(a)
    ws = torch.zeros(fp4.fp4_linear_workspace_bytes(F[fmt], m, n, k), dtype=torch.uint8, device="cuda")
    prev = fp4.fp4_set_exchange_spin_limit(0)
    try:
        y = fp4.fp4_linear(x, wq, workspace=ws)
        torch.cuda.synchronize()
    finally:
        fp4.fp4_set_exchange_spin_limit(prev)
    assert torch.isnan(y.float()).all()
    assert fp4.fp4_workspace_flags(ws) == fp4.WS_EXCHANGE_TIMEOUT
    ws.zero_()
    c_ref, l_ref = oracle.gemm(oracle.quantize(F[fmt], a), oracle.quantize(F[fmt], w))
    y2 = fp4.fp4_linear(x, wq, workspace=ws)
    assert_gemm_close(bf16_out_to_f64(y2), c_ref, l_ref, "after a give-up")
    assert fp4.fp4_workspace_flags(ws) == 0


@pytest.mark.parametrize("fmt,m,n,k,switch", [("nvfp4", 32, 5120, 5120, "decode"),
                                              ("mxfp4", 8, 5200, 5120, "decode"),
                                              ("mxfp4", 4096, 4096, 1152, "large"),
                                              ("nvfp4", 1024, 2048, 2048, "large")])
def test_single_launch_graph_replay(fmt, m, n, k, switch):
    """The single-launch linears (producer workgroups and ready counts reset by
    the last consumer) captured in a HIP graph: every replay, with eager work
    and synchronizations between them, equals the eager result bit for bit and
    leaves the workspace flags clear."""
    print(f"[graph-1launch] {switch} fmt={fmt} m={m} n={n} k={k}", flush=True)
    setter = fp4.fp4_set_decode_linear_fusion if switch == "decode" else fp4.fp4_set_large_linear_fusion
    prev = setter(True)
    try:
        st = (torch.tensor([1.25], dtype=torch.float32, device="cuda")
              if (switch == "large" and fmt == "nvfp4") else None)
        assert fp4.fp4_linear_launches(F[fmt], m, n, k, st is not None) == 1
        a = synth.normal((m, k), 1.0, 61, m + k)
        w = synth.normal((n, k), 0.02, 61, n + k)
        wq = fp4.fp4_quantize_weight(to_dev(w), F[fmt])
        x = to_dev(a)
        ws = torch.zeros(fp4.fp4_linear_workspace_bytes(F[fmt], m, n, k), dtype=torch.uint8, device="cuda")
        out = torch.empty(m, n, dtype=torch.bfloat16, device="cuda")
        eager = fp4.fp4_linear(x, wq, static_scale=st, out=torch.empty_like(out), workspace=ws).clone()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fp4.fp4_linear(x, wq, static_scale=st, out=out, workspace=ws)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fp4.fp4_linear(x, wq, static_scale=st, out=out, workspace=ws)
        for rep in range(4):
            out.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager), f"replay {rep} differs from eager"
            other = fp4.fp4_linear(x, wq, static_scale=st, workspace=ws)   # eager, same workspace
            torch.cuda.synchronize()
            assert torch.equal(other, eager)
        assert fp4.fp4_workspace_flags(ws) == 0
    finally:
        setter(prev)
