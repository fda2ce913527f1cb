"""GPU parity of the quantization recipes: block Hadamard rotation (either
format) and the overflow-aware MXFP4 exponent. Codes, scales and tensor
scales must equal the oracle's byte for byte; products of rotated operands
meet the usual GEMM tolerance against the oracle's product of the same
quantized operands."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_quantize_amd as fp4
import oracle
import synth
from tests.gpu_helpers import F, assert_canonical_equal, assert_gemm_close, bf16_out_to_f64, to_dev

pytestmark = pytest.mark.gpu

FMTS = ["nvfp4", "mxfp4"]


def _flags(fmt, rotate, oas):
    return F[fmt] | (fp4.ROTATE if rotate else 0) | (fp4.MX_OAS if oas else 0)


def _ref(fmt, bits, rotate, oas, static=None):
    mode = oracle.STATIC if static is not None else oracle.DYNAMIC
    return oracle.quantize(F[fmt], bits, mode=mode, static_scale=static, rotate=rotate, oas=oas)


# (m, k): single-launch (small) and two-launch (large) quantizer paths
SHAPES = [(1, 32), (17, 2880), (1, 17408), (40, 5120), (320, 16384)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m,k", SHAPES)
@pytest.mark.parametrize("layout", ["canonical", "tiled"])
def test_rotated_activation_quantization(fmt, m, k, layout):
    print(f"[recipe-rot] fmt={fmt} m={m} k={k} layout={layout}", flush=True)
    bits = synth.student_t((m, k), 3.0, 1.0, 51, m * 31 + k, plant=80.0, n_plant=max(1, m * k // 500))
    ref = _ref(fmt, bits, True, False)
    lay = fp4.TILED if layout == "tiled" else fp4.CANONICAL
    q = fp4.fp4_quantize_act(to_dev(bits), _flags(fmt, True, False), layout=lay)
    if lay == fp4.TILED:
        q = fp4.fp4_export_canonical(q)
    assert_canonical_equal(q, ref, F[fmt], what=f"rotated act {m}x{k} {layout}")


@pytest.mark.parametrize("static", [0.01, 1e-30])
def test_rotated_static_scale(static):
    bits = synth.normal((24, 4096), 3.0, 52, 1)
    ref = _ref("nvfp4", bits, True, False, static=static)
    st = torch.tensor([static], dtype=torch.float32, device="cuda")
    q = fp4.fp4_quantize_act(to_dev(bits), fp4.NVFP4 | fp4.ROTATE, static_scale=st)
    assert_canonical_equal(q, ref, oracle.NVFP4, what=f"rotated static {static}")


@pytest.mark.parametrize("fmt", FMTS)
def test_rotated_every_finite_bf16_value(fmt):
    """Every finite bf16 pattern below 2^120 in magnitude, shuffled into rows
    (the rotation's contract), through the rotated quantizer."""
    bits = np.arange(0, 0x10000, dtype=np.uint32)
    exp = (bits >> 7) & 0xFF
    bits = bits[exp < 127 + 120].astype(np.uint16)
    rng = np.random.default_rng(4)
    rng.shuffle(bits)
    k = 2048
    rows = len(bits) // k
    x = bits[: rows * k].reshape(rows, k)
    print(f"[recipe-rot] every bf16 fmt={fmt} rows={rows}", flush=True)
    q = fp4.fp4_quantize_act(to_dev(x), _flags(fmt, True, False))
    assert_canonical_equal(q, _ref(fmt, x, True, False), F[fmt], what="rotated every bf16")


def _wide_range_rows(rows, k, seed):
    """Blocks whose nonzero magnitudes span up to 2^250, with large values that
    cancel exactly inside a rotation sum, subnormals and zeros: the rotation's
    exact integer path (a binary64 transform is not exact on them)."""
    rng = np.random.default_rng(seed)
    e = rng.integers(-133, 119, (rows, k))
    x = rng.choice([-1.0, 1.0], (rows, k)) * rng.integers(1, 256, (rows, k)) * 2.0 ** (e - 7)
    x[rng.random((rows, k)) < 0.1] = 0.0
    big = 2.0 ** rng.integers(60, 110, (rows, 1))
    x[:, 0::16], x[:, 1::16] = big, -big
    x[::2, 2::32] = 2.0 ** -133
    return synth.bf16_bits(x.astype(np.float32))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m,k", [(5, 256), (48, 4096), (320, 2880)])
def test_rotated_wide_range_blocks(fmt, m, k):
    print(f"[recipe-rot] wide-range fmt={fmt} m={m} k={k}", flush=True)
    bits = _wide_range_rows(m, k, 7 * m + k)
    ref = _ref(fmt, bits, True, False)
    for lay in (fp4.CANONICAL, fp4.TILED):
        q = fp4.fp4_quantize_act(to_dev(bits), _flags(fmt, True, False), layout=lay)
        if lay == fp4.TILED:
            q = fp4.fp4_export_canonical(q)
        assert_canonical_equal(q, ref, F[fmt], what=f"rotated wide-range {m}x{k} layout {lay}")


def _tier_boundary_rows(rows, k, block, seed):
    """bf16 blocks around the rotation's FP32 / binary64 boundary: per block an
    exponent spread of 10-13 fields (FP32 is exact up to 16 - log2(block)),
    the smallest exponent field near 34 in half of them (the 32-value
    rotation's FP32 product bound), significands rich in exact bf16 midpoints
    after the transform, zeros and negative zeros."""
    rng = np.random.default_rng(seed)
    nb = k // block
    spread = rng.integers(10, 14, (rows, nb, 1))
    fmin = np.where(rng.random((rows, nb, 1)) < 0.5, rng.integers(33, 36, (rows, nb, 1)),
                    rng.integers(60, 200, (rows, nb, 1)))
    f = fmin + (rng.random((rows, nb, block)) * (spread + 1)).astype(np.int64)
    f[:, :, 0] = fmin[:, :, 0]                    # the block's spread is attained
    f[:, :, 1] = (fmin + spread)[:, :, 0]
    m = np.where(rng.random((rows, nb, block)) < 0.5, rng.integers(0, 128, (rows, nb, block)),
                 rng.choice([0, 0x40], (rows, nb, block)))
    sign = rng.integers(0, 2, (rows, nb, block)) << 15
    bits = (sign | (f << 7) | m).astype(np.uint16)
    z = rng.random((rows, nb, block)) < 0.05
    bits[z] = (sign[z]).astype(np.uint16)           # +0 and -0
    return bits.reshape(rows, k)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m,k", [(8, 4096), (300, 2880)])
def test_rotated_tier_boundary_blocks(fmt, m, k):
    """Exact rotation across its FP32 / binary64 boundary: codes and scales
    byte for byte the oracle's, in both layouts."""
    print(f"[recipe-rot] tier-boundary fmt={fmt} m={m} k={k}", flush=True)
    block = 16 if fmt == "nvfp4" else 32
    bits = _tier_boundary_rows(m, k, block, 11 * m + k)
    ref = _ref(fmt, bits, True, False)
    for lay in (fp4.CANONICAL, fp4.TILED):
        q = fp4.fp4_quantize_act(to_dev(bits), _flags(fmt, True, False), layout=lay)
        if lay == fp4.TILED:
            q = fp4.fp4_export_canonical(q)
        assert_canonical_equal(q, ref, F[fmt], what=f"rotated tier-boundary {m}x{k} layout {lay}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k", [(33, 96), (520, 2880)])
def test_rotated_weight_cache(fmt, n, k):
    w = synth.normal((n, k), 0.02, 53, n + k)
    wq = fp4.fp4_quantize_weight(to_dev(w), _flags(fmt, True, False))
    assert_canonical_equal(fp4.fp4_export_canonical(wq), _ref(fmt, w, True, False), F[fmt],
                           what=f"rotated weight {n}x{k}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m,k,n", [(1, 5120, 512), (8, 2880, 4096), (32, 5120, 1024),
                                   (300, 1024, 640), (520, 4096, 1000)])
def test_rotated_linear(fmt, m, k, n):
    """fp4_linear through a rotated weight: the activations are rotated with
    the weight's recipe (fused, decode and tiled paths)."""
    print(f"[recipe-linear] fmt={fmt} m={m} k={k} n={n}", flush=True)
    a = synth.student_t((m, k), 3.0, 1.0, 54, m + k, plant=60.0, n_plant=max(1, m * k // 1000))
    w = synth.normal((n, k), 0.02, 54, n + k)
    qa, qw = _ref(fmt, a, True, False), _ref(fmt, w, True, False)
    c_ref, l_ref = oracle.gemm(qa, qw)
    wq = fp4.fp4_quantize_weight(to_dev(w), _flags(fmt, True, False))
    y = bf16_out_to_f64(fp4.fp4_linear(to_dev(a), wq))
    assert_gemm_close(y, c_ref, l_ref, f"rotated linear {m}x{k}x{n}")
    # and through the separate quantize + GEMM calls
    qg = fp4.fp4_quantize_act(to_dev(a), _flags(fmt, True, False), layout=fp4.TILED)
    c = bf16_out_to_f64(fp4.fp4_gemm(qg, wq))
    assert_gemm_close(c, c_ref, l_ref, f"rotated gemm {m}x{k}x{n}")


# ------------------------------------------------------------------- OAS

@pytest.mark.parametrize("m,k", [(1, 32), (17, 2880), (40, 5120), (320, 16384)])
@pytest.mark.parametrize("layout", ["canonical", "tiled"])
def test_oas_activation_quantization(m, k, layout):
    print(f"[recipe-oas] m={m} k={k} layout={layout}", flush=True)
    bits = synth.normal((m, k), 1.0, 55, m * 7 + k)
    ref = _ref("mxfp4", bits, False, True)
    lay = fp4.TILED if layout == "tiled" else fp4.CANONICAL
    q = fp4.fp4_quantize_act(to_dev(bits), fp4.MXFP4 | fp4.MX_OAS, layout=lay)
    if lay == fp4.TILED:
        q = fp4.fp4_export_canonical(q)
    assert_canonical_equal(q, ref, oracle.MXFP4, what=f"oas act {m}x{k} {layout}")


def test_oas_every_finite_bf16_value():
    """Every block maximum mantissa, including those in (6, 8) * 2^e that the
    overflow-aware exponent moves up, sorted so blocks share binades."""
    bits = np.arange(0, 0x10000, dtype=np.uint32)
    exp = (bits >> 7) & 0xFF
    bits = np.sort(bits[exp != 0xFF].astype(np.uint16))
    k = 2560
    rows = len(bits) // k
    x = bits[: rows * k].reshape(rows, k)
    for rot in (False, True):
        xx = x if not rot else x[:, :]
        if rot:   # the rotation's contract: |x| < 2^120
            keep = ((xx >> 7) & 0xFF) < 127 + 120
            xx = np.where(keep, xx, np.uint16(0)).astype(np.uint16)
        q = fp4.fp4_quantize_act(to_dev(xx), _flags("mxfp4", rot, True))
        assert_canonical_equal(q, _ref("mxfp4", xx, rot, True), oracle.MXFP4,
                               what=f"oas every bf16 rotate={rot}")


@pytest.mark.parametrize("m,k,n", [(1, 5120, 512), (16, 2880, 1024), (32, 5120, 640),
                                   (300, 1024, 640)])
def test_oas_linear(m, k, n):
    """OAS weights and activations (fused, decode and tiled paths); a GEMM of
    an OAS activation with a default-rule weight is accepted too."""
    print(f"[recipe-oas-linear] m={m} k={k} n={n}", flush=True)
    a = synth.normal((m, k), 1.0, 56, m + k)
    w = synth.normal((n, k), 0.02, 56, n + k)
    qa, qw = _ref("mxfp4", a, False, True), _ref("mxfp4", w, False, True)
    c_ref, l_ref = oracle.gemm(qa, qw)
    wq = fp4.fp4_quantize_weight(to_dev(w), fp4.MXFP4 | fp4.MX_OAS)
    y = bf16_out_to_f64(fp4.fp4_linear(to_dev(a), wq))
    assert_gemm_close(y, c_ref, l_ref, f"oas linear {m}x{k}x{n}")
    wd = fp4.fp4_quantize_weight(to_dev(w), fp4.MXFP4)
    qg = fp4.fp4_quantize_act(to_dev(a), fp4.MXFP4 | fp4.MX_OAS, layout=fp4.TILED)
    c_ref2, l_ref2 = oracle.gemm(qa, _ref("mxfp4", w, False, False))
    assert_gemm_close(bf16_out_to_f64(fp4.fp4_gemm(qg, wd)), c_ref2, l_ref2, "oas act x default weight")


# ------------------------------------------------ MXFP4 macro-block scaling

def _mbs_flags(rotate=False, oas=False):
    return fp4.MXFP4 | fp4.MX_MBS | (fp4.ROTATE if rotate else 0) | (fp4.MX_OAS if oas else 0)


def _assert_mbs_equal(q, ref, what):
    """Codes and E8M0 bytes (byte for byte) and macro-block scales (bit for bit)."""
    if q.layout == fp4.TILED:
        q = fp4.fp4_export_canonical(q)
    assert_canonical_equal(q, ref, oracle.MXFP4, what=what)
    torch.cuda.synchronize()
    got = q.macro_2d().cpu().numpy()
    assert got.shape == ref.macro.shape, what
    diff = np.argwhere(got.view(np.uint32) != ref.macro.view(np.uint32))
    assert len(diff) == 0, f"{what}: {len(diff)} macro scales differ, first {tuple(diff[0])}: " \
                           f"gpu {got[tuple(diff[0])]!r} ref {ref.macro[tuple(diff[0])]!r}"


@pytest.mark.parametrize("m,k", [(1, 32), (3, 96), (17, 2880), (40, 5120), (320, 16384)])
@pytest.mark.parametrize("layout", ["canonical", "tiled"])
@pytest.mark.parametrize("rotate,oas", [(False, False), (False, True), (True, False)])
def test_mbs_activation_quantization(m, k, layout, rotate, oas):
    print(f"[recipe-mbs] m={m} k={k} layout={layout} rotate={rotate} oas={oas}", flush=True)
    bits = synth.student_t((m, k), 3.0, 2.0, 61, m * 37 + k, plant=200.0, n_plant=max(1, m * k // 700))
    ref = oracle.quantize(oracle.MXFP4, bits, rotate=rotate, oas=oas, mbs=True)
    lay = fp4.TILED if layout == "tiled" else fp4.CANONICAL
    q = fp4.fp4_quantize_act(to_dev(bits), _mbs_flags(rotate, oas), layout=lay)
    _assert_mbs_equal(q, ref, f"mbs act {m}x{k} {layout}")


@pytest.mark.parametrize("n,k", [(33, 96), (520, 2880), (256, 16384)])
def test_mbs_weight_cache_and_dequantize(n, k):
    w = synth.normal((n, k), 0.02, 62, n + k)
    ref = oracle.quantize(oracle.MXFP4, w, mbs=True)
    wq = fp4.fp4_quantize_weight(to_dev(w), _mbs_flags())
    _assert_mbs_equal(wq, ref, f"mbs weight {n}x{k}")
    # x^ = q * 2^e_b * S_mb, rounded once to FP32
    got = fp4.fp4_dequantize(wq).cpu().numpy()
    want = oracle.dequantize(ref).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("m,n,k", [(1, 272, 640), (8, 520, 2880), (32, 1040, 5120), (100, 300, 1024),
                                   (33, 8200, 256), (300, 520, 2880), (256, 384, 3072)])
def test_mbs_gemm_and_linear(m, n, k):
    """Products of macro-block-scaled operands: fp4_linear, fp4_gemm on tiled
    and canonical activations (with and without the re-tiling workspace)."""
    print(f"[recipe-mbs] gemm m={m} n={n} k={k}", flush=True)
    a = synth.student_t((m, k), 3.0, 2.0, 63, m * 31 + k, plant=150.0, n_plant=3)
    w = synth.normal((n, k), 0.02, 63, n * 17 + k)
    qa_ref = oracle.quantize(oracle.MXFP4, a, mbs=True)
    qw_ref = oracle.quantize(oracle.MXFP4, w, mbs=True)
    c_ref, l_ref = oracle.gemm(qa_ref, qw_ref)
    wq = fp4.fp4_quantize_weight(to_dev(w), _mbs_flags())
    x = to_dev(a)
    y = bf16_out_to_f64(fp4.fp4_linear(x, wq))
    assert_gemm_close(y, c_ref, l_ref, f"mbs linear {m}x{n}x{k}")
    for lay in (fp4.TILED, fp4.CANONICAL):
        qa = fp4.fp4_quantize_act(x, _mbs_flags(), layout=lay)
        c = bf16_out_to_f64(fp4.fp4_gemm(qa, wq))
        assert_gemm_close(c, c_ref, l_ref, f"mbs gemm layout {lay}")
        if lay == fp4.CANONICAL and m > 128:
            tiny = torch.zeros(16, dtype=torch.uint8, device="cuda")
            c2 = bf16_out_to_f64(fp4.fp4_gemm(qa, wq, workspace=tiny))
            assert_gemm_close(c2, c_ref, l_ref, "mbs gemm canonical, no workspace")


def test_mbs_operands_must_match():
    w = synth.normal((64, 256), 0.02, 64, 1)
    a = synth.normal((8, 256), 1.0, 64, 2)
    wq = fp4.fp4_quantize_weight(to_dev(w), _mbs_flags())
    qa = fp4.fp4_quantize_act(to_dev(a), fp4.MXFP4)
    with pytest.raises(fp4.Fp4Error, match="FORMAT_MISMATCH"):
        fp4.fp4_gemm(qa, wq)
    with pytest.raises(fp4.Fp4Error, match="FORMAT_MISMATCH"):
        fp4.fp4_linear_w4a16(to_dev(a), wq)
