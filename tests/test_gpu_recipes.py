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
