"""GPU quantization parity: codes, scales and tensor scales byte-identical to the oracle."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_quantize_amd as fp4
import oracle
import synth
from tests.gpu_helpers import F, assert_canonical_equal, to_dev

pytestmark = pytest.mark.gpu

FMTS = ["nvfp4", "mxfp4"]


def _act_case(fmt, bits, what, static=None):
    print(f"[quant-act] {what} fmt={fmt} shape={bits.shape}", flush=True)
    f = F[fmt]
    ref = oracle.quantize(f, bits, mode=oracle.STATIC if static is not None else oracle.DYNAMIC,
                          static_scale=static)
    st = None if static is None else torch.tensor([static], dtype=torch.float32, device="cuda")
    q = fp4.fp4_quantize_act(to_dev(bits), f, static_scale=st)
    assert_canonical_equal(q, ref, f, what=what)
    return q, ref


@pytest.mark.parametrize("fmt", FMTS)
def test_single_gemm_activation(fmt):
    a, _ = synth.single_gemm_inputs(0)
    _act_case(fmt, a, "A[16,256] with x100 outliers")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m,k", [(1, 32), (3, 96), (17, 2880), (40, 5120), (129, 544), (1, 17408),
                                 # NVFP4 dynamic: the largest M * K whose workgroups each take
                                 # the whole tensor's maximum, and the next size up
                                 (8, 6144), (8, 6176)])
def test_ragged_shapes(fmt, m, k):
    bits = synth.normal((m, k), 1.0, 1, m * 100003 + k)
    _act_case(fmt, bits, f"ragged {m}x{k}")


@pytest.mark.parametrize("fmt", FMTS)
def test_every_finite_bf16_value(fmt):
    """All 65,280 finite bf16 patterns (both zeros included), shuffled into rows."""
    bits = np.arange(0, 0x10000, dtype=np.uint32)
    exp = (bits >> 7) & 0xFF
    bits = bits[exp != 0xFF].astype(np.uint16)
    rng = np.random.default_rng(0)
    rng.shuffle(bits)
    k = 2560
    rows = len(bits) // k
    x = bits[: rows * k].reshape(rows, k)
    _act_case(fmt, x, "every finite bf16")
    # sorted order too: blocks of neighbouring magnitudes exercise every scale
    xs = np.sort(bits)[: rows * k].reshape(rows, k)
    _act_case(fmt, xs, "every finite bf16, sorted")


@pytest.mark.parametrize("fmt", FMTS)
def test_tiny_and_huge_magnitudes(fmt):
    rng = np.random.default_rng(5)
    for scale in (2.0 ** -126, 2.0 ** -110, 2.0 ** -70, 2.0 ** 60, 2.0 ** 120):
        x = synth.bf16_bits((rng.standard_normal((8, 256)) * scale).astype(np.float32))
        _act_case(fmt, x, f"magnitude {scale:g}")
    z = np.zeros((4, 64), np.uint16)
    z[1, 5] = 0x8000
    _act_case(fmt, z, "all zeros")


def test_nvfp4_ties_and_midpoints():
    """Blocks whose elements sit exactly on rounding midpoints of their scale."""
    rng = np.random.default_rng(3)
    rows = []
    for _ in range(256):
        s = float(2.0 ** rng.integers(-8, 8)) * (1 + rng.integers(0, 8) / 8)
        mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0]) * s
        blk = np.concatenate([[6 * s], rng.choice(mids, 15) * rng.choice([-1, 1], 15)])
        rows.append(blk)
    xf = np.array(rows, np.float32).reshape(16, 256)
    x = synth.bf16_bits(xf)
    _act_case("nvfp4", x, "midpoints, dynamic")
    _act_case("nvfp4", x, "midpoints, static 1/448", static=float(np.float32(1 / 448)))
    # power-of-two S_t: block scales come out exact (s_b = s, or 2s up to the
    # 448 saturation) and quotients land exactly on the midpoints (ties)
    _act_case("nvfp4", x, "midpoints, static 1 (exact ties)", static=1.0)
    _act_case("nvfp4", x, "midpoints, static 1/2 (exact ties)", static=0.5)
    # dynamic with an exact S_t: amax = 42 = 2688 * 2^-6 gives S_t = 2^-6
    xd = xf * np.float32(2.0 ** -6)
    xd[0, 0] = 42.0
    _act_case("nvfp4", synth.bf16_bits(xd), "midpoints, dynamic S_t = 2^-6 (exact ties)")


def test_prefill_planted_outliers_two_level():
    """t(3)*4 activations with planted +-3616 entries: block maxima beyond 2688."""
    a, _ = synth.prefill_inputs("q", seed=0, m=512)
    q, ref = _act_case("nvfp4", a, "prefill t3 with 3616 plants")
    assert ref.scales.max() == 0x7E


@pytest.mark.parametrize("static", [1.0, 0.01, 3.5, 1e-30])
def test_static_scale_saturates(static):
    a, _ = synth.prefill_inputs("k", seed=1, m=64)
    _act_case("nvfp4", a, f"static S_t={static}", static=float(np.float32(static)))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k", [(256, 256), (520, 2880), (33, 96), (1024, 5120)])
def test_weight_cache_layout(fmt, n, k):
    print(f"[quant-weight] fmt={fmt} n={n} k={k}", flush=True)
    f = F[fmt]
    w = synth.normal((n, k), 0.02, 2, n * 7 + k)
    ref = oracle.quantize(f, w)
    wq = fp4.fp4_quantize_weight(to_dev(w), f)
    canon = fp4.fp4_export_canonical(wq)
    assert_canonical_equal(canon, ref, f, what=f"weight {n}x{k}")
    # dequantized values: RN_fp32 of the exact q * s_b * S_t
    dq = fp4.fp4_dequantize(wq).cpu().numpy()
    ref_dq = oracle.dequantize(ref).astype(np.float32)
    assert np.array_equal(dq, ref_dq)
    dq2 = fp4.fp4_dequantize(canon).cpu().numpy()
    assert np.array_equal(dq2, ref_dq)


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_is_deterministic(fmt):
    a = synth.normal((64, 4096), 1.0, 9, 1)
    x = to_dev(a)
    q1 = fp4.fp4_quantize_act(x, F[fmt])
    q2 = fp4.fp4_quantize_act(x, F[fmt])
    torch.cuda.synchronize()
    assert torch.equal(q1.codes, q2.codes) and torch.equal(q1.scales, q2.scales)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m,k", [(1, 5120), (8, 17408), (32, 17408), (17, 2880), (300, 544)])
def test_tiled_activation_layout(fmt, m, k):
    """Activations quantized into the fragment-tiled layout hold the same bytes."""
    print(f"[quant-act-tiled] fmt={fmt} m={m} k={k}", flush=True)
    f = F[fmt]
    bits = synth.normal((m, k), 1.0, 14, m * 7 + k)
    ref = oracle.quantize(f, bits)
    q = fp4.fp4_quantize_act(to_dev(bits), f, layout=fp4.TILED)
    assert_canonical_equal(fp4.fp4_export_canonical(q), ref, f, what=f"tiled act {m}x{k}")


@pytest.mark.parametrize("fmt", FMTS)
def test_single_launch_limit(fmt):
    """Both sides of the single-launch / two-launch switch (2^17 blocks per call)."""
    f = F[fmt]
    for m in (64, 65) if fmt == "nvfp4" else (128, 129):
        bits = synth.normal((m, 32768), 1.0, 15, m)
        print(f"[quant-limit] fmt={fmt} m={m}", flush=True)
        _act_case(fmt, bits, f"limit m={m}")


@pytest.mark.parametrize("m,k,launches", [(300, 8192, 2), (1000, 3008, 2), (4096, 3072, 2), (4100, 4000, 2),
                                          (4096, 8192, 2), (4112, 8192, 3)])
def test_mid_size_one_pass(m, k, launches):
    """NVFP4 activations with the dynamic scale past the single-launch
    quantizer's size, into the tiled layout: up to 16384 fragments in one pass
    (each wave holding 1, 2 or 4 fragments while the workgroups exchange their
    maxima), past that the two-pass path; ragged rows and K included. Codes,
    scales and S_t byte-identical to the oracle."""
    print(f"[quant-mid] m={m} k={k}", flush=True)
    assert fp4.fp4_linear_launches(fp4.NVFP4, m, 64, k) == launches
    bits = synth.normal((m, k), 1.0, 17, m * 3 + k)
    ref = oracle.quantize(0, bits)
    q = fp4.fp4_quantize_act(to_dev(bits), 0, layout=fp4.TILED)
    assert_canonical_equal(fp4.fp4_export_canonical(q), ref, 0, what=f"mid-size tiled {m}x{k}")


def _sweep_shapes():
    """Seeded (rows, K) pairs on both sides of the quantizer's path bounds:
    the single-launch size (2^17 blocks), the one-pass mid-size bound (16384
    fragments of 16 x 128) and the two-pass path, with ragged rows and K."""
    g = np.random.default_rng(20261203)
    shapes = []
    for lo, hi in ((1, 64), (64, 600), (600, 3000), (3000, 9000)):
        for _ in range(3):
            rows = int(g.integers(lo, hi))
            k = int(g.integers(1, 8192 // 32 + 1)) * 32 if rows < 3000 else int(g.integers(1, 64)) * 32
            shapes.append((rows, k))
    return shapes


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m,k", _sweep_shapes())
def test_seeded_shape_sweep(fmt, m, k):
    """Codes, scales and S_t byte-identical to the oracle in both layouts,
    on seeded shapes spread over every quantizer path; NVFP4 also with a
    static scale."""
    print(f"[quant-sweep] fmt={fmt} m={m} k={k}", flush=True)
    f = F[fmt]
    bits = synth.student_t((m, k), 3.0, 1.5, 27, m * 11 + k)
    ref = oracle.quantize(f, bits)
    q = fp4.fp4_quantize_act(to_dev(bits), f)
    assert_canonical_equal(q, ref, f, what=f"sweep canonical {m}x{k}")
    qt = fp4.fp4_quantize_act(to_dev(bits), f, layout=fp4.TILED)
    assert_canonical_equal(fp4.fp4_export_canonical(qt), ref, f, what=f"sweep tiled {m}x{k}")
    if fmt == "nvfp4":
        st = float(np.float32(0.37))
        ref_s = oracle.quantize(f, bits, mode=oracle.STATIC, static_scale=st)
        qs = fp4.fp4_quantize_act(to_dev(bits), f, layout=fp4.TILED,
                                  static_scale=torch.tensor([st], dtype=torch.float32, device="cuda"))
        assert_canonical_equal(fp4.fp4_export_canonical(qs), ref_s, f, what=f"sweep static {m}x{k}")


def test_mid_size_give_up_is_visible():
    """The one-pass mid-size quantizer's exchange gives up visibly, as the
    single-launch one does (forced from the host with a wait of zero polls):
    NaN tensor scale and linear outputs, the sticky flag set until cleared;
    the same workspaces then give the oracle's results."""
    m, k, n = 4096, 3072, 64
    print(f"[quant-mid] give-up m={m} k={k}", flush=True)
    a = synth.normal((m, k), 1.0, 22, 5)
    w = synth.normal((n, k), 0.02, 22, 6)
    assert fp4.fp4_linear_launches(fp4.NVFP4, m, n, k) == 2
    wq = fp4.fp4_quantize_weight(to_dev(w), fp4.NVFP4)
    x = to_dev(a)
    ws_q = torch.zeros(fp4.lib().fp4_quantize_workspace_bytes(fp4.NVFP4, m, k), dtype=torch.uint8,
                       device="cuda")
    ws_l = torch.zeros(fp4.fp4_linear_workspace_bytes(fp4.NVFP4, m, n, k), dtype=torch.uint8,
                       device="cuda")
    prev = fp4.fp4_set_exchange_spin_limit(0)
    try:
        q = fp4.fp4_quantize_act(x, fp4.NVFP4, layout=fp4.TILED, workspace=ws_q)
        y = fp4.fp4_linear(x, wq, workspace=ws_l)
        torch.cuda.synchronize()
    finally:
        fp4.fp4_set_exchange_spin_limit(prev)
    assert np.isnan(q.tensor_scale.cpu().item())
    assert torch.isnan(y.float()).all()
    assert fp4.fp4_workspace_flags(ws_q, clear=True) == fp4.WS_EXCHANGE_TIMEOUT
    assert fp4.fp4_workspace_flags(ws_l, clear=True) == fp4.WS_EXCHANGE_TIMEOUT
    ref = oracle.quantize(oracle.NVFP4, a)
    q2 = fp4.fp4_quantize_act(x, fp4.NVFP4, layout=fp4.TILED, workspace=ws_q)
    assert_canonical_equal(fp4.fp4_export_canonical(q2), ref, oracle.NVFP4, what="mid-size after a give-up")
    c_ref, l_ref = oracle.gemm(ref, oracle.quantize(oracle.NVFP4, w))
    y2 = fp4.fp4_linear(x, wq, workspace=ws_l).float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(y2 - c_ref) <= oracle.gemm_tolerance(c_ref, l_ref))
    assert fp4.fp4_workspace_flags(ws_q) == 0 and fp4.fp4_workspace_flags(ws_l) == 0


def test_workspace_shared_across_calls():
    """One zero-filled workspace serves a sequence of dynamic NVFP4 calls of
    different shapes and every code path (single launch, one-pass mid-size
    in the tiled layout, two passes): the max-exchange words recycle."""
    ws = torch.zeros(fp4.lib().fp4_quantize_workspace_bytes(0, 1, 16), dtype=torch.uint8, device="cuda")
    shapes = [(1, 5120), (32, 17408), (4, 64), (96, 32768), (8, 256), (1, 16), (300, 2880), (1000, 3008),
              (2, 96)]
    for rep in range(2):
        for i, (m, k) in enumerate(shapes):
            bits = synth.normal((m, k), 0.5 + i, 16, rep * 100 + i)
            ref = oracle.quantize_nvfp4(bits)
            q = fp4.fp4_quantize_act(to_dev(bits), 0, workspace=ws)
            assert_canonical_equal(q, ref, 0, what=f"shared workspace call {rep}/{i} {m}x{k}")
            # the tiled layout (rows padded to 16: another grid size) on the same words
            qt = fp4.fp4_quantize_act(to_dev(bits), 0, layout=fp4.TILED, workspace=ws)
            assert_canonical_equal(fp4.fp4_export_canonical(qt), ref, 0,
                                   what=f"shared workspace tiled call {rep}/{i} {m}x{k}")


@pytest.mark.parametrize("m,k", [(32, 5120), (32, 17408)])
def test_exchange_give_up_is_visible(m, k):
    """The single-launch NVFP4 quantizer's workgroups wait (bounded) for each
    other's maxima. A workgroup that gives up must not encode with a stale
    maximum: the call's tensor scale is NaN (so is every product made with it)
    and the workspace's sticky flag is set until cleared. Forced from the host
    with a wait of zero polls, so that no kernel waits at all; the same
    workspaces then serve correct calls."""
    n = 256
    print(f"[quant-act] exchange give-up m={m} k={k}", flush=True)
    a = synth.normal((m, k), 1.0, 21, m + k)
    w = synth.normal((n, k), 0.02, 21, 2)
    prev_fusion = fp4.fp4_set_decode_linear_fusion(False)   # the two-launch linear
    try:
        assert fp4.fp4_linear_launches(fp4.NVFP4, m, n, k) == 2   # quantizer with the exchange
        _exchange_give_up(m, k, n, a, w)
    finally:
        fp4.fp4_set_decode_linear_fusion(prev_fusion)


def _exchange_give_up(m, k, n, a, w):
    wq = fp4.fp4_quantize_weight(to_dev(w), fp4.NVFP4)
    x = to_dev(a)
    ws_q = torch.zeros(fp4.lib().fp4_quantize_workspace_bytes(fp4.NVFP4, m, k), dtype=torch.uint8,
                       device="cuda")
    ws_l = torch.zeros(fp4.fp4_linear_workspace_bytes(fp4.NVFP4, m, n, k), dtype=torch.uint8,
                       device="cuda")
    prev = fp4.fp4_set_exchange_spin_limit(0)
    try:
        q = fp4.fp4_quantize_act(x, fp4.NVFP4, workspace=ws_q)
        y = fp4.fp4_linear(x, wq, workspace=ws_l)
        torch.cuda.synchronize()
    finally:
        fp4.fp4_set_exchange_spin_limit(prev)
    assert np.isnan(q.tensor_scale.cpu().item())
    assert torch.isnan(y.float()).all()
    assert fp4.fp4_workspace_flags(ws_q) == fp4.WS_EXCHANGE_TIMEOUT
    assert fp4.fp4_workspace_flags(ws_l, clear=True) == fp4.WS_EXCHANGE_TIMEOUT
    assert fp4.fp4_workspace_flags(ws_l) == 0
    assert fp4.fp4_workspace_flags(ws_q, clear=True) == fp4.WS_EXCHANGE_TIMEOUT
    # with the default wait the same workspaces give the oracle's results
    ref = oracle.quantize(oracle.NVFP4, a)
    q2 = fp4.fp4_quantize_act(x, fp4.NVFP4, workspace=ws_q)
    assert_canonical_equal(q2, ref, oracle.NVFP4, what="after a give-up")
    c_ref, l_ref = oracle.gemm(ref, oracle.quantize(oracle.NVFP4, w))
    y2 = fp4.fp4_linear(x, wq, workspace=ws_l).float().cpu().numpy().astype(np.float64)
    tol = oracle.gemm_tolerance(c_ref, l_ref)
    assert np.all(np.abs(y2 - c_ref) <= tol)
    assert fp4.fp4_workspace_flags(ws_q) == 0 and fp4.fp4_workspace_flags(ws_l) == 0
