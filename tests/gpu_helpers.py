"""Shared helpers of the GPU parity tests (host side only)."""
import numpy as np
import torch

import oracle

F = {"nvfp4": oracle.NVFP4, "mxfp4": oracle.MXFP4}


def to_dev(bits: np.ndarray) -> torch.Tensor:
    """bf16 bit patterns (uint16) -> bf16 CUDA tensor with the same bytes."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def canon_to_host(q):
    """GPU canonical tensor -> (codes [R, pitch], scales [R, spitch], ts) numpy."""
    torch.cuda.synchronize()
    return (q.codes_2d().cpu().numpy(), q.scales_2d().cpu().numpy(),
            np.float32(q.tensor_scale.cpu().item()))


def assert_canonical_equal(q_gpu, q_ref: "oracle.Quantized", fmt: int, check_ts=True, what=""):
    codes, scales, ts = canon_to_host(q_gpu)
    k = q_ref.k
    bs = oracle.BLOCK[fmt]
    rows = q_ref.rows
    c_diff = np.argwhere(codes[:, : k // 2] != q_ref.codes)
    s_diff = np.argwhere(scales[:, : k // bs] != q_ref.scales)
    msg = f"{what}: {len(c_diff)} code bytes and {len(s_diff)} scale bytes differ"
    if len(c_diff):
        r, j = c_diff[0]
        msg += f"; first code diff row {r} byte {j}: gpu {codes[r, j]:#04x} ref {q_ref.codes[r, j]:#04x}"
    if len(s_diff):
        r, j = s_diff[0]
        msg += f"; first scale diff row {r} block {j}: gpu {scales[r, j]:#04x} ref {q_ref.scales[r, j]:#04x}"
    assert len(c_diff) == 0 and len(s_diff) == 0, msg
    assert np.all(codes[:, k // 2:] == 0), f"{what}: nonzero code padding"
    assert np.all(scales[:, k // bs:] == 0), f"{what}: nonzero scale padding"
    assert codes.shape[0] == rows
    if check_ts and fmt == oracle.NVFP4:
        assert ts == q_ref.tensor_scale, f"{what}: tensor scale gpu {ts!r} ref {q_ref.tensor_scale!r}"


def bf16_out_to_f64(y: torch.Tensor) -> np.ndarray:
    return y.float().cpu().numpy().astype(np.float64)


def assert_gemm_close(c_gpu: np.ndarray, c_ref: np.ndarray, l_ref: np.ndarray, what=""):
    tol = oracle.gemm_tolerance(c_ref, l_ref)
    err = np.abs(c_gpu - c_ref)
    bad = err > tol
    if bad.any():
        idx = np.argwhere(bad)[0]
        raise AssertionError(
            f"{what}: {bad.sum()} of {bad.size} outputs outside tolerance; first at {tuple(idx)}: "
            f"gpu {c_gpu[tuple(idx)]!r} ref {c_ref[tuple(idx)]!r} tol {tol[tuple(idx)]!r}")


def mid_rule(m, n, k, cap=12 << 20):
    """The slice count the mid-size kernel takes a shape with, restated: at
    most one workgroup of four weight tiles per CU (256), at least four
    fragments of K a slice, partial sums within `cap`, and used only with at
    least 32 fragments a slice (8 a wave); 0 when it does not apply."""
    if not 33 <= m <= 128:
        return 0
    kt, nt = -(-k // 128), -(-n // 16)
    ncol = -(-nt // 4)
    s = min(max(1, 256 // ncol), max(1, kt // 4))
    while s > 1 and s * m * n * 4 > cap:
        s -= 1
    return s if -(-kt // s) >= 32 else 0
