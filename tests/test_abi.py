"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, sizes its buffers as documented and rejects bad arguments on the host
before touching a device."""
import ctypes
import os
import re

import pytest

import block_scaled_fp4_quantize_amd as fp4

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "fp4.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(fp4_[a-z_0-9]+)\s*\(", src)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    L = fp4.lib()
    names = declared_functions()
    assert len(names) >= 15
    for name in names:
        assert hasattr(L, name), name


def test_sizes_and_pitches():
    L = fp4.lib()
    # canonical: rows x K_pad/2 codes, rows x K_pad/B scales; K_pad = round_up(K, 128)
    assert L.fp4_codes_bytes(fp4.NVFP4, fp4.CANONICAL, 3, 2880) == 3 * 2944 // 2
    assert L.fp4_scales_bytes(fp4.NVFP4, fp4.CANONICAL, 3, 2880) == 3 * 2944 // 16
    assert L.fp4_scales_bytes(fp4.MXFP4, fp4.CANONICAL, 3, 2880) == 3 * 2944 // 32
    # tiled: rows padded to 16
    assert L.fp4_codes_bytes(fp4.NVFP4, fp4.TILED, 17, 256) == 32 * 128
    assert L.fp4_scales_bytes(fp4.MXFP4, fp4.TILED, 17, 256) == 32 * 8
    # 4.5 and 4.25 bits per value when nothing is padded
    k, n = 5120, 5120
    for fmt, bits in ((fp4.NVFP4, 4.5), (fp4.MXFP4, 4.25)):
        tot = L.fp4_codes_bytes(fmt, fp4.TILED, n, k) + L.fp4_scales_bytes(fmt, fp4.TILED, n, k)
        assert tot * 8 / (n * k) == bits
    assert L.fp4_block_size(fp4.NVFP4) == 16 and L.fp4_block_size(fp4.MXFP4) == 32
    assert L.fp4_block_size(7) == 0
    assert L.fp4_codes_bytes(9, 0, 4, 32) == 0
    assert L.fp4_quantize_workspace_bytes(fp4.NVFP4, 8, 64) >= 4096
    assert L.fp4_quantize_workspace_bytes(fp4.MXFP4, 8, 64) == 0
    assert L.fp4_gemm_workspace_bytes(fp4.NVFP4, 8, 64, 64) == 0
    assert L.fp4_gemm_workspace_bytes(fp4.NVFP4, 128, 64, 64) == 0
    # M > 128: a tiled copy of the activations (rows padded to 16, K to 128)
    assert L.fp4_gemm_workspace_bytes(fp4.NVFP4, 200, 64, 2880) >= 208 * 2944 // 2 + 208 * 2944 // 16
    assert L.fp4_gemm_workspace_bytes(fp4.MXFP4, 200, 64, 2880) >= 208 * 2944 // 2 + 208 * 2944 // 32
    assert L.fp4_linear_workspace_bytes(fp4.NVFP4, 8, 5120, 5120) > 0


def test_mid_gemm_workspace_and_launches():
    """33-128 rows on large weights: the mid-size GEMM, at most one workgroup
    per CU (64 output columns each) and K split so that each of its four waves
    streams at least 8 fragments; its FP32 partial sums (splits * M * N
    floats, at most 12 MiB) sit in the GEMM and linear workspaces, and a
    combining launch adds them. Smaller shapes keep the skinny kernel."""
    L = fp4.lib()
    mib = 1 << 20
    # K x N = 17408 x 5120: 80 column groups -> 3 slices of 46 fragments
    assert L.fp4_gemm_workspace_bytes(fp4.NVFP4, 128, 5120, 17408) == 3 * 128 * 5120 * 4
    assert L.fp4_gemm_workspace_bytes(fp4.MXFP4, 64, 5120, 17408) == 3 * 64 * 5120 * 4
    # K x N = 5120 x 17408: 272 column groups -> one slice of 40 fragments
    assert L.fp4_gemm_workspace_bytes(fp4.NVFP4, 128, 17408, 5120) == 0
    # macro-block scales and 32 rows keep the skinny kernel
    assert L.fp4_gemm_workspace_bytes(fp4.MXFP4 | fp4.MX_MBS, 128, 5120, 17408) == 0
    assert L.fp4_gemm_workspace_bytes(fp4.NVFP4, 32, 5120, 17408) == 0
    # which GEMM fp4_linear runs: slices of the mid-size kernel, 0 for another
    assert L.fp4_linear_mid_splits(fp4.NVFP4, 128, 5120, 17408) == 3
    assert L.fp4_linear_mid_splits(fp4.MXFP4, 65, 17408, 5120) == 1
    assert L.fp4_linear_mid_splits(fp4.NVFP4, 128, 5760, 2880) == 0
    assert L.fp4_linear_mid_splits(fp4.NVFP4, 32, 5120, 17408) == 0
    assert L.fp4_linear_mid_splits(fp4.NVFP4, 129, 5120, 17408) == 0
    assert L.fp4_linear_mid_splits(fp4.MXFP4 | fp4.MX_MBS, 128, 5120, 17408) == 0
    assert L.fp4_linear_mid_splits(fp4.NVFP4, 128, 5120, 17400) == 0   # K % 16
    prev = L.fp4_set_mid_gemm(0)
    try:
        assert L.fp4_linear_mid_splits(fp4.NVFP4, 128, 5120, 17408) == 0
    finally:
        L.fp4_set_mid_gemm(prev)
    # (K, N) -> fp4_linear's launches: quantize, GEMM, and the combine for 3 slices
    mid = {(5120, 17408): 2, (17408, 5120): 3}
    for fmt in (fp4.NVFP4, fp4.MXFP4):
        for m in (33, 64, 128):
            for (k, n) in ((2880, 4096), (2880, 512), (4096, 2880), (2880, 5760), (5760, 2880),
                           (5120, 5120), (5120, 17408), (17408, 5120)):
                g = L.fp4_gemm_workspace_bytes(fmt, m, n, k)
                assert g <= 12 * mib
                lin = L.fp4_linear_workspace_bytes(fmt, m, n, k)
                assert lin >= g
                # every such linear still fits the allocation-free array
                assert lin <= fp4.NOALLOC_SCRATCH_BYTES
                assert L.fp4_linear_launches(fmt, m, n, k, 0) == mid.get((k, n), 2)
                prev = L.fp4_set_mid_gemm(0)
                try:
                    assert L.fp4_linear_launches(fmt, m, n, k, 0) == 2
                finally:
                    assert L.fp4_set_mid_gemm(prev) == 0


def test_mid_gemm_rule_on_seeded_shapes():
    """The library's choice of the mid-size GEMM and its slice count equal the
    rule restated in the tests, on 2000 seeded shapes of 1-200 rows."""
    import numpy as np
    from tests.gpu_helpers import mid_rule
    L = fp4.lib()
    g = np.random.default_rng(7)
    for _ in range(2000):
        m, n, k = int(g.integers(1, 201)), int(g.integers(1, 40000)), int(g.integers(1, 700)) * 32
        want = mid_rule(m, n, k)
        for f in (fp4.NVFP4, fp4.MXFP4):
            assert L.fp4_linear_mid_splits(f, m, n, k) == want, (f, m, n, k)


def test_tensor_init_fills_pitches():
    L = fp4.lib()
    t = fp4.fp4_tensor()
    assert L.fp4_tensor_init(ctypes.byref(t), fp4.NVFP4, fp4.CANONICAL, 5, 2880, 16, 32, 64) == 0
    assert t.codes_pitch == 1472 and t.scales_pitch == 184 and t.rows == 5 and t.cols == 2880
    assert L.fp4_tensor_init(ctypes.byref(t), fp4.MXFP4, fp4.CANONICAL, 5, 48, 16, 32, 0) == 2
    assert b"block size 32" in L.fp4_last_error()


def _status(name):
    return {0: "FP4_OK", 1: "FP4_ERR_INVALID_ARG", 2: "FP4_ERR_SHAPE", 3: "FP4_ERR_ALIGNMENT",
            4: "FP4_ERR_WORKSPACE", 5: "FP4_ERR_FORMAT_MISMATCH", 6: "FP4_ERR_DEVICE",
            7: "FP4_ERR_HIP"}[name]


def test_status_strings():
    L = fp4.lib()
    for s in range(8):
        assert L.fp4_status_string(s).decode() == _status(s)


def test_host_validation_rejects_before_launch():
    """Each error path returns its status without reaching the device check."""
    L = fp4.lib()
    good = fp4.fp4_tensor()
    assert L.fp4_tensor_init(ctypes.byref(good), fp4.NVFP4, fp4.CANONICAL, 4, 64, 4096, 8192, 64) == 0
    w = fp4.fp4_tensor()
    assert L.fp4_tensor_init(ctypes.byref(w), fp4.NVFP4, fp4.TILED, 32, 64, 4096, 8192, 64) == 0
    # null input
    assert L.fp4_quantize_act(0, None, 4, 64, None, ctypes.byref(good), 1024, 4096, None) == 1
    # K not a multiple of the block
    assert L.fp4_quantize_act(0, 4096, 4, 40, None, ctypes.byref(good), 1024, 4096, None) == 2
    # misaligned input
    assert L.fp4_quantize_act(0, 4097, 4, 64, None, ctypes.byref(good), 1024, 4096, None) == 3
    # workspace too small for the dynamic scale
    assert L.fp4_quantize_act(0, 4096, 4, 64, None, ctypes.byref(good), 1024, 16, None) == 4
    # MXFP4 with a static scale
    mx = fp4.fp4_tensor()
    assert L.fp4_tensor_init(ctypes.byref(mx), fp4.MXFP4, fp4.CANONICAL, 4, 64, 4096, 8192, 0) == 0
    assert L.fp4_quantize_act(1, 4096, 4, 64, 64, ctypes.byref(mx), 0, 0, None) == 1
    # descriptor of another shape
    assert L.fp4_quantize_act(0, 4096, 16, 64, None, ctypes.byref(w), 1024, 8192, None) == 5
    # weights go to the tiled layout only
    assert L.fp4_quantize_weight(0, 4096, 4, 64, ctypes.byref(good), 1024, 8192, None) == 5
    # gemm: format mismatch, K mismatch, null output, small ldc
    wmx = fp4.fp4_tensor()
    assert L.fp4_tensor_init(ctypes.byref(wmx), fp4.MXFP4, fp4.TILED, 32, 64, 4096, 8192, 0) == 0
    assert L.fp4_gemm(ctypes.byref(good), ctypes.byref(wmx), 4096, 32, None, 0, None) == 5
    w128 = fp4.fp4_tensor()
    assert L.fp4_tensor_init(ctypes.byref(w128), fp4.NVFP4, fp4.TILED, 32, 128, 4096, 8192, 64) == 0
    assert L.fp4_gemm(ctypes.byref(good), ctypes.byref(w128), 4096, 32, None, 0, None) == 2
    assert L.fp4_gemm(ctypes.byref(good), ctypes.byref(w), None, 32, None, 0, None) == 1
    assert L.fp4_gemm(ctypes.byref(good), ctypes.byref(w), 4096, 16, None, 0, None) == 2
    # linear: workspace missing
    assert L.fp4_linear(4096, 4, ctypes.byref(w), None, 8192, None, 0, None) == 4
    # NVFP4 descriptor without a tensor scale
    bad = fp4.fp4_tensor()
    assert L.fp4_tensor_init(ctypes.byref(bad), fp4.NVFP4, fp4.CANONICAL, 4, 64, 4096, 8192, None) == 0
    assert L.fp4_gemm(ctypes.byref(bad), ctypes.byref(w), 4096, 32, None, 0, None) == 1
    assert b"tensor_scale" in L.fp4_last_error()
    # skinny path: canonical activation rows addressed past 2^31 bytes
    wide = fp4.fp4_tensor()
    assert L.fp4_tensor_init(ctypes.byref(wide), fp4.NVFP4, fp4.CANONICAL, 4, 64, 4096, 8192, 64) == 0
    wide.codes_pitch = 1 << 29
    assert L.fp4_gemm(ctypes.byref(wide), ctypes.byref(w), 4096, 32, None, 0, None) == 2
    assert b"2^31" in L.fp4_last_error()


def test_linear_launch_count():
    L = fp4.lib()
    # M = 1 decode shapes run as one fused launch (NVFP4: M * K_pad * tiles up
    # to 8M for one row; up to 4M and at most 512 weight tiles for more rows,
    # where the per-workgroup encode would otherwise repeat too often)
    for k, n in ((5120, 5120), (5120, 17408), (17408, 5120)):
        assert L.fp4_linear_launches(fp4.NVFP4, 1, n, k, 0) == 1
        assert L.fp4_linear_launches(fp4.MXFP4, 1, n, k, 0) == 1
    assert L.fp4_linear_launches(fp4.NVFP4, 1, 8192, 16384, 0) == 1
    assert L.fp4_linear_launches(fp4.NVFP4, 1, 8208, 16384, 0) == 2
    assert L.fp4_linear_launches(fp4.NVFP4, 2, 5120, 5120, 0) == 1
    assert L.fp4_linear_launches(fp4.NVFP4, 2, 17408, 5120, 0) == 2
    assert L.fp4_linear_launches(fp4.NVFP4, 4, 5120, 5120, 0) == 2
    # larger activations: quantize + GEMM (NVFP4 dynamic past 16384 fragments,
    # or rotated past the single-launch size, needs a reduction launch)
    assert L.fp4_linear_launches(fp4.NVFP4, 32, 5120, 5120, 0) == 2
    assert L.fp4_linear_launches(fp4.NVFP4, 4096, 3072, 3072, 0) == 2
    assert L.fp4_linear_launches(fp4.NVFP4, 4096, 3072, 8192, 0) == 2
    assert L.fp4_linear_launches(fp4.NVFP4, 4112, 3072, 8192, 0) == 3
    assert L.fp4_linear_launches(fp4.NVFP4 | fp4.ROTATE, 4096, 3072, 3072, 0) == 3
    assert L.fp4_linear_launches(fp4.NVFP4, 16384, 16384, 16384, 0) == 3
    # 1-32 rows with producer workgroups inside the skinny GEMM's launch, once
    # switched on; rotated and macro-block-scaled activations excepted
    prev = L.fp4_set_decode_linear_fusion(1)
    assert prev == 0
    try:
        for k, n in ((5120, 5120), (5120, 17408), (17408, 5120)):
            for m in (1, 2, 4, 8, 32):
                assert L.fp4_linear_launches(fp4.NVFP4, m, n, k, 0) == 1
                assert L.fp4_linear_launches(fp4.MXFP4, m, n, k, 0) == 1
                assert L.fp4_linear_launches(fp4.NVFP4, m, n, k, 1) == 1
        assert L.fp4_linear_launches(fp4.NVFP4 | fp4.ROTATE, 8, 5120, 5120, 0) == 2
        assert L.fp4_linear_launches(fp4.MXFP4 | fp4.MX_MBS, 8, 5120, 5120, 0) == 2
        assert L.fp4_linear_launches(fp4.MXFP4 | fp4.MX_OAS, 8, 5120, 5120, 0) == 1
        assert L.fp4_linear_launches(fp4.NVFP4, 33, 5120, 5120, 0) == 2
        # at most 1024 activation fragments (128 producers of eight waves)
        assert L.fp4_linear_launches(fp4.MXFP4, 32, 256, 65536, 0) == 1
        assert L.fp4_linear_launches(fp4.MXFP4, 32, 256, 65536 + 128, 0) == 2
        assert L.fp4_linear_launches(fp4.NVFP4, 16, 256, 2 * 65536, 1) == 1
    finally:
        assert L.fp4_set_decode_linear_fusion(prev) == 1
    # large M with a static scale (NVFP4) or MXFP4: quantize + GEMM by default,
    # quantization inside the GEMM launch once fusion is switched on
    assert L.fp4_linear_launches(fp4.NVFP4, 4096, 3072, 3072, 1) == 2
    assert L.fp4_linear_launches(fp4.MXFP4, 4096, 3072, 3072, 0) == 2
    prev = L.fp4_set_large_linear_fusion(1)
    assert prev == 0
    try:
        assert L.fp4_linear_launches(fp4.NVFP4, 4096, 3072, 3072, 1) == 1
        assert L.fp4_linear_launches(fp4.MXFP4, 4096, 3072, 3072, 0) == 1
        assert L.fp4_linear_launches(fp4.MXFP4 | fp4.MX_MBS, 4096, 3072, 3072, 0) == 2
        assert L.fp4_linear_launches(fp4.NVFP4, 4096, 3072, 3072, 0) == 2
        assert L.fp4_linear_launches(fp4.NVFP4, 8192, 3072, 8192, 0) == 3
    finally:
        assert L.fp4_set_large_linear_fusion(prev) == 1
    assert L.fp4_linear_launches(fp4.NVFP4, 4, 64, 40, 0) == 0


def test_recipe_flags_validation():
    """Recipe flags ride in the format value: sizes ignore them, bad
    combinations are rejected, and a rotated operand never meets an unrotated
    one in a GEMM."""
    L = fp4.lib()
    for base in (fp4.NVFP4, fp4.MXFP4):
        for flags in (fp4.ROTATE,):
            assert L.fp4_codes_bytes(base | flags, fp4.TILED, 17, 256) == L.fp4_codes_bytes(base, fp4.TILED, 17, 256)
            assert L.fp4_scales_bytes(base | flags, fp4.CANONICAL, 3, 2880) == L.fp4_scales_bytes(base, fp4.CANONICAL, 3, 2880)
            assert L.fp4_block_size(base | flags) == L.fp4_block_size(base)
    assert L.fp4_block_size(fp4.MXFP4 | fp4.MX_OAS | fp4.ROTATE) == 32
    # OAS is an MXFP4 rule; unknown bits are rejected
    assert L.fp4_block_size(fp4.NVFP4 | fp4.MX_OAS) == 0
    assert L.fp4_block_size(fp4.MXFP4 | 0x800) == 0
    t = fp4.fp4_tensor()
    assert L.fp4_tensor_init(ctypes.byref(t), fp4.NVFP4 | fp4.MX_OAS, fp4.CANONICAL, 4, 64, 4096, 8192, 64) == 1
    # a rotated activation with an unrotated weight (and the reverse)
    a_rot, w_rot, a, w = fp4.fp4_tensor(), fp4.fp4_tensor(), fp4.fp4_tensor(), fp4.fp4_tensor()
    assert L.fp4_tensor_init(ctypes.byref(a_rot), fp4.MXFP4 | fp4.ROTATE, fp4.CANONICAL, 4, 64, 4096, 8192, 0) == 0
    assert L.fp4_tensor_init(ctypes.byref(w_rot), fp4.MXFP4 | fp4.ROTATE, fp4.TILED, 32, 64, 4096, 8192, 0) == 0
    assert L.fp4_tensor_init(ctypes.byref(a), fp4.MXFP4, fp4.CANONICAL, 4, 64, 4096, 8192, 0) == 0
    assert L.fp4_tensor_init(ctypes.byref(w), fp4.MXFP4 | fp4.MX_OAS, fp4.TILED, 32, 64, 4096, 8192, 0) == 0
    assert L.fp4_gemm(ctypes.byref(a_rot), ctypes.byref(w), 4096, 32, None, 0, None) == 5
    assert b"rotation" in L.fp4_last_error()
    assert L.fp4_gemm(ctypes.byref(a), ctypes.byref(w_rot), 4096, 32, None, 0, None) == 5
    # the binding's string form
    assert fp4._fmt("mxfp4+rotate+oas") == fp4.MXFP4 | fp4.ROTATE | fp4.MX_OAS
    assert fp4._fmt("nvfp4+rotate") == fp4.NVFP4 | fp4.ROTATE
    with pytest.raises(ValueError):
        fp4._fmt(fp4.MXFP4 | 0x800)


def test_w4a16_host_validation():
    L = fp4.lib()
    w = fp4.fp4_tensor()
    assert L.fp4_tensor_init(ctypes.byref(w), fp4.NVFP4, fp4.TILED, 32, 64, 4096, 8192, 64) == 0
    wr = fp4.fp4_tensor()
    assert L.fp4_tensor_init(ctypes.byref(wr), fp4.MXFP4 | fp4.ROTATE, fp4.TILED, 32, 64, 4096, 8192, 0) == 0
    assert L.fp4_linear_w4a16(4096, 4, ctypes.byref(wr), 8192, 32, None) == 5     # rotated weight
    assert b"rotated" in L.fp4_last_error()
    assert L.fp4_linear_w4a16(None, 4, ctypes.byref(w), 8192, 32, None) == 1      # null input
    assert L.fp4_linear_w4a16(4097, 4, ctypes.byref(w), 8192, 32, None) == 3      # misaligned
    assert L.fp4_linear_w4a16(4096, 4, ctypes.byref(w), 8192, 16, None) == 2      # ldy < N
    assert L.fp4_linear_w4a16(4096, 0, ctypes.byref(w), 8192, 32, None) == 1      # m = 0
    c = fp4.fp4_tensor()
    assert L.fp4_tensor_init(ctypes.byref(c), fp4.NVFP4, fp4.CANONICAL, 32, 64, 4096, 8192, 64) == 0
    assert L.fp4_linear_w4a16(4096, 4, ctypes.byref(c), 8192, 32, None) == 5      # not tiled


def test_last_error_is_per_thread():
    """fp4_last_error() belongs to the calling thread: threads that fail in
    different ways, interleaved, each read their own message."""
    import threading
    L = fp4.lib()
    desc = fp4.fp4_tensor()
    assert L.fp4_tensor_init(ctypes.byref(desc), fp4.NVFP4, fp4.CANONICAL, 4, 64, 4096, 8192, 64) == 0
    results, barrier = {}, threading.Barrier(8)

    def worker(i):
        barrier.wait()
        out = []
        for _ in range(200):
            if i % 2 == 0:   # null activations
                st = L.fp4_quantize_act(0, None, 4, 64, None, ctypes.byref(desc), 1024, 4096, None)
            else:            # K not a multiple of the block
                st = L.fp4_quantize_act(0, 4096, 4, 40, None, ctypes.byref(desc), 1024, 4096, None)
            out.append((st, L.fp4_last_error()))
        results[i] = out

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    for i, out in results.items():
        for st, msg in out:
            if i % 2 == 0:
                assert st == 1 and b"null" in msg, msg
            else:
                assert st == 2 and b"multiple" in msg, msg


def test_workspace_flags_and_spin_limit_host_side():
    """The flag query validates on the host; the spin-limit hook returns the
    previous value (no device needed for either)."""
    L = fp4.lib()
    flags = ctypes.c_uint32(7)
    assert L.fp4_workspace_flags(None, 1 << 20, ctypes.byref(flags), 0, None) == 1
    buf = ctypes.create_string_buffer(64)
    assert L.fp4_workspace_flags(buf, 64, ctypes.byref(flags), 0, None) == 4
    assert b"flags" in L.fp4_last_error()
    assert L.fp4_workspace_flags(buf, 1 << 20, None, 0, None) == 1
    prev = L.fp4_set_exchange_spin_limit(5)
    assert prev == 1 << 22
    assert L.fp4_set_exchange_spin_limit(prev) == 5


def test_mbs_flag_sizes_and_validity():
    """MXFP4 | FP4_MX_MBS: the scales buffer also holds one float per row and
    128-value segment (tiled: 16 per fragment; canonical: after the E8M0 rows,
    16-byte aligned); NVFP4 rejects the flag."""
    L = fp4.lib()
    mbs = fp4.MXFP4 | fp4.MX_MBS
    assert L.fp4_scales_bytes(mbs, fp4.TILED, 17, 256) == 32 * 8 + 32 * 2 * 4
    assert L.fp4_scales_bytes(mbs, fp4.CANONICAL, 3, 2880) == 288 + 3 * 23 * 4   # round_up(3 * 92, 16)
    assert L.fp4_scales_bytes(fp4.NVFP4 | fp4.MX_MBS, fp4.TILED, 16, 256) == 0
    t = fp4.fp4_tensor()
    assert L.fp4_tensor_init(ctypes.byref(t), fp4.NVFP4 | fp4.MX_MBS, fp4.CANONICAL, 4, 64, 16, 32, 64) == 1
    assert L.fp4_tensor_init(ctypes.byref(t), mbs | fp4.ROTATE | fp4.MX_OAS, fp4.CANONICAL, 4, 64, 16, 32, 0) == 0
    assert L.fp4_linear_workspace_bytes(mbs, 8, 64, 5120) > L.fp4_linear_workspace_bytes(fp4.MXFP4, 8, 64, 5120)
