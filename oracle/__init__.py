"""CPU oracle for block-scaled FP4 quantization and GEMM (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It is a thin ctypes wrapper over the plain
C implementation in ``fp4_oracle.c`` (binary64 and integer arithmetic, no shared
code with the GPU library); that file's header lists the passages of the pages
it follows and every reading taken where they are silent.

Conventions (the same as the C file):
  * inputs are bf16 bit patterns in ``numpy.uint16`` arrays, row-major;
  * codes are ``uint8`` ``[rows, k/2]`` with even k in the low nibble;
  * scales are ``uint8`` ``[rows, k/16]`` (E4M3, NVFP4) or ``[rows, k/32]``
    (E8M0, MXFP4);
  * NVFP4 also returns the FP32 per-tensor decode scale S_t.

Parity status: every function here is pinned by a test under ``tests/`` against
values the pages print, closed forms or brute force, except the MXFP4 block
exponent rule, which the pages do not print (pinned by invariants only). The
block rotation is pinned against an exact integer matrix product with the
library Sylvester Hadamard matrix and against closed forms; the OAS exponent
against a brute-force search.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

NVFP4, MXFP4 = 0, 1
DYNAMIC, STATIC, NAIVE = 0, 1, 2
BLOCK = {NVFP4: 16, MXFP4: 32}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libfp4oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with the host C compiler (plain C99, no fast-math)."""
    if not force and os.path.exists(_LIB_PATH) and (
        os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC)
    ):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-fPIC", "-shared",
           "-ffp-contract=off", "-fno-fast-math", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.orc_bf16_value.restype = ctypes.c_double
        lib.orc_bf16_value.argtypes = [ctypes.c_uint16]
        lib.orc_e2m1_value.restype = ctypes.c_double
        lib.orc_e2m1_value.argtypes = [ctypes.c_int]
        lib.orc_e4m3_value.restype = ctypes.c_double
        lib.orc_e4m3_value.argtypes = [ctypes.c_int]
        lib.orc_e8m0_value.restype = ctypes.c_double
        lib.orc_e8m0_value.argtypes = [ctypes.c_int]
        lib.orc_e4m3_from_real.restype = ctypes.c_int
        lib.orc_e4m3_from_real.argtypes = [ctypes.c_double, ctypes.c_int]
        lib.orc_e4m3_from_real_array.restype = None
        lib.orc_e4m3_from_real_array.argtypes = [P, I64, ctypes.c_int, P]
        lib.orc_mx_exponent.restype = ctypes.c_int
        lib.orc_mx_exponent.argtypes = [ctypes.c_double]
        lib.orc_amax.restype = ctypes.c_double
        lib.orc_amax.argtypes = [P, I64]
        lib.orc_tensor_scale.restype = ctypes.c_float
        lib.orc_tensor_scale.argtypes = [P, I64]
        lib.orc_quantize_nvfp4.restype = ctypes.c_int
        lib.orc_quantize_nvfp4.argtypes = [P, I64, I64, ctypes.c_int, ctypes.c_float,
                                           P, P, P]
        lib.orc_quantize_mxfp4.restype = ctypes.c_int
        lib.orc_quantize_mxfp4.argtypes = [P, I64, I64, P, P]
        lib.orc_quantize_mxfp4_rule.restype = ctypes.c_int
        lib.orc_quantize_mxfp4_rule.argtypes = [P, I64, I64, ctypes.c_int, P, P]
        lib.orc_mx_exponent_oas.restype = ctypes.c_int
        lib.orc_mx_exponent_oas.argtypes = [ctypes.c_double]
        lib.orc_mbs_scale.restype = ctypes.c_float
        lib.orc_mbs_scale.argtypes = [ctypes.c_double]
        lib.orc_mbs_exponent.restype = ctypes.c_int
        lib.orc_mbs_exponent.argtypes = [ctypes.c_double, ctypes.c_float, ctypes.c_int]
        lib.orc_quantize_mxfp4_mbs.restype = ctypes.c_int
        lib.orc_quantize_mxfp4_mbs.argtypes = [P, I64, I64, ctypes.c_int, P, P, P]
        lib.orc_dequantize_ms.restype = None
        lib.orc_dequantize_ms.argtypes = [ctypes.c_int, P, P, P, ctypes.c_float, I64, I64, P]
        lib.orc_gemm_ms.restype = None
        lib.orc_gemm_ms.argtypes = [ctypes.c_int, P, P, P, ctypes.c_float, P, P, P, ctypes.c_float,
                                    I64, I64, I64, P, P]
        lib.orc_gemm_sampled_ms.restype = None
        lib.orc_gemm_sampled_ms.argtypes = [ctypes.c_int, P, P, P, ctypes.c_float, P, P, P,
                                            ctypes.c_float, I64, P, P, I64, P, P]
        lib.orc_hadamard_norm.restype = ctypes.c_float
        lib.orc_hadamard_norm.argtypes = [ctypes.c_int]
        lib.orc_hadamard_bf16.restype = ctypes.c_int
        lib.orc_hadamard_bf16.argtypes = [P, I64, I64, ctypes.c_int, P]
        lib.orc_dequantize.restype = None
        lib.orc_dequantize.argtypes = [ctypes.c_int, P, P, ctypes.c_float, I64, I64, P]
        lib.orc_gemm.restype = None
        lib.orc_gemm.argtypes = [ctypes.c_int, P, P, ctypes.c_float, P, P, ctypes.c_float,
                                 I64, I64, I64, P, P]
        lib.orc_gemm_sampled.restype = None
        lib.orc_gemm_sampled.argtypes = [ctypes.c_int, P, P, ctypes.c_float, P, P,
                                         ctypes.c_float, I64, P, P, I64, P, P]
        lib.orc_gemm_w4a16.restype = None
        lib.orc_gemm_w4a16.argtypes = [ctypes.c_int, P, P, P, ctypes.c_float, I64, I64, I64,
                                       P, P]
        lib.orc_gemm_w4a16_sampled.restype = None
        lib.orc_gemm_w4a16_sampled.argtypes = [ctypes.c_int, P, P, P, ctypes.c_float, I64,
                                               P, P, I64, P, P]
        _lib = lib
        return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _bf16(x) -> np.ndarray:
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16:
        raise TypeError("oracle inputs are bf16 bit patterns (numpy.uint16)")
    if x.ndim != 2:
        raise ValueError("oracle inputs are 2-D [rows, k]")
    return x


class Quantized:
    """Canonical quantized tensor: codes [R, K/2], scales [R, K/B], tensor scale,
    and for MXFP4 with macro-block scaling the FP32 scales macro [R, ceil(K/128)]
    (None otherwise)."""

    def __init__(self, fmt, codes, scales, tensor_scale, k, macro=None):
        self.fmt = fmt
        self.codes = codes
        self.scales = scales
        self.tensor_scale = np.float32(tensor_scale)
        self.k = k
        self.macro = None if macro is None else np.ascontiguousarray(macro, dtype=np.float32)

    def row_slice(self, r0, r1):
        return Quantized(self.fmt, self.codes[r0:r1], self.scales[r0:r1], self.tensor_scale,
                         self.k, None if self.macro is None else self.macro[r0:r1])

    @property
    def rows(self):
        return self.codes.shape[0]


# ------------------------------------------------------------------ codecs

def bf16_value(bits: int) -> float:
    return _load().orc_bf16_value(int(bits))


def e2m1_value(code: int) -> float:
    return _load().orc_e2m1_value(int(code))


def e4m3_value(byte: int) -> float:
    return _load().orc_e4m3_value(int(byte))


def e8m0_value(byte: int) -> float:
    return _load().orc_e8m0_value(int(byte))


def e4m3_from_real(v, saturate: bool = True) -> np.ndarray:
    """Nearest E4M3 byte (ties to even) of non-negative reals given as float64."""
    v = np.ascontiguousarray(np.atleast_1d(v), dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint8)
    _load().orc_e4m3_from_real_array(_ptr(v), v.size, int(bool(saturate)), _ptr(out))
    return out


def mx_exponent(amax: float) -> int:
    return _load().orc_mx_exponent(float(amax))


def amax(x) -> float:
    x = np.ascontiguousarray(x, dtype=np.uint16)
    return _load().orc_amax(_ptr(x), x.size)


def tensor_scale(x) -> np.float32:
    x = np.ascontiguousarray(x, dtype=np.uint16)
    return np.float32(_load().orc_tensor_scale(_ptr(x), x.size))


# ------------------------------------------------------------ quantization

def quantize_nvfp4(x, mode: int = DYNAMIC, static_scale: float | None = None) -> Quantized:
    x = _bf16(x)
    r, k = x.shape
    codes = np.zeros((r, k // 2), dtype=np.uint8)
    scales = np.zeros((r, k // 16), dtype=np.uint8)
    ts = np.zeros(1, dtype=np.float32)
    st = 0.0 if static_scale is None else float(static_scale)
    rc = _load().orc_quantize_nvfp4(_ptr(x), r, k, mode, st, _ptr(codes), _ptr(scales),
                                    _ptr(ts))
    if rc != 0:
        raise ValueError("oracle NVFP4 quantize rejected its arguments")
    return Quantized(NVFP4, codes, scales, ts[0], k)


def quantize_mxfp4(x, oas: bool = False) -> Quantized:
    x = _bf16(x)
    r, k = x.shape
    codes = np.zeros((r, k // 2), dtype=np.uint8)
    scales = np.zeros((r, k // 32), dtype=np.uint8)
    rc = _load().orc_quantize_mxfp4_rule(_ptr(x), r, k, int(bool(oas)), _ptr(codes),
                                         _ptr(scales))
    if rc != 0:
        raise ValueError("oracle MXFP4 quantize rejected its arguments")
    return Quantized(MXFP4, codes, scales, 1.0, k)


def quantize_mxfp4_mbs(x, oas: bool = False) -> Quantized:
    """MXFP4 with macro-block scaling: 128-value segments along k each get an
    FP32 scale in [1, 2) (see the C file's header for the reading)."""
    x = _bf16(x)
    r, k = x.shape
    codes = np.zeros((r, k // 2), dtype=np.uint8)
    scales = np.zeros((r, k // 32), dtype=np.uint8)
    macro = np.zeros((r, (k + 127) // 128), dtype=np.float32)
    rc = _load().orc_quantize_mxfp4_mbs(_ptr(x), r, k, int(bool(oas)), _ptr(codes), _ptr(scales),
                                        _ptr(macro))
    if rc != 0:
        raise ValueError("oracle MXFP4 (MBS) quantize rejected its arguments")
    return Quantized(MXFP4, codes, scales, 1.0, k, macro)


def mbs_scale(g: float) -> np.float32:
    return np.float32(_load().orc_mbs_scale(float(g)))


def mbs_exponent(ab: float, s, oas: bool = False) -> int:
    return _load().orc_mbs_exponent(float(ab), float(s), int(bool(oas)))


def mx_exponent_oas(amax: float) -> int:
    """Overflow-aware MXFP4 block exponent (smallest e with amax <= 6 * 2^e)."""
    return _load().orc_mx_exponent_oas(float(amax))


def hadamard_norm(bs: int) -> np.float32:
    return np.float32(_load().orc_hadamard_norm(int(bs)))


def hadamard(x, bs: int) -> np.ndarray:
    """Block rotation of bf16 rows: H_bs x / sqrt(bs) per block of bs values
    along k, binary32 fast transform, rounded to bf16 (uint16 bit patterns)."""
    x = _bf16(x)
    r, k = x.shape
    out = np.zeros((r, k), dtype=np.uint16)
    rc = _load().orc_hadamard_bf16(_ptr(x), r, k, int(bs), _ptr(out))
    if rc != 0:
        raise ValueError("oracle rotation rejected its arguments")
    return out


def quantize(fmt: int, x, mode: int = DYNAMIC, static_scale=None, rotate: bool = False,
             oas: bool = False, mbs: bool = False) -> Quantized:
    """Quantize x; rotate=True applies the block rotation (size = the block)
    first; oas=True (MXFP4) takes the overflow-aware block exponent; mbs=True
    (MXFP4) adds the macro-block scales."""
    if rotate:
        x = hadamard(x, BLOCK[fmt])
    if fmt == NVFP4:
        if oas or mbs:
            raise ValueError("OAS and MBS are MXFP4 scale rules")
        return quantize_nvfp4(x, mode, static_scale)
    if mode != DYNAMIC or static_scale is not None:
        raise ValueError("MXFP4 has no per-tensor scale")
    return quantize_mxfp4_mbs(x, oas) if mbs else quantize_mxfp4(x, oas)


def _mptr(q: Quantized):
    return None if q.macro is None else _ptr(q.macro)


def dequantize(q: Quantized) -> np.ndarray:
    """x^ in binary64, [R, K] (includes the NVFP4 per-tensor factor and the
    macro-block scales)."""
    out = np.empty((q.rows, q.k), dtype=np.float64)
    _load().orc_dequantize_ms(q.fmt, _ptr(q.codes), _ptr(q.scales), _mptr(q),
                              float(q.tensor_scale), q.rows, q.k, _ptr(out))
    return out


def _unit(q: Quantized) -> np.ndarray:
    """q * s_b (times S_mb) without the per-tensor factor (what the GEMM contracts)."""
    out = np.empty((q.rows, q.k), dtype=np.float64)
    _load().orc_dequantize_ms(q.fmt, _ptr(q.codes), _ptr(q.scales), _mptr(q), 1.0, q.rows,
                              q.k, _ptr(out))
    return out


def alpha(a: Quantized, w: Quantized) -> float:
    if a.fmt == NVFP4:
        return float(np.float64(a.tensor_scale) * np.float64(w.tensor_scale))
    return 1.0


def _check_pair(a: Quantized, w: Quantized):
    if a.fmt != w.fmt or a.k != w.k:
        raise ValueError("operands differ in format or K")
    if (a.macro is None) != (w.macro is None):
        raise ValueError("operands differ in macro-block scaling")


def gemm_loop(a: Quantized, w: Quantized):
    """C = alpha * A' W'^T and L = alpha * |A'| |W'|^T, summed in k order (C loop)."""
    _check_pair(a, w)
    m, n = a.rows, w.rows
    c = np.empty((m, n), dtype=np.float64)
    l = np.empty((m, n), dtype=np.float64)
    _load().orc_gemm_ms(a.fmt, _ptr(a.codes), _ptr(a.scales), _mptr(a), float(a.tensor_scale),
                        _ptr(w.codes), _ptr(w.scales), _mptr(w), float(w.tensor_scale), m, n,
                        a.k, _ptr(c), _ptr(l))
    return c, l


def gemm(a: Quantized, w: Quantized):
    """Same contraction with a binary64 library matmul as the summation step."""
    _check_pair(a, w)
    ad, wd = _unit(a), _unit(w)
    al = alpha(a, w)
    return al * (ad @ wd.T), al * (np.abs(ad) @ np.abs(wd).T)


def gemm_sampled(a: Quantized, w: Quantized, rows, cols):
    """C and L at entries (rows[i], cols[i]), k-ordered binary64 sums."""
    _check_pair(a, w)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape:
        raise ValueError("rows and cols differ in length")
    if rows.size and (rows.min() < 0 or rows.max() >= a.rows or cols.min() < 0
                      or cols.max() >= w.rows):
        raise IndexError("sample index out of range")
    c = np.empty(rows.size, dtype=np.float64)
    l = np.empty(rows.size, dtype=np.float64)
    _load().orc_gemm_sampled_ms(a.fmt, _ptr(a.codes), _ptr(a.scales), _mptr(a),
                                float(a.tensor_scale), _ptr(w.codes), _ptr(w.scales), _mptr(w),
                                float(w.tensor_scale), a.k, _ptr(rows), _ptr(cols), rows.size,
                                _ptr(c), _ptr(l))
    return c, l


def gemm_w4a16(x, w: Quantized):
    if w.macro is not None:
        raise ValueError("the weight-only product takes no macro-block scales")
    return _gemm_w4a16(x, w)


def _gemm_w4a16(x, w: Quantized):
    """Weight-only product: C = S_tW * x W'^T with bf16 activations x [M, K]
    and the quantized weight (binary64, k-ordered); L = the magnitude sum."""
    x = _bf16(x)
    m, k = x.shape
    if k != w.k:
        raise ValueError("x and w differ in K")
    n = w.rows
    c = np.empty((m, n), dtype=np.float64)
    l = np.empty((m, n), dtype=np.float64)
    _load().orc_gemm_w4a16(w.fmt, _ptr(x), _ptr(w.codes), _ptr(w.scales), float(w.tensor_scale),
                           m, n, k, _ptr(c), _ptr(l))
    return c, l


def gemm_w4a16_sampled(x, w: Quantized, rows, cols):
    x = _bf16(x)
    m, k = x.shape
    if k != w.k:
        raise ValueError("x and w differ in K")
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape:
        raise ValueError("rows and cols differ in length")
    if rows.size and (rows.min() < 0 or rows.max() >= m or cols.min() < 0 or cols.max() >= w.rows):
        raise IndexError("sample index out of range")
    c = np.empty(rows.size, dtype=np.float64)
    l = np.empty(rows.size, dtype=np.float64)
    _load().orc_gemm_w4a16_sampled(w.fmt, _ptr(x), _ptr(w.codes), _ptr(w.scales),
                                   float(w.tensor_scale), k, _ptr(rows), _ptr(cols), rows.size,
                                   _ptr(c), _ptr(l))
    return c, l


def bf16_ulp(c: np.ndarray) -> np.ndarray:
    """One bf16 ulp of the binade of |c|: 2^(floor(log2|c|) - 7), floored at 2^-133."""
    c = np.abs(np.asarray(c, dtype=np.float64))
    _, e = np.frexp(c)
    ulp = np.ldexp(1.0, (e - 1) - 7)
    return np.where(c > 0, np.maximum(ulp, 2.0 ** -133), 2.0 ** -133)


def gemm_tolerance(c_ref, l_ref, rel: float = 1e-5):
    """Allowed |C_gpu - C_ref|: rel * L + one bf16 ulp of C_ref."""
    return rel * np.asarray(l_ref) + bf16_ulp(c_ref)
