"""Python binding of the gfx950 W4A4 block-scaled FP4 library (``libfp4amd.so``).

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
declared in ``include/fp4.h``; PyTorch supplies device memory and the current
stream. The functions carry the C names:

    fp4_quantize_weight(w, fmt)                 -> Fp4Tensor (weight cache layout)
    fp4_quantize_act(a, fmt, static_scale=None) -> Fp4Tensor (canonical layout)
    fp4_gemm(a_q, w_q)                          -> bf16 [M, N] = A^ W^T
    fp4_linear(x, w_q, static_scale=None)       -> bf16 [M, N]
    fp4_linear_w4a16(x, w_q)                    -> bf16 [M, N] (bf16 activations)
    fp4_export_canonical(w_q)                   -> Fp4Tensor (canonical copy)
    fp4_dequantize(t)                           -> fp32 [rows, K]

There is no CPU fallback: if the library is missing or the device is not
gfx950, the calls raise.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

NVFP4, MXFP4 = 0, 1
# recipe flags OR-ed into a format (include/fp4.h): block Hadamard rotation
# before quantization; MXFP4 overflow-aware block exponent
ROTATE, MX_OAS, MX_MBS = 0x100, 0x200, 0x400
CANONICAL, TILED = 0, 1
WEIGHT_TILED = TILED
FORMATS = {"nvfp4": NVFP4, "mxfp4": MXFP4}

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp4amd.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "fp4.h")


class fp4_tensor(ctypes.Structure):
    _fields_ = [
        ("fmt", ctypes.c_int32),
        ("layout", ctypes.c_int32),
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("codes_pitch", ctypes.c_int64),
        ("scales_pitch", ctypes.c_int64),
        ("codes", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("tensor_scale", ctypes.c_void_p),
    ]


_lib = None
_lock = threading.Lock()


def lib():
    """Load ``libfp4amd.so`` (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        T = ctypes.POINTER(fp4_tensor)
        sig = {
            "fp4_block_size": (I32, [I32]),
            "fp4_codes_bytes": (SZ, [I32, I32, I64, I64]),
            "fp4_scales_bytes": (SZ, [I32, I32, I64, I64]),
            "fp4_tensor_init": (I32, [T, I32, I32, I64, I64, P, P, P]),
            "fp4_quantize_workspace_bytes": (SZ, [I32, I64, I64]),
            "fp4_quantize_weight": (I32, [I32, P, I64, I64, T, P, SZ, P]),
            "fp4_quantize_act": (I32, [I32, P, I64, I64, P, T, P, SZ, P]),
            "fp4_gemm_workspace_bytes": (SZ, [I32, I64, I64, I64]),
            "fp4_gemm": (I32, [T, T, P, I64, P, SZ, P]),
            "fp4_linear_workspace_bytes": (SZ, [I32, I64, I64, I64]),
            "fp4_linear": (I32, [P, I64, T, P, P, P, SZ, P]),
            "fp4_linear_noalloc": (I32, [P, I64, T, P, P, P]),
            "fp4_linear_w4a16": (I32, [P, I64, T, P, I64, P]),
            "fp4_linear_launches": (I32, [I32, I64, I64, I64, I32]),
            "fp4_export_canonical": (I32, [T, T, P]),
            "fp4_dequantize": (I32, [T, P, I64, P]),
            "fp4_workspace_flags": (I32, [P, SZ, ctypes.POINTER(ctypes.c_uint32), I32, P]),
            "fp4_set_exchange_spin_limit": (ctypes.c_uint32, [ctypes.c_uint32]),
            "fp4_set_nvfp4_tile_mode": (I32, [I32]),
            "fp4_set_large_linear_fusion": (I32, [I32]),
            "fp4_set_decode_linear_fusion": (I32, [I32]),
            "fp4_set_mid_gemm": (I32, [I32]),
            "fp4_linear_mid_splits": (I32, [I32, I64, I64, I64]),
            "fp4_status_string": (ctypes.c_char_p, [I32]),
            "fp4_last_error": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
        return L


class Fp4Error(RuntimeError):
    pass


def _check(status: int):
    if status != 0:
        L = lib()
        raise Fp4Error("%s: %s" % (L.fp4_status_string(status).decode(),
                                   L.fp4_last_error().decode()))


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _fmt(fmt) -> int:
    """A format: NVFP4/MXFP4 (or "nvfp4"/"mxfp4", optionally with "+rotate"
    and "+oas" suffixes), possibly OR-ed with ROTATE / MX_OAS."""
    if isinstance(fmt, str):
        parts = fmt.lower().split("+")
        flags = {"rotate": ROTATE, "oas": MX_OAS, "mbs": MX_MBS}
        fmt = FORMATS[parts[0]]
        for p in parts[1:]:
            fmt |= flags[p]
    fmt = int(fmt)
    if fmt & 0xFF not in (NVFP4, MXFP4) or fmt & ~(0xFF | ROTATE | MX_OAS | MX_MBS):
        raise ValueError("format must be NVFP4 (0) or MXFP4 (1), optionally | ROTATE | MX_OAS | MX_MBS")
    return fmt


def _bf16_2d(x: torch.Tensor, name: str) -> torch.Tensor:
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_cuda:
        raise ValueError(f"{name} must be a 2-D bfloat16 CUDA tensor")
    return x.contiguous()


class Fp4Tensor:
    """Quantized tensor: device buffers owned by torch plus the C descriptor."""

    def __init__(self, fmt: int, layout: int, rows: int, k: int, device):
        L = lib()
        self.fmt, self.layout, self.rows, self.k = fmt, layout, rows, k
        nc = L.fp4_codes_bytes(fmt, layout, rows, k)
        ns = L.fp4_scales_bytes(fmt, layout, rows, k)
        if nc == 0 or ns == 0:
            raise ValueError("invalid FP4 tensor shape")
        self.codes = torch.empty(nc, dtype=torch.uint8, device=device)
        self.scales = torch.empty(ns, dtype=torch.uint8, device=device)
        self.tensor_scale = torch.empty(1, dtype=torch.float32, device=device)
        self.desc = fp4_tensor()
        _check(L.fp4_tensor_init(ctypes.byref(self.desc), fmt, layout, rows, k,
                                 _ptr(self.codes), _ptr(self.scales), _ptr(self.tensor_scale)))

    @property
    def device(self):
        return self.codes.device

    def codes_2d(self) -> torch.Tensor:
        """Canonical codes as [rows, codes_pitch] bytes."""
        assert self.layout == CANONICAL
        return self.codes.view(self.rows, self.desc.codes_pitch)

    def scales_2d(self) -> torch.Tensor:
        assert self.layout == CANONICAL
        return self.scales[: self.rows * self.desc.scales_pitch].view(self.rows, self.desc.scales_pitch)

    def macro_2d(self) -> torch.Tensor:
        """Canonical macro-block scales (MX_MBS) as float32 [rows, K_pad/128]."""
        assert self.layout == CANONICAL and self.fmt & MX_MBS
        off = -(-self.rows * self.desc.scales_pitch // 16) * 16
        mp = -(-self.k // 128)
        return self.scales[off: off + self.rows * mp * 4].view(torch.float32).view(self.rows, mp)


def fp4_quantize_weight(w: torch.Tensor, fmt=NVFP4) -> Fp4Tensor:
    fmt = _fmt(fmt)
    w = _bf16_2d(w, "w")
    n, k = w.shape
    L = lib()
    out = Fp4Tensor(fmt, TILED, n, k, w.device)
    nws = L.fp4_quantize_workspace_bytes(fmt, n, k)
    ws = torch.zeros(max(nws, 1), dtype=torch.uint8, device=w.device)
    _check(L.fp4_quantize_weight(fmt, _ptr(w), n, k, ctypes.byref(out.desc), _ptr(ws), nws,
                                 _stream(w.device)))
    return out


def fp4_quantize_act(a: torch.Tensor, fmt=NVFP4, static_scale: torch.Tensor | None = None,
                     layout: int = CANONICAL, workspace: torch.Tensor | None = None,
                     out: Fp4Tensor | None = None) -> Fp4Tensor:
    """Quantize activations into a new tensor, or into `out` (same format,
    layout and shape)."""
    fmt = _fmt(fmt)
    a = _bf16_2d(a, "a")
    m, k = a.shape
    L = lib()
    if out is None:
        out = Fp4Tensor(fmt, layout, m, k, a.device)
    nws = L.fp4_quantize_workspace_bytes(fmt, m, k)
    ws = workspace
    if ws is None:   # zero-filled once, as the C ABI requires
        ws = torch.zeros(max(nws, 1), dtype=torch.uint8, device=a.device)
    _check(L.fp4_quantize_act(fmt, _ptr(a), m, k, _ptr(static_scale), ctypes.byref(out.desc),
                              _ptr(ws), ws.numel(), _stream(a.device)))
    return out


def fp4_gemm(a: Fp4Tensor, w: Fp4Tensor, out: torch.Tensor | None = None,
             workspace: torch.Tensor | None = None) -> torch.Tensor:
    L = lib()
    m, n = a.rows, w.rows
    if out is None:
        out = torch.empty(m, n, dtype=torch.bfloat16, device=a.device)
    nws = L.fp4_gemm_workspace_bytes(a.fmt, m, n, a.k)
    if workspace is None and nws > 0:
        # room for the tiled copy of large canonical activations, or for the
        # mid-size GEMM's partial sums (tiled activations, 33-128 rows)
        workspace = torch.empty(nws, dtype=torch.uint8, device=a.device)
    _check(L.fp4_gemm(ctypes.byref(a.desc), ctypes.byref(w.desc), _ptr(out), out.stride(0),
                      _ptr(workspace), 0 if workspace is None else workspace.numel(),
                      _stream(a.device)))
    return out


def fp4_linear_workspace_bytes(fmt, m: int, n: int, k: int) -> int:
    return lib().fp4_linear_workspace_bytes(_fmt(fmt), m, n, k)


def fp4_linear_launches(fmt, m: int, n: int, k: int, static_scale: bool = False) -> int:
    return lib().fp4_linear_launches(_fmt(fmt), m, n, k, int(bool(static_scale)))


def fp4_linear(x: torch.Tensor, w: Fp4Tensor, static_scale: torch.Tensor | None = None,
               out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    x = _bf16_2d(x, "x")
    m = x.shape[0]
    if x.shape[1] != w.k:
        raise ValueError("x has K=%d, weight has K=%d" % (x.shape[1], w.k))
    L = lib()
    if out is None:
        out = torch.empty(m, w.rows, dtype=torch.bfloat16, device=x.device)
    nws = L.fp4_linear_workspace_bytes(w.fmt, m, w.rows, w.k)
    if workspace is None:   # zero-filled once, as the C ABI requires
        workspace = torch.zeros(max(nws, 1), dtype=torch.uint8, device=x.device)
    _check(L.fp4_linear(_ptr(x), m, ctypes.byref(w.desc), _ptr(static_scale), _ptr(out),
                        _ptr(workspace), workspace.numel(), _stream(x.device)))
    return out


NOALLOC_SCRATCH_BYTES = 16 << 20


def fp4_linear_noalloc(x: torch.Tensor, w: Fp4Tensor, static_scale: torch.Tensor | None = None,
                       out: torch.Tensor | None = None) -> torch.Tensor:
    """fp4_linear whose workspace is the library's own device array (the C call
    allocates nothing; pass `out` to allocate nothing here either)."""
    x = _bf16_2d(x, "x")
    m = x.shape[0]
    if x.shape[1] != w.k:
        raise ValueError("x has K=%d, weight has K=%d" % (x.shape[1], w.k))
    if out is None:
        out = torch.empty(m, w.rows, dtype=torch.bfloat16, device=x.device)
    _check(lib().fp4_linear_noalloc(_ptr(x), m, ctypes.byref(w.desc), _ptr(static_scale), _ptr(out),
                                    _stream(x.device)))
    return out


def fp4_linear_w4a16(x: torch.Tensor, w: Fp4Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Weight-only linear: bf16 activations times the FP4 weight cache."""
    x = _bf16_2d(x, "x")
    m = x.shape[0]
    if x.shape[1] != w.k:
        raise ValueError("x has K=%d, weight has K=%d" % (x.shape[1], w.k))
    if out is None:
        out = torch.empty(m, w.rows, dtype=torch.bfloat16, device=x.device)
    _check(lib().fp4_linear_w4a16(_ptr(x), m, ctypes.byref(w.desc), _ptr(out), out.stride(0),
                                  _stream(x.device)))
    return out


WS_EXCHANGE_TIMEOUT = 1


def fp4_workspace_flags(workspace: torch.Tensor, clear: bool = False) -> int:
    """Sticky error flags recorded in a quantize or linear workspace (waits for
    the current stream); clear=True clears them."""
    flags = ctypes.c_uint32(0)
    _check(lib().fp4_workspace_flags(_ptr(workspace), workspace.numel(), ctypes.byref(flags),
                                     int(bool(clear)), _stream(workspace.device)))
    return flags.value


def fp4_set_exchange_spin_limit(polls: int) -> int:
    """Test aid: polls before a workgroup of the quantizer's maximum exchange
    gives up (0: at once). Returns the previous value."""
    return lib().fp4_set_exchange_spin_limit(int(polls))


def fp4_set_large_linear_fusion(on: bool) -> bool:
    """Whether fp4_linear quantizes large-M activations inside the GEMM launch
    (static NVFP4 scale or MXFP4; off by default). Process-wide; returns the
    previous setting."""
    return bool(lib().fp4_set_large_linear_fusion(int(bool(on))))


def fp4_set_decode_linear_fusion(on: bool) -> bool:
    """Whether fp4_linear with at most 32 activation rows quantizes them inside
    the skinny GEMM's launch (off by default). Process-wide; returns the
    previous setting."""
    return bool(lib().fp4_set_decode_linear_fusion(int(bool(on))))


def fp4_set_mid_gemm(on: bool) -> bool:
    """Whether the GEMM of 33-128 activation rows runs on the mid-size kernel
    (four weight tiles per workgroup, K split with an ordered FP32 combine; on
    by default) or on the skinny kernel. Process-wide; returns the previous
    setting."""
    return bool(lib().fp4_set_mid_gemm(int(bool(on))))


def fp4_linear_mid_splits(fmt, m: int, n: int, k: int) -> int:
    """K slices of fp4_linear's mid-size GEMM for this shape (0: another kernel)."""
    return lib().fp4_linear_mid_splits(_fmt(fmt), m, n, k)


NV_TILE_REGISTERS, NV_TILE_LDS = 0, 1


def fp4_set_nvfp4_tile_mode(mode: int) -> int:
    """Where the NVFP4 256 x 256 tile GEMM converts codes to f16: NV_TILE_REGISTERS
    (each wave that uses a fragment) or NV_TILE_LDS (once per workgroup, into
    LDS). Process-wide; returns the previous mode."""
    prev = lib().fp4_set_nvfp4_tile_mode(int(mode))
    if prev < 0:
        raise ValueError("mode must be NV_TILE_REGISTERS or NV_TILE_LDS")
    return prev


def fp4_export_canonical(t: Fp4Tensor) -> Fp4Tensor:
    out = Fp4Tensor(t.fmt, CANONICAL, t.rows, t.k, t.device)
    _check(lib().fp4_export_canonical(ctypes.byref(t.desc), ctypes.byref(out.desc),
                                      _stream(t.device)))
    return out


def fp4_dequantize(t: Fp4Tensor) -> torch.Tensor:
    out = torch.empty(t.rows, t.k, dtype=torch.float32, device=t.device)
    _check(lib().fp4_dequantize(ctypes.byref(t.desc), _ptr(out), t.k, _stream(t.device)))
    return out
