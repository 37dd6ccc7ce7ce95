"""Python binding of libhr.so (ctypes): randomized Hadamard rotation, fused
int4 / int8 quantization, HARP-style butterfly, int4 dequant and the W4A4 /
W4A8 GEMMs on MI355X (gfx950).

Argument marshalling only: every step runs in the library's HIP kernels on
torch's current stream.  Tensors must be CUDA tensors, contiguous, of the
dtypes stated per function; outputs are allocated with torch when not given.
The library must be built in-tree first (``python
hadamard_rotation_int4_amd/build.py``); importing without it raises ImportError.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["HRError", "rotate", "rotate_quant_int4", "rotate_quant_int8", "butterfly_coeffs",
           "butterfly_apply", "harp_blocks", "harp_apply", "dequant_int4", "w4a4_gemm", "w4a8_gemm",
           "lib", "LIB_PATH", "SYMBOLS",
           "HR_OK", "HR_EINVAL", "HR_EUNSUPPORTED", "HR_EDEVICE", "HR_F32", "HR_BF16", "HR_F16"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhr.so")

HR_OK, HR_EINVAL, HR_EUNSUPPORTED, HR_EDEVICE = 0, 1, 2, 3
HR_F32, HR_BF16, HR_F16 = 0, 1, 2

_i32, _i64, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p

# name -> (restype, argtypes); mirrors include/hr.h
SYMBOLS = {
    "hr_abi_version": (_i32, []),
    "hr_status_string": (ctypes.c_char_p, [_i32]),
    "hr_last_error": (ctypes.c_char_p, []),
    "hr_rotate": (_i32, [_vp, _i32, _vp, _i64, _i32, _i32, _vp, _vp, _vp]),
    "hr_rotate_quant_int4": (_i32, [_vp, _i32, _i64, _i32, _i32, _vp, _vp, _i32, _vp, _vp, _i32, _vp]),
    "hr_rotate_quant_int8": (_i32, [_vp, _i32, _i64, _i32, _i32, _vp, _vp, _i32, _vp, _vp, _i32, _vp]),
    "hr_butterfly_coeffs": (_i32, [_vp, _i32, _i32, _vp, _vp]),
    "hr_butterfly_apply": (_i32, [_vp, _vp, _i64, _i32, _vp, _i32, _vp, _i32, _i32, _vp, _vp, _i32, _vp]),
    "hr_harp_blocks": (_i32, [_vp, _i32, _vp, _vp, _vp, _vp]),
    "hr_harp_apply": (_i32, [_vp, _vp, _i64, _vp, _i32, _vp, _i32, _i32, _vp, _vp, _i32, _vp]),
    "hr_dequant_int4": (_i32, [_vp, _vp, _i32, _i64, _i32, _i32, _vp, _vp]),
    "hr_w4a4_gemm": (_i32, [_vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _i32, _vp, _vp, _vp]),
    "hr_w4a8_gemm": (_i32, [_vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _i32, _vp, _vp, _vp]),
    "hr_w8a8_gemm": (_i32, [_vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _i32, _vp, _vp, _vp]),
}


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python hadamard_rotation_int4_amd/build.py`")
    handle = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SYMBOLS.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    return handle


lib = _load()


class HRError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        msg = lib.hr_last_error().decode(errors="replace")
        super().__init__(f"{fn}: {lib.hr_status_string(status).decode()}: {msg}")


def _check(status: int, fn: str) -> None:
    if status != HR_OK:
        raise HRError(status, fn)


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dtype_code(dt) -> int:
    if dt == torch.float32:
        return HR_F32
    if dt == torch.bfloat16:
        return HR_BF16
    if dt == torch.float16:
        return HR_F16
    raise TypeError(f"unsupported dtype {dt}")


def rotate(x: torch.Tensor, signs: torch.Tensor | None = None, block: torch.Tensor | None = None,
           out: torch.Tensor | None = None) -> torch.Tensor:
    """y = (O kron H_p)(d * x)/sqrt(p) per row (hr_rotate).  x: [rows][n] bf16/fp32;
    signs: int8 [n] or None; block: fp32 [m][m] or None (m = 1)."""
    rows, n = x.shape
    m = 1 if block is None else int(block.shape[0])
    y = out if out is not None else torch.empty((rows, n), dtype=torch.float32, device=x.device)
    _check(lib.hr_rotate(_ptr(x), _dtype_code(x.dtype), _ptr(y), rows, n, m, _ptr(signs),
                         _ptr(block), _stream(x.device)), "hr_rotate")
    return y


def rotate_quant_int4(x: torch.Tensor, group: int, signs: torch.Tensor | None = None,
                      block: torch.Tensor | None = None, scale_dtype=torch.float16,
                      codes: torch.Tensor | None = None, scales: torch.Tensor | None = None):
    """Fused rotation + per-group int4 quantization (hr_rotate_quant_int4).
    Returns (codes uint8 [rows][n/2], scales [rows][n/group] of scale_dtype)."""
    rows, n = x.shape
    m = 1 if block is None else int(block.shape[0])
    if codes is None:
        codes = torch.empty((rows, n // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, n // group), dtype=scale_dtype, device=x.device)
    _check(lib.hr_rotate_quant_int4(_ptr(x), _dtype_code(x.dtype), rows, n, m, _ptr(signs),
                                    _ptr(block), group, _ptr(codes), _ptr(scales),
                                    _dtype_code(scales.dtype), _stream(x.device)),
           "hr_rotate_quant_int4")
    return codes, scales


def rotate_quant_int8(x: torch.Tensor, group: int, signs: torch.Tensor | None = None,
                      block: torch.Tensor | None = None, scale_dtype=torch.float16,
                      codes: torch.Tensor | None = None, scales: torch.Tensor | None = None):
    """Fused rotation + per-group int8 quantization (hr_rotate_quant_int8).
    Returns (codes int8 [rows][n], scales [rows][n/group] of scale_dtype)."""
    rows, n = x.shape
    m = 1 if block is None else int(block.shape[0])
    if codes is None:
        codes = torch.empty((rows, n), dtype=torch.int8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, n // group), dtype=scale_dtype, device=x.device)
    _check(lib.hr_rotate_quant_int8(_ptr(x), _dtype_code(x.dtype), rows, n, m, _ptr(signs),
                                    _ptr(block), group, _ptr(codes), _ptr(scales),
                                    _dtype_code(scales.dtype), _stream(x.device)),
           "hr_rotate_quant_int8")
    return codes, scales


def butterfly_coeffs(angles: torch.Tensor, precondition: bool = False) -> torch.Tensor:
    """Per-pair coefficient table [log2 n][n/2][2] fp32 from angles [log2 n][n/2]."""
    L, half = angles.shape
    coeffs = torch.empty((L, half, 2), dtype=torch.float32, device=angles.device)
    _check(lib.hr_butterfly_coeffs(_ptr(angles), 2 * half, int(precondition), _ptr(coeffs),
                                   _stream(angles.device)), "hr_butterfly_coeffs")
    return coeffs


def butterfly_apply(x: torch.Tensor, coeffs: torch.Tensor, precondition: bool = False,
                    perm: torch.Tensor | None = None, inverse: bool = False,
                    want_y: bool = True, group: int | None = None, scale_dtype=torch.float16,
                    out: torch.Tensor | None = None):
    """Butterfly (or its transpose) per row, optionally quantized.
    Returns y, or (y_or_None, codes, scales) when ``group`` is given."""
    rows, n = x.shape
    y = None
    if want_y:
        y = out if out is not None else torch.empty((rows, n), dtype=torch.float32, device=x.device)
    codes = scales = None
    g = 0
    sd = HR_F16
    if group is not None:
        g = group
        codes = torch.empty((rows, n // 2), dtype=torch.uint8, device=x.device)
        scales = torch.empty((rows, n // group), dtype=scale_dtype, device=x.device)
        sd = _dtype_code(scale_dtype)
    _check(lib.hr_butterfly_apply(_ptr(x), _ptr(y), rows, n, _ptr(coeffs), int(precondition),
                                  _ptr(perm), int(inverse), g, _ptr(codes), _ptr(scales), sd,
                                  _stream(x.device)), "hr_butterfly_apply")
    if group is None:
        return y
    return y, codes, scales


def _radices(radices):
    r = (ctypes.c_int32 * len(radices))(*[int(b) for b in radices])
    return r, len(radices)


def harp_blocks(radices, theta: torch.Tensor, fallbacks: torch.Tensor | None = None) -> torch.Tensor:
    """Dense blocks of a HARP schedule (hr_harp_blocks).  radices: a Python
    sequence; theta: fp32 parameters; fallbacks: fp32 concatenated [b][b]
    mixers of the radices that are not powers of two (or None)."""
    arr, m = _radices(radices)
    d = 1
    for b in radices:
        d *= int(b)
    blocks = torch.empty(d * sum(int(b) for b in radices), dtype=torch.float32, device=theta.device)
    _check(lib.hr_harp_blocks(arr, m, _ptr(theta), _ptr(fallbacks), _ptr(blocks),
                              _stream(theta.device)), "hr_harp_blocks")
    return blocks


def harp_apply(x: torch.Tensor, radices, blocks: torch.Tensor, inverse: bool = False,
               want_y: bool = True, group: int | None = None, scale_dtype=torch.float16,
               out: torch.Tensor | None = None):
    """The HARP processor (or its transpose) per row (hr_harp_apply).
    Returns y, or (y_or_None, codes, scales) when ``group`` is given."""
    rows, d = x.shape
    arr, m = _radices(radices)
    y = None
    if want_y:
        y = out if out is not None else torch.empty((rows, d), dtype=torch.float32, device=x.device)
    codes = scales = None
    g, sd = 0, HR_F16
    if group is not None:
        g = group
        codes = torch.empty((rows, d // 2), dtype=torch.uint8, device=x.device)
        scales = torch.empty((rows, d // group), dtype=scale_dtype, device=x.device)
        sd = _dtype_code(scale_dtype)
    _check(lib.hr_harp_apply(_ptr(x), _ptr(y), rows, arr, m, _ptr(blocks), int(inverse), g,
                             _ptr(codes), _ptr(scales), sd, _stream(x.device)), "hr_harp_apply")
    if group is None:
        return y
    return y, codes, scales


def dequant_int4(codes: torch.Tensor, scales: torch.Tensor, group: int,
                 out: torch.Tensor | None = None) -> torch.Tensor:
    """x_hat = q * s (hr_dequant_int4).  codes uint8 [rows][n/2]."""
    rows, half = codes.shape
    n = 2 * half
    o = out if out is not None else torch.empty((rows, n), dtype=torch.float32, device=codes.device)
    _check(lib.hr_dequant_int4(_ptr(codes), _ptr(scales), _dtype_code(scales.dtype), rows, n, group,
                               _ptr(o), _stream(codes.device)), "hr_dequant_int4")
    return o


def w4a4_gemm(a_codes: torch.Tensor, a_scales: torch.Tensor, w_codes: torch.Tensor,
              w_scales: torch.Tensor, group: int, out: torch.Tensor | None = None,
              group_acc: bool = False):
    """C = A W^T with per-group scales (hr_w4a4_gemm).  Returns C, or (C, acc)
    with the exact per-group int32 sums [M][N][K/group] when group_acc."""
    M, half = a_codes.shape
    N = int(w_codes.shape[0])
    K = 2 * half
    if a_scales.dtype != w_scales.dtype:
        raise TypeError("a_scales and w_scales must share a dtype")
    c = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=a_codes.device)
    acc = None
    if group_acc:
        acc = torch.empty((M, N, K // group), dtype=torch.int32, device=a_codes.device)
    _check(lib.hr_w4a4_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(w_codes), _ptr(w_scales),
                            _dtype_code(a_scales.dtype), M, N, K, group, _ptr(c), _ptr(acc),
                            _stream(a_codes.device)), "hr_w4a4_gemm")
    return (c, acc) if group_acc else c


def w4a8_gemm(a_codes: torch.Tensor, a_scales: torch.Tensor, w_codes: torch.Tensor,
              w_scales: torch.Tensor, group: int, out: torch.Tensor | None = None,
              group_acc: bool = False):
    """C = A W^T with int8 activation codes a_codes [M][K] and packed int4
    weights (hr_w4a8_gemm).  Returns as w4a4_gemm."""
    if a_codes.dtype != torch.int8:
        raise TypeError("a_codes must be int8 [M][K]")
    M, K = a_codes.shape
    N = int(w_codes.shape[0])
    if a_scales.dtype != w_scales.dtype:
        raise TypeError("a_scales and w_scales must share a dtype")
    c = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=a_codes.device)
    acc = None
    if group_acc:
        acc = torch.empty((M, N, K // group), dtype=torch.int32, device=a_codes.device)
    _check(lib.hr_w4a8_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(w_codes), _ptr(w_scales),
                            _dtype_code(a_scales.dtype), M, N, K, group, _ptr(c), _ptr(acc),
                            _stream(a_codes.device)), "hr_w4a8_gemm")
    return (c, acc) if group_acc else c


def w8a8_gemm(a_codes: torch.Tensor, a_scales: torch.Tensor, w_codes: torch.Tensor,
              w_scales: torch.Tensor, group: int, out: torch.Tensor | None = None,
              group_acc: bool = False):
    """C = A W^T with both operands held one int8 code per element:
    a_codes [M][K], w_codes [N][K] (hr_w8a8_gemm).  Returns as w4a4_gemm."""
    if a_codes.dtype != torch.int8 or w_codes.dtype != torch.int8:
        raise TypeError("a_codes and w_codes must be int8 [M][K] and [N][K]")
    M, K = a_codes.shape
    N = int(w_codes.shape[0])
    if a_scales.dtype != w_scales.dtype:
        raise TypeError("a_scales and w_scales must share a dtype")
    c = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=a_codes.device)
    acc = None
    if group_acc:
        acc = torch.empty((M, N, K // group), dtype=torch.int32, device=a_codes.device)
    _check(lib.hr_w8a8_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(w_codes), _ptr(w_scales),
                            _dtype_code(a_scales.dtype), M, N, K, group, _ptr(c), _ptr(acc),
                            _stream(a_codes.device)), "hr_w8a8_gemm")
    return (c, acc) if group_acc else c
