"""Python binding of libhr.so (ctypes): randomized Hadamard rotation, fused
int4 / int8 quantization, HARP-style butterfly and mixed-radix processor, int4
dequant, the W4A4 / W4A8 / W8A8 GEMMs and the online-rotation decode GEMM on
MI355X (gfx950).

Argument marshalling only: every step runs in the library's HIP kernels on
torch's current stream.  Every tensor argument is checked (dtype, shape,
contiguity, then device) against the sizes passed to the C call before the
call is made, and outputs are allocated with torch when not given.  The
library must be built in-tree first (``python
hadamard_rotation_int4_amd/build.py``); importing without it, or with a
library built from other sources, raises ImportError.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import srchash

__all__ = ["HRError", "rotate", "rotate_quant_int4", "rotate_quant_int8", "quant_int4", "quant_int8",
           "butterfly_coeffs", "butterfly_apply", "harp_blocks", "harp_apply", "harp_n_params", "harp_table_size",
           "dequant_int4", "w4a4_gemm", "w4a8_gemm", "w8a8_gemm", "rotate_quant_w4a4_gemm",
           "fp6_rows", "w4a4_to_fp6", "rotate_quant_fp6", "w4a4_gemm_fp6",
           "lib", "LIB_PATH", "SYMBOLS",
           "HR_OK", "HR_EINVAL", "HR_EUNSUPPORTED", "HR_EDEVICE", "HR_F32", "HR_BF16", "HR_F16"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhr.so")

HR_OK, HR_EINVAL, HR_EUNSUPPORTED, HR_EDEVICE = 0, 1, 2, 3
HR_F32, HR_BF16, HR_F16 = 0, 1, 2

_i32, _i64, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p

# name -> (restype, argtypes); mirrors include/hr.h
SYMBOLS = {
    "hr_abi_version": (_i32, []),
    "hr_build_id": (ctypes.c_char_p, []),
    "hr_status_string": (ctypes.c_char_p, [_i32]),
    "hr_last_error": (ctypes.c_char_p, []),
    "hr_rotate": (_i32, [_vp, _i32, _vp, _i64, _i32, _i32, _vp, _vp, _vp]),
    "hr_rotate_quant_int4": (_i32, [_vp, _i32, _i64, _i32, _i32, _vp, _vp, _i32, _vp, _vp, _i32, _vp]),
    "hr_rotate_quant_int8": (_i32, [_vp, _i32, _i64, _i32, _i32, _vp, _vp, _i32, _vp, _vp, _i32, _vp]),
    "hr_quant_int4": (_i32, [_vp, _i32, _i64, _i32, _i32, _vp, _vp, _i32, _vp]),
    "hr_quant_int8": (_i32, [_vp, _i32, _i64, _i32, _i32, _vp, _vp, _i32, _vp]),
    "hr_butterfly_coeffs": (_i32, [_vp, _i32, _i32, _vp, _vp]),
    "hr_butterfly_apply": (_i32, [_vp, _vp, _i64, _i32, _vp, _i32, _vp, _i32, _i32, _vp, _vp, _i32, _vp]),
    "hr_harp_blocks": (_i32, [_vp, _i32, _vp, _vp, _vp, _vp]),
    "hr_harp_apply": (_i32, [_vp, _vp, _i64, _vp, _i32, _vp, _i32, _i32, _vp, _vp, _i32, _vp]),
    "hr_dequant_int4": (_i32, [_vp, _vp, _i32, _i64, _i32, _i32, _vp, _vp]),
    "hr_w4a4_gemm": (_i32, [_vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _i32, _vp, _vp, _vp]),
    "hr_w4a8_gemm": (_i32, [_vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _i32, _vp, _vp, _vp]),
    "hr_w8a8_gemm": (_i32, [_vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _i32, _vp, _vp, _vp]),
    "hr_rotate_quant_w4a4_gemm": (_i32, [_vp, _i32, _vp, _i32, _vp, _vp, _i32, _i64, _i64, _i64, _vp,
                                         _vp, _vp, _vp]),
    "hr_w4a4_to_fp6": (_i32, [_vp, _vp, _i32, _i64, _i64, _i32, _vp, _vp, _vp]),
    "hr_rotate_quant_fp6": (_i32, [_vp, _i32, _vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp]),
    "hr_w4a4_gemm_fp6": (_i32, [_vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _i32, _vp, _vp, _vp]),
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
    built = handle.hr_build_id().decode()
    want = srchash.source_hash()
    if built != want:
        raise ImportError(f"{LIB_PATH} was built from other sources (build id {built}, sources "
                          f"{want}): rebuild it with `python hadamard_rotation_int4_amd/build.py`")
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


_DT_NAME = {torch.float32: "float32", torch.bfloat16: "bfloat16", torch.float16: "float16",
            torch.int8: "int8", torch.uint8: "uint8", torch.int32: "int32"}


def _arg(t, name: str, dtypes, shape):
    """Check tensor ``t``: dtype in ``dtypes``, exact ``shape``, contiguous.
    Returns (name, t); None passes through.  Devices are checked afterwards
    by _ptrs, so every dtype and shape error is reported first."""
    if t is None:
        return (name, None)
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if not isinstance(dtypes, (tuple, list)):
        dtypes = (dtypes,)
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in "
                        f"{[_DT_NAME.get(d, str(d)) for d in dtypes]}")
    shape = tuple(int(v) for v in shape)
    if tuple(t.shape) != shape:
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {shape}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: tensor must be contiguous")
    return (name, t)


def _ptrs(*args):
    """Device pointers of checked tensors (None -> NULL): each must be a GPU
    tensor, all on the device of the first one."""
    dev = None
    out = []
    for name, t in args:
        if t is None:
            out.append(None)
            continue
        if not t.is_cuda:
            raise ValueError(f"{name}: tensor must live on the GPU")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name}: on {t.device}, expected {dev}")
        out.append(t.data_ptr())
    return out


def _rows_of(x, name: str, dtypes):
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(x).__name__}")
    if x.dim() != 2:
        raise ValueError(f"{name}: expected a 2-D [rows][n] tensor, got shape {tuple(x.shape)}")
    if x.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {x.dtype} not in {[_DT_NAME[d] for d in dtypes]}")
    return int(x.shape[0]), int(x.shape[1])


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


def _scale_dtype(dt):
    if dt not in (torch.float16, torch.float32):
        raise TypeError(f"scale_dtype must be torch.float16 or torch.float32, got {dt}")
    return dt


def _group(group, n: int) -> int:
    g = int(group)
    if g <= 0 or n % g:
        raise ValueError(f"group={g} must be a positive divisor of the row length {n}")
    return g


def _block_m(block, n: int) -> int:
    if block is None:
        return 1
    if not isinstance(block, torch.Tensor) or block.dim() != 2 or block.shape[0] != block.shape[1]:
        raise ValueError("block must be a square [m][m] tensor")
    m = int(block.shape[0])
    if m < 1 or n % m:
        raise ValueError(f"block size m={m} must divide the row length {n}")
    return m


# ------------------------------------------------------------------ rotation

def rotate(x: torch.Tensor, signs: torch.Tensor | None = None, block: torch.Tensor | None = None,
           out: torch.Tensor | None = None) -> torch.Tensor:
    """y = (O kron H_p)(d * x)/sqrt(p) per row (hr_rotate).  x: [rows][n] bf16/fp32;
    signs: int8 [n] or None; block: fp32 [m][m] or None (m = 1)."""
    rows, n = _rows_of(x, "x", (torch.bfloat16, torch.float32))
    m = _block_m(block, n)
    ax = _arg(x, "x", (torch.bfloat16, torch.float32), (rows, n))
    asg = _arg(signs, "signs", torch.int8, (n,))
    ab = _arg(block, "block", torch.float32, (m, m))
    _arg(out, "out", torch.float32, (rows, n))
    y = out if out is not None else torch.empty((rows, n), dtype=torch.float32, device=x.device)
    px, ps, pb, py = _ptrs(ax, asg, ab, ("out", y))
    _check(lib.hr_rotate(px, _dtype_code(x.dtype), py, rows, n, m, ps, pb, _stream(x.device)), "hr_rotate")
    return y


def _rotate_quant(fn, bits, x, group, signs, block, scale_dtype, codes, scales):
    rows, n = _rows_of(x, "x", (torch.bfloat16, torch.float32))
    m = _block_m(block, n)
    g = _group(group, n)
    sd = _scale_dtype(scales.dtype if isinstance(scales, torch.Tensor) else scale_dtype)
    cdt, cshape = (torch.uint8, (rows, n // 2)) if bits == 4 else (torch.int8, (rows, n))
    ax = _arg(x, "x", (torch.bfloat16, torch.float32), (rows, n))
    asg = _arg(signs, "signs", torch.int8, (n,))
    ab = _arg(block, "block", torch.float32, (m, m))
    _arg(codes, "codes", cdt, cshape)
    _arg(scales, "scales", sd, (rows, n // g))
    dev = x.device
    if codes is None:
        codes = torch.empty(cshape, dtype=cdt, device=dev)
    if scales is None:
        scales = torch.empty((rows, n // g), dtype=sd, device=dev)
    px, ps, pb, pc, pq = _ptrs(ax, asg, ab, ("codes", codes), ("scales", scales))
    _check(getattr(lib, fn)(px, _dtype_code(x.dtype), rows, n, m, ps, pb, g, pc, pq, _dtype_code(sd),
                            _stream(dev)), fn)
    return codes, scales


def rotate_quant_int4(x: torch.Tensor, group: int, signs: torch.Tensor | None = None,
                      block: torch.Tensor | None = None, scale_dtype=torch.float16,
                      codes: torch.Tensor | None = None, scales: torch.Tensor | None = None):
    """Fused rotation + per-group int4 quantization (hr_rotate_quant_int4).
    Returns (codes uint8 [rows][n/2], scales [rows][n/group] of scale_dtype)."""
    return _rotate_quant("hr_rotate_quant_int4", 4, x, group, signs, block, scale_dtype, codes, scales)


def rotate_quant_int8(x: torch.Tensor, group: int, signs: torch.Tensor | None = None,
                      block: torch.Tensor | None = None, scale_dtype=torch.float16,
                      codes: torch.Tensor | None = None, scales: torch.Tensor | None = None):
    """Fused rotation + per-group int8 quantization (hr_rotate_quant_int8).
    Returns (codes int8 [rows][n], scales [rows][n/group] of scale_dtype)."""
    return _rotate_quant("hr_rotate_quant_int8", 8, x, group, signs, block, scale_dtype, codes, scales)


def _quant(fn, bits, x, group, scale_dtype, codes, scales):
    rows, n = _rows_of(x, "x", (torch.bfloat16, torch.float32))
    g = _group(group, n)
    sd = _scale_dtype(scales.dtype if isinstance(scales, torch.Tensor) else scale_dtype)
    cdt, cshape = (torch.uint8, (rows, n // 2)) if bits == 4 else (torch.int8, (rows, n))
    ax = _arg(x, "x", (torch.bfloat16, torch.float32), (rows, n))
    _arg(codes, "codes", cdt, cshape)
    _arg(scales, "scales", sd, (rows, n // g))
    dev = x.device
    if codes is None:
        codes = torch.empty(cshape, dtype=cdt, device=dev)
    if scales is None:
        scales = torch.empty((rows, n // g), dtype=sd, device=dev)
    px, pc, pq = _ptrs(ax, ("codes", codes), ("scales", scales))
    _check(getattr(lib, fn)(px, _dtype_code(x.dtype), rows, n, g, pc, pq, _dtype_code(sd), _stream(dev)),
           fn)
    return codes, scales


def quant_int4(x: torch.Tensor, group: int, scale_dtype=torch.float16,
               codes: torch.Tensor | None = None, scales: torch.Tensor | None = None):
    """Per-group int4 quantization without a rotation (hr_quant_int4).
    Returns (codes uint8 [rows][n/2], scales [rows][n/group])."""
    return _quant("hr_quant_int4", 4, x, group, scale_dtype, codes, scales)


def quant_int8(x: torch.Tensor, group: int, scale_dtype=torch.float16,
               codes: torch.Tensor | None = None, scales: torch.Tensor | None = None):
    """Per-group int8 quantization without a rotation (hr_quant_int8).
    Returns (codes int8 [rows][n], scales [rows][n/group])."""
    return _quant("hr_quant_int8", 8, x, group, scale_dtype, codes, scales)


# ------------------------------------------------------------------ butterfly

def _log2_exact(n: int, what: str) -> int:
    if n <= 0 or n & (n - 1):
        raise ValueError(f"{what}={n} is not a power of two")
    return n.bit_length() - 1


def butterfly_coeffs(angles: torch.Tensor, precondition: bool = False) -> torch.Tensor:
    """Per-pair coefficient table [log2 n][n/2][2] fp32 from angles [log2 n][n/2]."""
    if not isinstance(angles, torch.Tensor) or angles.dim() != 2:
        raise ValueError("angles must be a 2-D [log2 n][n/2] tensor")
    L, half = (int(v) for v in angles.shape)
    n = 2 * half
    if _log2_exact(n, "n") != L:
        raise ValueError(f"angles has {L} stages, expected log2(n) = {_log2_exact(n, 'n')} for n = {n}")
    aa = _arg(angles, "angles", torch.float32, (L, half))
    coeffs = torch.empty((L, half, 2), dtype=torch.float32, device=angles.device)
    pa, pc = _ptrs(aa, ("coeffs", coeffs))
    _check(lib.hr_butterfly_coeffs(pa, n, int(precondition), pc, _stream(angles.device)),
           "hr_butterfly_coeffs")
    return coeffs


def butterfly_apply(x: torch.Tensor, coeffs: torch.Tensor, precondition: bool = False,
                    perm: torch.Tensor | None = None, inverse: bool = False,
                    want_y: bool = True, group: int | None = None, scale_dtype=torch.float16,
                    out: torch.Tensor | None = None):
    """Butterfly (or its transpose) per row, optionally quantized.
    Returns y, or (y_or_None, codes, scales) when ``group`` is given."""
    rows, n = _rows_of(x, "x", (torch.float32,))
    L = _log2_exact(n, "n")
    ax = _arg(x, "x", torch.float32, (rows, n))
    aco = _arg(coeffs, "coeffs", torch.float32, (L, n // 2, 2))
    ap = _arg(perm, "perm", torch.int32, (n,))
    _arg(out, "out", torch.float32, (rows, n))
    g, sd, sdt = 0, HR_F16, None
    if group is not None:
        g = _group(group, n)
        sdt = _scale_dtype(scale_dtype)
        sd = _dtype_code(sdt)
    dev = x.device
    y = None
    if want_y:
        y = out if out is not None else torch.empty((rows, n), dtype=torch.float32, device=dev)
    codes = scales = None
    if group is not None:
        codes = torch.empty((rows, n // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((rows, n // g), dtype=sdt, device=dev)
    px, pco, pp, py, pc, pq = _ptrs(ax, aco, ap, ("out", y), ("codes", codes), ("scales", scales))
    _check(lib.hr_butterfly_apply(px, py, rows, n, pco, int(precondition), pp, int(inverse), g, pc, pq, sd,
                                  _stream(dev)), "hr_butterfly_apply")
    if group is None:
        return y
    return y, codes, scales


# ------------------------------------------------------------------ HARP

def harp_n_params(b: int) -> int:
    """Parameters per block of radix b: one angle for b = 2, else b(b-1)/2."""
    return 1 if b == 2 else b * (b - 1) // 2


def _radices(radices):
    rs = [int(b) for b in radices]
    if not rs:
        raise ValueError("radices must not be empty")
    r = (ctypes.c_int32 * len(rs))(*rs)
    d = 1
    for b in rs:
        d *= b
    return r, len(rs), rs, d


def harp_table_size(radices) -> int:
    """Floats in the block table of a schedule: per stage ceil(b^2 / 4) quads
    of d / b blocks."""
    rs = [int(b) for b in radices]
    d = 1
    for b in rs:
        d *= b
    return sum(4 * ((b * b + 3) // 4) * (d // b) for b in rs)


def harp_blocks(radices, theta: torch.Tensor, fallbacks: torch.Tensor | None = None) -> torch.Tensor:
    """Dense blocks of a HARP schedule (hr_harp_blocks).  radices: a Python
    sequence; theta: fp32 parameters [sum_t (d/b_t) P_t]; fallbacks: fp32
    concatenated [b][b] mixers of the radices that are not powers of two (or
    None)."""
    arr, m, rs, d = _radices(radices)
    n_theta = sum((d // b) * harp_n_params(b) for b in rs)
    n_fb = sum(b * b for b in rs if b & (b - 1))
    at = _arg(theta, "theta", torch.float32, (n_theta,))
    af = _arg(fallbacks, "fallbacks", torch.float32, (n_fb,))
    blocks = torch.empty(harp_table_size(rs), dtype=torch.float32, device=theta.device)
    pt, pf, pb = _ptrs(at, af, ("blocks", blocks))
    _check(lib.hr_harp_blocks(arr, m, pt, pf, pb, _stream(theta.device)), "hr_harp_blocks")
    return blocks


def harp_apply(x: torch.Tensor, radices, blocks: torch.Tensor, inverse: bool = False,
               want_y: bool = True, group: int | None = None, scale_dtype=torch.float16,
               out: torch.Tensor | None = None):
    """The HARP processor (or its transpose) per row (hr_harp_apply).
    Returns y, or (y_or_None, codes, scales) when ``group`` is given."""
    rows, d = _rows_of(x, "x", (torch.float32,))
    arr, m, rs, dd = _radices(radices)
    if dd != d:
        raise ValueError(f"the radices multiply to {dd}, but rows have {d} elements")
    ax = _arg(x, "x", torch.float32, (rows, d))
    ab = _arg(blocks, "blocks", torch.float32, (harp_table_size(rs),))
    _arg(out, "out", torch.float32, (rows, d))
    g, sd, sdt = 0, HR_F16, None
    if group is not None:
        g = _group(group, d)
        sdt = _scale_dtype(scale_dtype)
        sd = _dtype_code(sdt)
    dev = x.device
    y = None
    if want_y:
        y = out if out is not None else torch.empty((rows, d), dtype=torch.float32, device=dev)
    codes = scales = None
    if group is not None:
        codes = torch.empty((rows, d // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((rows, d // g), dtype=sdt, device=dev)
    px, pb, py, pc, pq = _ptrs(ax, ab, ("out", y), ("codes", codes), ("scales", scales))
    _check(lib.hr_harp_apply(px, py, rows, arr, m, pb, int(inverse), g, pc, pq, sd, _stream(dev)),
           "hr_harp_apply")
    if group is None:
        return y
    return y, codes, scales


# ------------------------------------------------------------------ dequant

def dequant_int4(codes: torch.Tensor, scales: torch.Tensor, group: int,
                 out: torch.Tensor | None = None) -> torch.Tensor:
    """x_hat = q * s (hr_dequant_int4).  codes uint8 [rows][n/2]; scales
    fp16/fp32 [rows][n/group]."""
    rows, half = _rows_of(codes, "codes", (torch.uint8,))
    n = 2 * half
    g = _group(group, n)
    ac = _arg(codes, "codes", torch.uint8, (rows, half))
    asc = _arg(scales, "scales", (torch.float16, torch.float32), (rows, n // g))
    _arg(out, "out", torch.float32, (rows, n))
    o = out if out is not None else torch.empty((rows, n), dtype=torch.float32, device=codes.device)
    pc, ps, po = _ptrs(ac, asc, ("out", o))
    _check(lib.hr_dequant_int4(pc, ps, _dtype_code(scales.dtype), rows, n, g, po, _stream(codes.device)),
           "hr_dequant_int4")
    return o


# ------------------------------------------------------------------ GEMMs

def _gemm(fn, a_int8, w_int8, a_codes, a_scales, w_codes, w_scales, group, out, group_acc):
    a_dt = torch.int8 if a_int8 else torch.uint8
    w_dt = torch.int8 if w_int8 else torch.uint8
    M, ka = _rows_of(a_codes, "a_codes", (a_dt,))
    N, kw = _rows_of(w_codes, "w_codes", (w_dt,))
    K = ka if a_int8 else 2 * ka
    if (kw if w_int8 else 2 * kw) != K:
        raise ValueError(f"w_codes {tuple(w_codes.shape)} does not match K = {K} of a_codes "
                         f"{tuple(a_codes.shape)}")
    g = _group(group, K)
    if not isinstance(a_scales, torch.Tensor) or not isinstance(w_scales, torch.Tensor):
        raise TypeError("a_scales and w_scales must be tensors")
    if a_scales.dtype != w_scales.dtype:
        raise TypeError("a_scales and w_scales must share a dtype")
    sd = _scale_dtype(a_scales.dtype)
    aa = _arg(a_codes, "a_codes", a_dt, (M, ka))
    asa = _arg(a_scales, "a_scales", sd, (M, K // g))
    aw = _arg(w_codes, "w_codes", w_dt, (N, kw))
    asw = _arg(w_scales, "w_scales", sd, (N, K // g))
    _arg(out, "out", torch.float32, (M, N))
    dev = a_codes.device
    c = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=dev)
    acc = torch.empty((M, N, K // g), dtype=torch.int32, device=dev) if group_acc else None
    pa, psa, pw, psw, pc, pacc = _ptrs(aa, asa, aw, asw, ("out", c), ("group_acc", acc))
    _check(getattr(lib, fn)(pa, psa, pw, psw, _dtype_code(sd), M, N, K, g, pc, pacc, _stream(dev)), fn)
    return (c, acc) if group_acc else c


def w4a4_gemm(a_codes: torch.Tensor, a_scales: torch.Tensor, w_codes: torch.Tensor,
              w_scales: torch.Tensor, group: int, out: torch.Tensor | None = None,
              group_acc: bool = False):
    """C = A W^T with per-group scales (hr_w4a4_gemm): a_codes uint8 [M][K/2],
    w_codes uint8 [N][K/2], scales [M][K/G], [N][K/G] (fp16 or fp32, same
    dtype).  Returns C, or (C, acc) with the exact per-group int32 sums
    [M][N][K/group] when group_acc."""
    return _gemm("hr_w4a4_gemm", False, False, a_codes, a_scales, w_codes, w_scales, group, out,
                 group_acc)


def w4a8_gemm(a_codes: torch.Tensor, a_scales: torch.Tensor, w_codes: torch.Tensor,
              w_scales: torch.Tensor, group: int, out: torch.Tensor | None = None,
              group_acc: bool = False):
    """C = A W^T with int8 activation codes a_codes [M][K] and packed int4
    weights w_codes uint8 [N][K/2] (hr_w4a8_gemm).  Returns as w4a4_gemm."""
    return _gemm("hr_w4a8_gemm", True, False, a_codes, a_scales, w_codes, w_scales, group, out,
                 group_acc)


def w8a8_gemm(a_codes: torch.Tensor, a_scales: torch.Tensor, w_codes: torch.Tensor,
              w_scales: torch.Tensor, group: int, out: torch.Tensor | None = None,
              group_acc: bool = False):
    """C = A W^T with both operands held one int8 code per element:
    a_codes [M][K], w_codes [N][K] (hr_w8a8_gemm).  Returns as w4a4_gemm."""
    return _gemm("hr_w8a8_gemm", True, True, a_codes, a_scales, w_codes, w_scales, group, out,
                 group_acc)


def rotate_quant_w4a4_gemm(x: torch.Tensor, w_codes: torch.Tensor, w_scales: torch.Tensor,
                           group: int, signs: torch.Tensor | None = None,
                           out: torch.Tensor | None = None, return_codes: bool = False):
    """Online rotation in the decode GEMM (hr_rotate_quant_w4a4_gemm): the bf16
    activation rows x [M][K] (M <= 16) are rotated, int4-quantized and
    multiplied with the packed int4 weights w_codes [N][K/2] in one kernel.
    Returns C [M][N] fp32, or (C, a_codes, a_scales) with the activation codes
    and scales the GEMM used when return_codes."""
    M, K = _rows_of(x, "x", (torch.bfloat16,))
    N, kw = _rows_of(w_codes, "w_codes", (torch.uint8,))
    if 2 * kw != K:
        raise ValueError(f"w_codes {tuple(w_codes.shape)} does not match K = {K} of x")
    g = _group(group, K)
    if not isinstance(w_scales, torch.Tensor):
        raise TypeError("w_scales must be a tensor")
    sd = _scale_dtype(w_scales.dtype)
    ax = _arg(x, "x", torch.bfloat16, (M, K))
    asg = _arg(signs, "signs", torch.int8, (K,))
    aw = _arg(w_codes, "w_codes", torch.uint8, (N, kw))
    asw = _arg(w_scales, "w_scales", sd, (N, K // g))
    _arg(out, "out", torch.float32, (M, N))
    dev = x.device
    c = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=dev)
    ac = asc = None
    if return_codes:
        ac = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
        asc = torch.empty((M, K // g), dtype=sd, device=dev)
    px, ps, pw, psw, pc, pac, pasc = _ptrs(ax, asg, aw, asw, ("out", c), ("a_codes", ac),
                                           ("a_scales", asc))
    _check(lib.hr_rotate_quant_w4a4_gemm(px, HR_BF16, ps, g, pw, psw, _dtype_code(sd), M, N, K, pc, pac,
                                         pasc, _stream(dev)), "hr_rotate_quant_w4a4_gemm")
    return (c, ac, asc) if return_codes else c


def fp6_rows(rows: int) -> int:
    """Rows of a tiled fp6 operand of `rows` rows (panels of 128)."""
    return (rows + 127) // 128 * 128


def w4a4_to_fp6(codes: torch.Tensor, scales: torch.Tensor | None = None, group: int | None = None,
                out: torch.Tensor | None = None, out_scales: torch.Tensor | None = None):
    """Packed int4 codes [rows][K/2] (and their scales [rows][K/G]) -> the
    tiled fp6 operand format of hr_w4a4_gemm_fp6 (hr_w4a4_to_fp6): the tiles
    as a [fp6_rows(rows)][K*3/4] uint8 tensor, and, with scales, the scales
    transposed to [K/G][fp6_rows(rows)].  Returns the tiles, or (tiles,
    scales) when scales are given."""
    rows, half = _rows_of(codes, "codes", (torch.uint8,))
    K = 2 * half
    if K % 128:
        raise ValueError(f"K={K} is not a multiple of 128")
    P = fp6_rows(rows)
    ac = _arg(codes, "codes", torch.uint8, (rows, half))
    _arg(out, "out", torch.uint8, (P, K * 3 // 4))
    o = out if out is not None else torch.empty((P, K * 3 // 4), dtype=torch.uint8, device=codes.device)
    if scales is None:
        if group is not None or out_scales is not None:
            raise ValueError("group and out_scales go with scales")
        pc, po = _ptrs(ac, ("out", o))
        _check(lib.hr_w4a4_to_fp6(pc, None, 0, rows, K, 0, po, None, _stream(codes.device)), "hr_w4a4_to_fp6")
        return o
    if not isinstance(scales, torch.Tensor):
        raise TypeError("scales must be a tensor")
    if group not in (128, 256) or K % group:
        raise ValueError(f"group={group} must be 128 or 256 and divide K={K}")
    sd = _scale_dtype(scales.dtype)
    asc = _arg(scales, "scales", sd, (rows, K // group))
    _arg(out_scales, "out_scales", sd, (K // group, P))
    os_ = out_scales if out_scales is not None else torch.empty((K // group, P), dtype=sd, device=codes.device)
    pc, ps, po, pos = _ptrs(ac, asc, ("out", o), ("out_scales", os_))
    _check(lib.hr_w4a4_to_fp6(pc, ps, _dtype_code(sd), rows, K, group, po, pos, _stream(codes.device)),
           "hr_w4a4_to_fp6")
    return o, os_


def rotate_quant_fp6(x: torch.Tensor, group: int, signs: torch.Tensor | None = None,
                     scale_dtype=torch.float16, out: torch.Tensor | None = None,
                     out_scales: torch.Tensor | None = None):
    """Rotation + int4 quantization of bf16 rows (n = 2048 or 4096) with the
    codes in the tiled fp6 format and the scales transposed
    (hr_rotate_quant_fp6): returns (tiles [fp6_rows(rows)][n*3/4] uint8,
    scales [n/G][fp6_rows(rows)]); the padding rows are not written."""
    rows, n = _rows_of(x, "x", (torch.bfloat16,))
    ax = _arg(x, "x", torch.bfloat16, (rows, n))
    asg = _arg(signs, "signs", torch.int8, (n,))
    if group not in (128, 256) or n not in (2048, 4096):
        raise ValueError(f"group={group} must be 128 or 256 and n={n} 2048 or 4096")
    sd = _scale_dtype(scale_dtype)
    P = fp6_rows(rows)
    _arg(out, "out", torch.uint8, (P, n * 3 // 4))
    _arg(out_scales, "out_scales", sd, (n // group, P))
    o = out if out is not None else torch.empty((P, n * 3 // 4), dtype=torch.uint8, device=x.device)
    os_ = out_scales if out_scales is not None else torch.empty((n // group, P), dtype=sd, device=x.device)
    px, ps, po, pos = _ptrs(ax, asg, ("out", o), ("out_scales", os_))
    _check(lib.hr_rotate_quant_fp6(px, HR_BF16, ps, rows, n, group, _dtype_code(sd), po, pos, _stream(x.device)),
           "hr_rotate_quant_fp6")
    return o, os_


def w4a4_gemm_fp6(a_f6: torch.Tensor, a_scales: torch.Tensor, w_f6: torch.Tensor,
                  w_scales: torch.Tensor, group: int, M: int, out: torch.Tensor | None = None,
                  group_acc: bool = False):
    """C = A W^T on operands in the tiled fp6 format (hr_w4a4_gemm_fp6), as
    w4a4_to_fp6 writes them: a_f6 [fp6_rows(M)][K*3/4] and a_scales
    [K/G][fp6_rows(M)] for the M activation rows, w_f6 [N][K*3/4] and w_scales
    [K/G][N] for the N weight rows.  Returns as w4a4_gemm."""
    if not isinstance(a_scales, torch.Tensor) or not isinstance(w_scales, torch.Tensor):
        raise TypeError("a_scales and w_scales must be tensors")
    if a_scales.dtype != w_scales.dtype:
        raise TypeError("a_scales and w_scales must share a dtype")
    if not isinstance(M, int) or M < 0:
        raise ValueError(f"M={M} must be a non-negative int")
    N, kw = _rows_of(w_f6, "w_f6", (torch.uint8,))
    _, ka = _rows_of(a_f6, "a_f6", (torch.uint8,))
    if ka % 3 or kw != ka:
        raise ValueError(f"a_f6 {tuple(a_f6.shape)} and w_f6 {tuple(w_f6.shape)} are not [.][K*3/4]")
    K = ka * 4 // 3
    g = _group(group, K)
    sd = _scale_dtype(a_scales.dtype)
    aa = _arg(a_f6, "a_f6", torch.uint8, (fp6_rows(M), ka))
    asa = _arg(a_scales, "a_scales", sd, (K // g, fp6_rows(M)))
    aw = _arg(w_f6, "w_f6", torch.uint8, (N, kw))
    asw = _arg(w_scales, "w_scales", sd, (K // g, N))
    _arg(out, "out", torch.float32, (M, N))
    dev = a_f6.device
    c = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=dev)
    acc = torch.empty((M, N, K // g), dtype=torch.int32, device=dev) if group_acc else None
    pa, psa, pw, psw, pc, pacc = _ptrs(aa, asa, aw, asw, ("out", c), ("group_acc", acc))
    _check(lib.hr_w4a4_gemm_fp6(pa, psa, pw, psw, _dtype_code(sd), M, N, K, g, pc, pacc, _stream(dev)),
           "hr_w4a4_gemm_fp6")
    return (c, acc) if group_acc else c
