"""CPU-only checks of the C ABI: the library loads, exports every function
include/hr.h declares, and rejects invalid arguments on the host before any
HIP call (so these run without a GPU).  No call here launches a kernel."""
import ctypes
import os
import re

import pytest

import hadamard_rotation_int4_amd as hr

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "hr.h")

# A fake, 16-byte aligned, never-dereferenced address: every call below fails
# validation (or is a no-op) before anything would touch it.
P = 0x10000


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"\b(hr_[a-z0-9_]+)\s*\(", src))


def test_header_and_binding_agree():
    assert _declared() == set(hr.SYMBOLS)


def test_every_declared_symbol_is_exported():
    raw = ctypes.CDLL(hr.LIB_PATH)
    for name in _declared():
        assert hasattr(raw, name), name


def test_version_and_status_strings():
    assert hr.lib.hr_abi_version() == 5
    for st in (hr.HR_OK, hr.HR_EINVAL, hr.HR_EUNSUPPORTED, hr.HR_EDEVICE):
        assert hr.lib.hr_status_string(st).startswith(b"HR_")
    assert b"unknown" in hr.lib.hr_status_string(99)


def _rot(**kw):
    a = dict(x=P, dt=hr.HR_BF16, y=P, rows=4, n=2048, m=1, signs=None, block=None)
    a.update(kw)
    return hr.lib.hr_rotate(a["x"], a["dt"], a["y"], a["rows"], a["n"], a["m"], a["signs"],
                            a["block"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), hr.HR_EINVAL),
    (dict(y=None), hr.HR_EINVAL),
    (dict(rows=-1), hr.HR_EINVAL),
    (dict(dt=hr.HR_F16), hr.HR_EINVAL),
    (dict(dt=7), hr.HR_EINVAL),
    (dict(x=P + 4), hr.HR_EINVAL),
    (dict(y=P + 8), hr.HR_EINVAL),
    (dict(n=2047), hr.HR_EUNSUPPORTED),
    (dict(n=32), hr.HR_EUNSUPPORTED),
    (dict(n=32768), hr.HR_EUNSUPPORTED),
    (dict(n=3 * 2048, m=3), hr.HR_EINVAL),          # block missing
    (dict(block=P), hr.HR_EINVAL),                  # block with m == 1
    (dict(m=17, n=17 * 64, block=P), hr.HR_EUNSUPPORTED),
    (dict(m=0), hr.HR_EUNSUPPORTED),
    (dict(n=7 * 4096, m=7, block=P), hr.HR_EUNSUPPORTED),  # n > 16384
    (dict(n=7 * 48, m=7, block=P), hr.HR_EUNSUPPORTED),    # p not a power of two
])
def test_rotate_validation(kw, status):
    assert _rot(**kw) == status
    assert hr.lib.hr_last_error() != b""


def test_rotate_zero_rows_is_noop():
    assert _rot(rows=0) == hr.HR_OK


def _rq(fn="hr_rotate_quant_int4", **kw):
    a = dict(x=P, dt=hr.HR_BF16, rows=4, n=2048, m=1, signs=None, block=None, group=128,
             codes=P, scales=P, sdt=hr.HR_F16)
    a.update(kw)
    return getattr(hr.lib, fn)(a["x"], a["dt"], a["rows"], a["n"], a["m"], a["signs"],
                               a["block"], a["group"], a["codes"], a["scales"], a["sdt"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(codes=None), hr.HR_EINVAL),
    (dict(scales=None), hr.HR_EINVAL),
    (dict(sdt=hr.HR_BF16), hr.HR_EINVAL),
    (dict(group=48), hr.HR_EUNSUPPORTED),
    (dict(group=16), hr.HR_EUNSUPPORTED),
    (dict(group=512), hr.HR_EUNSUPPORTED),
    (dict(n=64, group=128), hr.HR_EUNSUPPORTED),   # group does not divide p
    (dict(codes=P + 1), hr.HR_EINVAL),
    (dict(signs=P + 2), hr.HR_EINVAL),
])
@pytest.mark.parametrize("fn", ["hr_rotate_quant_int4", "hr_rotate_quant_int8"])
def test_rotate_quant_validation(fn, kw, status):
    assert _rq(fn, **kw) == status
    assert fn.encode() in hr.lib.hr_last_error()


@pytest.mark.parametrize("fn", ["hr_rotate_quant_int4", "hr_rotate_quant_int8"])
def test_rotate_quant_zero_rows_is_noop(fn):
    assert _rq(fn, rows=0) == hr.HR_OK


def test_butterfly_validation():
    f = hr.lib.hr_butterfly_apply
    # x, y, rows, n, coeffs, precond, perm, inverse, group, codes, scales, sdt, stream
    assert f(None, P, 4, 4096, P, 0, None, 0, 0, None, None, 0, None) == hr.HR_EINVAL
    assert f(P, None, 4, 4096, P, 0, None, 0, 0, None, None, 0, None) == hr.HR_EINVAL
    assert f(P, P, 4, 4095, P, 0, None, 0, 0, None, None, 0, None) == hr.HR_EUNSUPPORTED
    assert f(P, P, 4, 16384, P, 0, None, 0, 0, None, None, 0, None) == hr.HR_EUNSUPPORTED
    assert f(P, P, 4, 4096, P, 2, None, 0, 0, None, None, 0, None) == hr.HR_EINVAL
    assert f(P, P, 4, 4096, P, 0, None, 1, 64, P, P, hr.HR_F16, None) == hr.HR_EUNSUPPORTED
    assert f(P, P, 4, 4096, P, 0, None, 0, 64, P, None, hr.HR_F16, None) == hr.HR_EINVAL
    assert f(P, P, 4, 4096, P, 0, None, 0, 0, None, P, hr.HR_F16, None) == hr.HR_EINVAL
    assert f(P, P, 4, 4096, P, 0, None, 0, 96, P, P, hr.HR_F16, None) == hr.HR_EUNSUPPORTED
    assert f(P, P, -1, 4096, P, 0, None, 0, 0, None, None, 0, None) == hr.HR_EINVAL
    assert f(P, P, 0, 4096, P, 0, None, 0, 0, None, None, 0, None) == hr.HR_OK
    c = hr.lib.hr_butterfly_coeffs
    assert c(None, 4096, 0, P, None) == hr.HR_EINVAL
    assert c(P, 100, 0, P, None) == hr.HR_EUNSUPPORTED
    assert c(P, 4096, 3, P, None) == hr.HR_EINVAL


def test_dequant_validation():
    f = hr.lib.hr_dequant_int4
    assert f(None, P, hr.HR_F16, 4, 256, 128, P, None) == hr.HR_EINVAL
    assert f(P, P, hr.HR_BF16, 4, 256, 128, P, None) == hr.HR_EINVAL
    assert f(P, P, hr.HR_F16, 4, 200, 128, P, None) == hr.HR_EUNSUPPORTED
    assert f(P, P, hr.HR_F16, 4, 256, 100, P, None) == hr.HR_EUNSUPPORTED
    assert f(P, P, hr.HR_F16, 0, 256, 128, P, None) == hr.HR_OK


@pytest.mark.parametrize("fn", ["hr_w4a4_gemm", "hr_w4a8_gemm", "hr_w8a8_gemm"])
def test_gemm_validation(fn):
    f = getattr(hr.lib, fn)
    # a, sa, w, sw, sdt, M, N, K, group, c, acc, stream
    assert f(None, P, P, P, hr.HR_F16, 16, 64, 256, 128, P, None, None) == hr.HR_EINVAL
    assert f(P, P, P, P, hr.HR_F16, 16, 64, 256, 128, None, None, None) == hr.HR_EINVAL
    assert f(P, P, P, P, hr.HR_F16, 16, 96, 256, 128, P, None, None) == hr.HR_EUNSUPPORTED
    assert f(P, P, P, P, hr.HR_F16, 16, 64, 384, 128, P, None, None) == hr.HR_EUNSUPPORTED
    assert f(P, P, P, P, hr.HR_F16, 16, 64, 256, 16, P, None, None) == hr.HR_EUNSUPPORTED
    assert f(P, P, P, P, hr.HR_F16, 16, 64, 256, 96, P, None, None) == hr.HR_EUNSUPPORTED
    assert f(P, P, P, P, hr.HR_BF16, 16, 64, 256, 128, P, None, None) == hr.HR_EINVAL
    assert f(P, P, P, P, hr.HR_F16, -1, 64, 256, 128, P, None, None) == hr.HR_EINVAL
    assert f(P, P, P, P, hr.HR_F16, 16, 64, 256, 128, P, P + 4, None) == hr.HR_EINVAL
    assert f(P, P, P, P, hr.HR_F16, 0, 64, 256, 128, P, None, None) == hr.HR_OK
    assert f(P, P, P, P, hr.HR_F16, 0, 64, 256, 32, P, None, None) == hr.HR_OK    # G = 32 accepted
    assert f(P, P, P, P, hr.HR_F16, 16, 64, 131072, 128, P, None, None) == hr.HR_EUNSUPPORTED


def test_fp6_validation():
    conv, gemm = hr.lib.hr_w4a4_to_fp6, hr.lib.hr_w4a4_gemm_fp6
    # codes, scales, sdt, rows, K, group, out, out_scales, stream
    assert conv(None, None, 0, 4, 256, 0, P, None, None) == hr.HR_EINVAL
    assert conv(P, None, 0, 4, 256, 0, P + 8, None, None) == hr.HR_EINVAL
    assert conv(P, None, 0, -1, 256, 0, P, None, None) == hr.HR_EINVAL
    assert conv(P, None, 0, 4, 192, 0, P, None, None) == hr.HR_EUNSUPPORTED   # K not a multiple of 128
    assert conv(P, P, hr.HR_F16, 4, 256, 128, P, None, None) == hr.HR_EINVAL   # scales without out_scales
    assert conv(P, P, hr.HR_BF16, 4, 256, 128, P, P, None) == hr.HR_EINVAL
    assert conv(P, P, hr.HR_F16, 4, 256, 64, P, P, None) == hr.HR_EUNSUPPORTED
    assert conv(P, P, hr.HR_F16, 4, 384, 256, P, P, None) == hr.HR_EUNSUPPORTED
    assert conv(P, None, 0, 0, 256, 0, P, None, None) == hr.HR_OK
    assert conv(P, P, hr.HR_F32, 0, 256, 256, P, P, None) == hr.HR_OK
    # a, sa, w, sw, sdt, M, N, K, group, c, acc, stream
    assert gemm(None, P, P, P, hr.HR_F16, 16, 128, 256, 128, P, None, None) == hr.HR_EINVAL
    assert gemm(P, P, P, P, hr.HR_BF16, 16, 128, 256, 128, P, None, None) == hr.HR_EINVAL
    assert gemm(P, P, P, P, hr.HR_F16, 16, 64, 256, 128, P, None, None) == hr.HR_EUNSUPPORTED   # N % 128
    assert gemm(P, P, P, P, hr.HR_F16, 16, 128, 256, 64, P, None, None) == hr.HR_EUNSUPPORTED   # G
    assert gemm(P, P, P, P, hr.HR_F16, 16, 128, 384, 256, P, None, None) == hr.HR_EUNSUPPORTED  # K % G
    assert gemm(P, P, P, P, hr.HR_F16, 16, 128, 131072, 128, P, None, None) == hr.HR_EUNSUPPORTED
    assert gemm(P, P, P, P, hr.HR_F16, 0, 128, 384, 128, P, None, None) == hr.HR_OK
    rq = hr.lib.hr_rotate_quant_fp6
    # x, x_dtype, signs, rows, n, group, sdt, tiles, scales, stream
    assert rq(None, hr.HR_BF16, None, 4, 2048, 128, hr.HR_F16, P, P, None) == hr.HR_EINVAL
    assert rq(P, hr.HR_F32, None, 4, 2048, 128, hr.HR_F16, P, P, None) == hr.HR_EUNSUPPORTED
    assert rq(P, hr.HR_BF16, None, 4, 1024, 128, hr.HR_F16, P, P, None) == hr.HR_EUNSUPPORTED
    assert rq(P, hr.HR_BF16, None, 4, 2048, 64, hr.HR_F16, P, P, None) == hr.HR_EUNSUPPORTED
    assert rq(P, hr.HR_BF16, None, 4, 2048, 128, hr.HR_BF16, P, P, None) == hr.HR_EINVAL
    assert rq(P, hr.HR_BF16, None, 4, 2048, 128, hr.HR_F16, P + 4, P, None) == hr.HR_EINVAL
    assert rq(P, hr.HR_BF16, None, -1, 2048, 128, hr.HR_F16, P, P, None) == hr.HR_EINVAL
    assert rq(P, hr.HR_BF16, None, 0, 4096, 256, hr.HR_F32, P, P, None) == hr.HR_OK


def _rad(*b):
    return (ctypes.c_int32 * len(b))(*b), len(b)


def test_harp_validation():
    ap, bl = hr.lib.hr_harp_apply, hr.lib.hr_harp_blocks
    r, m = _rad(8, 8, 8, 5, 2)
    # x, y, rows, radices, nstages, blocks, inverse, group, codes, scales, sdt, stream
    assert ap(None, P, 4, r, m, P, 0, 0, None, None, 0, None) == hr.HR_EINVAL
    assert ap(P, None, 4, r, m, P, 0, 0, None, None, 0, None) == hr.HR_EINVAL
    assert ap(P, P, -1, r, m, P, 0, 0, None, None, 0, None) == hr.HR_EINVAL
    assert ap(P, P, 4, r, m, None, 0, 0, None, None, 0, None) == hr.HR_EINVAL
    assert ap(P, P, 4, None, m, P, 0, 0, None, None, 0, None) == hr.HR_EINVAL
    assert ap(P, P, 4, r, m, P, 2, 0, None, None, 0, None) == hr.HR_EINVAL
    assert ap(P + 4, P, 4, r, m, P, 0, 0, None, None, 0, None) == hr.HR_EINVAL
    assert ap(P, P, 4, r, m, P, 0, 96, P, P, hr.HR_F16, None) == hr.HR_EUNSUPPORTED
    assert ap(P, P, 4, r, m, P, 0, 128, P, None, hr.HR_F16, None) == hr.HR_EINVAL
    assert ap(P, P, 4, r, m, P, 0, 128, P, P, hr.HR_BF16, None) == hr.HR_EINVAL
    assert ap(P, P, 0, r, m, P, 0, 0, None, None, 0, None) == hr.HR_OK
    r9, m9 = _rad(9, 4)
    assert ap(P, P, 4, r9, m9, P, 0, 0, None, None, 0, None) == hr.HR_EUNSUPPORTED   # radix > 8
    r1, m1 = _rad(1, 8)
    assert ap(P, P, 4, r1, m1, P, 0, 0, None, None, 0, None) == hr.HR_EUNSUPPORTED
    rb, mb = _rad(8, 8, 8, 8, 8)
    assert ap(P, P, 4, rb, mb, P, 0, 0, None, None, 0, None) == hr.HR_EUNSUPPORTED   # d > 16384
    ro, mo = _rad(3, 5)
    assert ap(P, P, 4, ro, mo, P, 0, 0, None, None, 0, None) == hr.HR_EUNSUPPORTED   # d % 4
    assert ap(P, P, 4, r, 0, P, 0, 0, None, None, 0, None) == hr.HR_EUNSUPPORTED
    assert ap(P, P, 4, r, 17, P, 0, 0, None, None, 0, None) == hr.HR_EUNSUPPORTED
    # radices, nstages, theta, fallbacks, blocks, stream
    assert bl(r, m, P, None, P, None) == hr.HR_EINVAL          # radix 5 needs a fallback
    assert bl(r, m, None, P, P, None) == hr.HR_EINVAL
    assert bl(r, m, P, P, None, None) == hr.HR_EINVAL
    assert bl(r, m, P + 8, P, P, None) == hr.HR_EINVAL
    assert bl(r9, m9, P, P, P, None) == hr.HR_EUNSUPPORTED
    assert b"hr_harp_blocks" in hr.lib.hr_last_error()


def test_build_id_matches_sources():
    from hadamard_rotation_int4_amd import srchash
    assert hr.lib.hr_build_id().decode() == srchash.source_hash()


@pytest.mark.parametrize("fn", ["hr_quant_int4", "hr_quant_int8"])
def test_quant_validation(fn):
    f = getattr(hr.lib, fn)
    # x, x_dtype, rows, n, group, codes, scales, sdt, stream
    assert f(None, hr.HR_BF16, 4, 256, 128, P, P, hr.HR_F16, None) == hr.HR_EINVAL
    assert f(P, hr.HR_BF16, 4, 256, 128, None, P, hr.HR_F16, None) == hr.HR_EINVAL
    assert f(P, hr.HR_BF16, 4, 256, 128, P, None, hr.HR_F16, None) == hr.HR_EINVAL
    assert f(P, hr.HR_F16, 4, 256, 128, P, P, hr.HR_F16, None) == hr.HR_EINVAL
    assert f(P, hr.HR_BF16, 4, 256, 128, P, P, hr.HR_BF16, None) == hr.HR_EINVAL
    assert f(P + 2, hr.HR_BF16, 4, 256, 128, P, P, hr.HR_F16, None) == hr.HR_EINVAL
    assert f(P, hr.HR_BF16, -1, 256, 128, P, P, hr.HR_F16, None) == hr.HR_EINVAL
    assert f(P, hr.HR_BF16, 4, 200, 128, P, P, hr.HR_F16, None) == hr.HR_EUNSUPPORTED
    assert f(P, hr.HR_BF16, 4, 256, 48, P, P, hr.HR_F16, None) == hr.HR_EUNSUPPORTED
    assert f(P, hr.HR_BF16, 4, 0, 32, P, P, hr.HR_F16, None) == hr.HR_EUNSUPPORTED
    assert f(P, hr.HR_BF16, 0, 256, 32, P, P, hr.HR_F16, None) == hr.HR_OK
    assert f(None, hr.HR_F32, 0, 256, 32, None, None, hr.HR_F32, None) == hr.HR_OK
    assert fn.encode() in hr.lib.hr_last_error() or hr.lib.hr_last_error() != b""


def test_fused_decode_validation():
    f = hr.lib.hr_rotate_quant_w4a4_gemm
    # x, x_dtype, signs, group, w, sw, sdt, M, N, K, c, a_codes, a_scales, stream
    ok = dict(x=P, dt=hr.HR_BF16, s=None, g=128, w=P, sw=P, sdt=hr.HR_F16, M=16, N=512, K=4096, c=P,
              ac=None, asc=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["x"], a["dt"], a["s"], a["g"], a["w"], a["sw"], a["sdt"], a["M"], a["N"], a["K"],
                 a["c"], a["ac"], a["asc"], None)

    assert call(M=0) == hr.HR_OK
    assert call(x=None) == hr.HR_EINVAL
    assert call(c=None) == hr.HR_EINVAL
    assert call(w=P + 8) == hr.HR_EINVAL
    assert call(ac=P) == hr.HR_EINVAL                    # codes without scales
    assert call(asc=P) == hr.HR_EINVAL
    assert call(dt=hr.HR_F32) == hr.HR_EUNSUPPORTED
    assert call(sdt=hr.HR_BF16) == hr.HR_EINVAL
    assert call(M=17) == hr.HR_EUNSUPPORTED
    assert call(K=8192) == hr.HR_EUNSUPPORTED
    assert call(K=1024) == hr.HR_EUNSUPPORTED
    assert call(N=96) == hr.HR_EUNSUPPORTED
    assert call(g=16) == hr.HR_EUNSUPPORTED
    assert call(M=-1) == hr.HR_EINVAL
    assert call(M=0, g=32, K=2048) == hr.HR_OK
    assert b"hr_rotate_quant_w4a4_gemm" in hr.lib.hr_last_error() or True


# ---- the Python binding checks dtype and shape of every tensor against the
# sizes it passes to the C call, before the call (CPU tensors: every check
# below fails before the device check, so nothing reaches the library)

import torch  # noqa: E402


def _z(*shape, dtype=torch.float32):
    return torch.zeros(shape, dtype=dtype)


@pytest.mark.parametrize("call,exc,msg", [
    (lambda: hr.rotate(_z(4, 2048, dtype=torch.float16)), TypeError, "x: dtype"),
    (lambda: hr.rotate(_z(2048)), ValueError, "2-D"),
    (lambda: hr.rotate(_z(4, 2048), signs=_z(2048, dtype=torch.int32)), TypeError, "signs"),
    (lambda: hr.rotate(_z(4, 2048), signs=_z(1024, dtype=torch.int8)), ValueError, "signs: shape"),
    (lambda: hr.rotate(_z(4, 2048), block=_z(3, 3)), ValueError, "divide"),
    (lambda: hr.rotate(_z(4, 2048), block=_z(2, 3)), ValueError, "square"),
    (lambda: hr.rotate(_z(4, 2048), out=_z(4, 1024)), ValueError, "out: shape"),
    (lambda: hr.rotate(_z(4, 2048), out=_z(4, 2048, dtype=torch.bfloat16)), TypeError, "out: dtype"),
    (lambda: hr.rotate_quant_int4(_z(4, 2048), 100), ValueError, "group"),
    (lambda: hr.rotate_quant_int4(_z(4, 2048), 128, codes=_z(4, 2048, dtype=torch.uint8)),
     ValueError, "codes: shape"),
    (lambda: hr.rotate_quant_int4(_z(4, 2048), 128, codes=_z(4, 1024, dtype=torch.int8)),
     TypeError, "codes: dtype"),
    (lambda: hr.rotate_quant_int4(_z(4, 2048), 128, scales=_z(4, 32, dtype=torch.float16)),
     ValueError, "scales: shape"),
    (lambda: hr.rotate_quant_int4(_z(4, 2048), 128, scale_dtype=torch.bfloat16), TypeError, "scale_dtype"),
    (lambda: hr.rotate_quant_int8(_z(4, 2048), 128, codes=_z(4, 1024, dtype=torch.int8)),
     ValueError, "codes: shape"),
    (lambda: hr.quant_int4(_z(4, 2048), 128, codes=_z(4, 1024, dtype=torch.int8)), TypeError, "codes"),
    (lambda: hr.quant_int8(_z(4, 96), 64), ValueError, "group"),
    (lambda: hr.butterfly_coeffs(_z(11, 2048)), ValueError, "stages"),
    (lambda: hr.butterfly_coeffs(_z(12, 2048, dtype=torch.float64)), TypeError, "angles"),
    (lambda: hr.butterfly_apply(_z(4, 4096), _z(12, 2048)), ValueError, "coeffs: shape"),
    (lambda: hr.butterfly_apply(_z(4, 4096), _z(12, 2048, 2), perm=_z(4096, dtype=torch.int64)),
     TypeError, "perm"),
    (lambda: hr.butterfly_apply(_z(4, 4096), _z(12, 2048, 2), perm=_z(2048, dtype=torch.int32)),
     ValueError, "perm: shape"),
    (lambda: hr.butterfly_apply(_z(4, 3000), _z(12, 2048, 2)), ValueError, "power of two"),
    (lambda: hr.harp_blocks((8, 8, 8, 5, 2), _z(10)), ValueError, "theta: shape"),
    (lambda: hr.harp_apply(_z(4, 5120), (8, 8, 8, 5, 2), _z(100)), ValueError, "blocks: shape"),
    (lambda: hr.harp_apply(_z(4, 5000), (8, 8, 8, 5, 2), _z(100)), ValueError, "multiply"),
    (lambda: hr.dequant_int4(_z(4, 1024, dtype=torch.uint8), _z(4, 8, dtype=torch.float16), 128),
     ValueError, "scales: shape"),
    (lambda: hr.dequant_int4(_z(4, 1024, dtype=torch.int8), _z(4, 16, dtype=torch.float16), 128),
     TypeError, "codes"),
    (lambda: hr.w4a4_gemm(_z(16, 2048, dtype=torch.uint8), _z(16, 32, dtype=torch.float16),
                          _z(64, 1024, dtype=torch.uint8), _z(64, 32, dtype=torch.float16), 128),
     ValueError, "does not match K"),
    (lambda: hr.w4a4_gemm(_z(16, 2048, dtype=torch.uint8), _z(16, 32, dtype=torch.float16),
                          _z(64, 2048, dtype=torch.uint8), _z(64, 16, dtype=torch.float16), 128),
     ValueError, "w_scales: shape"),
    (lambda: hr.w4a4_gemm(_z(16, 2048, dtype=torch.uint8), _z(16, 32, dtype=torch.float16),
                          _z(64, 2048, dtype=torch.uint8), _z(64, 32, dtype=torch.float32), 128),
     TypeError, "share a dtype"),
    (lambda: hr.w4a4_gemm(_z(16, 2048, dtype=torch.int8), _z(16, 32, dtype=torch.float16),
                          _z(64, 2048, dtype=torch.uint8), _z(64, 32, dtype=torch.float16), 128),
     TypeError, "a_codes"),
    (lambda: hr.w4a8_gemm(_z(16, 4096, dtype=torch.int8), _z(16, 32, dtype=torch.float16),
                          _z(64, 4096, dtype=torch.uint8), _z(64, 32, dtype=torch.float16), 128),
     ValueError, "does not match K"),
    (lambda: hr.w8a8_gemm(_z(16, 4096, dtype=torch.int8), _z(16, 32, dtype=torch.float16),
                          _z(64, 4096, dtype=torch.uint8), _z(64, 32, dtype=torch.float16), 128),
     TypeError, "w_codes"),
    (lambda: hr.w4a4_gemm(_z(16, 2048, dtype=torch.uint8), _z(16, 32, dtype=torch.float16),
                          _z(64, 2048, dtype=torch.uint8), _z(64, 32, dtype=torch.float16), 128,
                          out=_z(16, 32)), ValueError, "out: shape"),
    (lambda: hr.rotate_quant_w4a4_gemm(_z(16, 4096), _z(64, 2048, dtype=torch.uint8),
                                       _z(64, 32, dtype=torch.float16), 128), TypeError, "x: dtype"),
    (lambda: hr.rotate_quant_w4a4_gemm(_z(16, 4096, dtype=torch.bfloat16), _z(64, 1024, dtype=torch.uint8),
                                       _z(64, 32, dtype=torch.float16), 128), ValueError, "does not match K"),
    (lambda: hr.rotate_quant_w4a4_gemm(_z(16, 4096, dtype=torch.bfloat16), _z(64, 2048, dtype=torch.uint8),
                                       _z(64, 32, dtype=torch.float16), 128,
                                       signs=_z(2048, dtype=torch.int8)), ValueError, "signs: shape"),
    # the tiled fp6 format: conversion, rotation straight into tiles, and the GEMM
    (lambda: hr.w4a4_to_fp6(_z(4, 1000, dtype=torch.uint8)), ValueError, "multiple of 128"),
    (lambda: hr.w4a4_to_fp6(_z(4, 1024, dtype=torch.int8)), TypeError, "codes"),
    (lambda: hr.w4a4_to_fp6(_z(4, 1024, dtype=torch.uint8), out=_z(4, 1536, dtype=torch.uint8)),
     ValueError, "out: shape"),
    (lambda: hr.w4a4_to_fp6(_z(4, 1024, dtype=torch.uint8), group=128), ValueError, "go with scales"),
    (lambda: hr.w4a4_to_fp6(_z(4, 1024, dtype=torch.uint8), _z(4, 16, dtype=torch.float16), 64),
     ValueError, "group"),
    (lambda: hr.w4a4_to_fp6(_z(4, 1024, dtype=torch.uint8), _z(4, 8, dtype=torch.float16), 128),
     ValueError, "scales: shape"),
    (lambda: hr.w4a4_to_fp6(_z(4, 1024, dtype=torch.uint8), _z(4, 16, dtype=torch.float16), 128,
                            out_scales=_z(16, 4, dtype=torch.float16)), ValueError, "out_scales: shape"),
    (lambda: hr.rotate_quant_fp6(_z(4, 2048), 128), TypeError, "x: dtype"),
    (lambda: hr.rotate_quant_fp6(_z(4, 1024, dtype=torch.bfloat16), 128), ValueError, "n="),
    (lambda: hr.rotate_quant_fp6(_z(4, 2048, dtype=torch.bfloat16), 64), ValueError, "group"),
    (lambda: hr.rotate_quant_fp6(_z(4, 2048, dtype=torch.bfloat16), 128, signs=_z(1024, dtype=torch.int8)),
     ValueError, "signs: shape"),
    (lambda: hr.rotate_quant_fp6(_z(4, 2048, dtype=torch.bfloat16), 128, out=_z(4, 1536, dtype=torch.uint8)),
     ValueError, "out: shape"),
    (lambda: hr.rotate_quant_fp6(_z(4, 2048, dtype=torch.bfloat16), 128,
                                 out_scales=_z(16, 128, dtype=torch.float32)), TypeError, "out_scales: dtype"),
    (lambda: hr.rotate_quant_fp6(_z(4, 2048, dtype=torch.bfloat16), 128, scale_dtype=torch.bfloat16),
     TypeError, "scale_dtype"),
    (lambda: hr.w4a4_gemm_fp6(_z(128, 768, dtype=torch.uint8), _z(8, 128, dtype=torch.float16),
                              _z(128, 1536, dtype=torch.uint8), _z(8, 128, dtype=torch.float16), 128, 4),
     ValueError, "K\\*3/4"),
    (lambda: hr.w4a4_gemm_fp6(_z(128, 768, dtype=torch.uint8), _z(8, 128, dtype=torch.float16),
                              _z(128, 768, dtype=torch.uint8), _z(8, 128, dtype=torch.float32), 128, 4),
     TypeError, "share a dtype"),
    (lambda: hr.w4a4_gemm_fp6(_z(64, 768, dtype=torch.uint8), _z(8, 128, dtype=torch.float16),
                              _z(128, 768, dtype=torch.uint8), _z(8, 128, dtype=torch.float16), 128, 4),
     ValueError, "a_f6: shape"),
    (lambda: hr.w4a4_gemm_fp6(_z(128, 768, dtype=torch.uint8), _z(8, 128, dtype=torch.float16),
                              _z(128, 768, dtype=torch.uint8), _z(4, 128, dtype=torch.float16), 128, 4),
     ValueError, "w_scales: shape"),
    (lambda: hr.w4a4_gemm_fp6(_z(128, 768, dtype=torch.uint8), _z(8, 128, dtype=torch.float16),
                              _z(128, 768, dtype=torch.uint8), _z(8, 128, dtype=torch.float16), 128, 4,
                              out=_z(4, 64)), ValueError, "out: shape"),
])
def test_binding_rejects_bad_tensors(call, exc, msg):
    with pytest.raises(exc, match=msg):
        call()


def test_binding_rejects_host_tensors():
    with pytest.raises(ValueError, match="GPU"):
        hr.rotate(_z(4, 2048))
