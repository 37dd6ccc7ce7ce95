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
    assert hr.lib.hr_abi_version() == 3
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
    assert f(P, P, P, P, hr.HR_F16, 16, 64, 256, 32, P, None, None) == hr.HR_EUNSUPPORTED
    assert f(P, P, P, P, hr.HR_BF16, 16, 64, 256, 128, P, None, None) == hr.HR_EINVAL
    assert f(P, P, P, P, hr.HR_F16, -1, 64, 256, 128, P, None, None) == hr.HR_EINVAL
    assert f(P, P, P, P, hr.HR_F16, 16, 64, 256, 128, P, P + 4, None) == hr.HR_EINVAL
    assert f(P, P, P, P, hr.HR_F16, 0, 64, 256, 128, P, None, None) == hr.HR_OK
    assert f(P, P, P, P, hr.HR_F16, 16, 64, 131072, 128, P, None, None) == hr.HR_EUNSUPPORTED


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
