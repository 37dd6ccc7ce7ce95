"""GPU parity of the W4A8 path (int8 activations, int4 weights) against the
oracle: hr_rotate_quant_int8 on every kernel path that serves it, and
hr_w4a8_gemm on the prefill, decode and simple kernels.  All calls go
through the C ABI (the ctypes binding)."""
import numpy as np
import pytest
import torch

import hr_inputs
import oracle
from parity import check_gemm, check_quant

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _hr():
    import hadamard_rotation_int4_amd as hr
    return hr


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


# ------------------------------------------------------ rotate + int8 quantize

@pytest.mark.parametrize("n,group", [(2048, 128), (2048, 32), (2048, 64), (2048, 256),
                                     (1024, 64), (4096, 128), (64, 32)])
@pytest.mark.parametrize("scale_mode", ["f16", "f32"])
def test_rotate_quant_int8(n, group, scale_mode):
    """bf16 rows: the matrix-core kernel at n = 2048, the generic kernel otherwise."""
    hr = _hr()
    inp = hr_inputs.rht_inputs(rows=301, n=n, seed=400 + n + group)
    sd = torch.float16 if scale_mode == "f16" else torch.float32
    codes, scales = hr.rotate_quant_int8(inp.x.to(DEV), group, _t(inp.signs), scale_dtype=sd)
    assert codes.dtype == torch.int8 and codes.shape == (301, n)
    y64 = oracle.hadamard.rht(inp.x.float().numpy(), inp.signs)
    check_quant(codes.cpu().numpy(), scales.cpu().numpy(), y64, group, scale_mode, bits=8)


def test_rotate_quant_int8_fp32_input():
    hr = _hr()
    n, group = 2048, 128
    x = np.random.default_rng(31).standard_normal((90, n)).astype(np.float32)
    x[5] = 0.0
    d = hr_inputs.sign_vector(np.random.default_rng(32), n)
    codes, scales = hr.rotate_quant_int8(_t(x), group, _t(d))
    codes, scales = codes.cpu().numpy(), scales.cpu().numpy()
    assert np.all(codes[5] == 0) and np.all(scales[5] == 0)
    check_quant(codes, scales, oracle.hadamard.rht(x, d), group, "f16", bits=8)


@pytest.mark.parametrize("group", [32, 128, 256])
def test_rotate_quant_int8_large_dynamic_range_bf16(group):
    """Rows spanning many binades (fp16-subnormal scales), a zero and a tiny row."""
    hr = _hr()
    n = 2048
    rng = np.random.default_rng(33 + group)
    x = (rng.standard_normal((67, n)) * np.exp2(rng.integers(-30, 10, size=(67, 1)))).astype(np.float32)
    x[7] = 0.0
    x[8] = 1e-30
    xb = torch.from_numpy(x).to(torch.bfloat16)
    d = hr_inputs.sign_vector(rng, n)
    codes, scales = hr.rotate_quant_int8(xb.to(DEV), group, _t(d))
    codes, scales = codes.cpu().numpy(), scales.cpu().numpy()
    assert np.all(codes[7] == 0) and np.all(scales[7] == 0)
    assert np.all(codes[8] == 0) and np.all(scales[8] == 0)
    check_quant(codes, scales, oracle.hadamard.rht(xb.float().numpy(), d), group, "f16", bits=8)


def test_rotate_quant_int8_mixed_radix():
    hr = _hr()
    m, p, group = 7, 2048, 128
    mi = hr_inputs.mixed_inputs(rows=19, m=m, p=p, seed=34)
    codes, scales = hr.rotate_quant_int8(mi.x.to(DEV), group, _t(mi.signs), _t(mi.block))
    y64 = oracle.mixed_radix.mixed_radix(mi.x.float().numpy(), mi.signs, mi.block, p)
    check_quant(codes.cpu().numpy(), scales.cpu().numpy(), y64, group, "f16", bits=8)


def test_rotate_quant_int8_zero_rows():
    hr = _hr()
    codes, scales = hr.rotate_quant_int8(torch.empty((0, 2048), dtype=torch.bfloat16, device=DEV), 128)
    assert codes.shape == (0, 2048)


# ---------------------------------------------------------------- W4A8 GEMM

def _gemm_case(M, N, K, group, scale_mode, seed):
    hr = _hr()
    gi = hr_inputs.gemm_w4a8_inputs(M=M, N=N, K=K, group=group, seed=seed)
    sd = np.float16 if scale_mode == "f16" else np.float32
    sa, sw = gi.a_scales.astype(sd), gi.w_scales.astype(sd)
    c, acc = hr.w4a8_gemm(_t(gi.a_codes), _t(sa), _t(gi.w_codes), _t(sw), group, group_acc=True)
    c_ref, acc_ref, bound = oracle.gemm.w4a8_gemm(gi.a_codes, sa, gi.w_codes, sw, group,
                                                  return_sums=True)
    check_gemm(c.cpu().numpy(), c_ref, bound, acc.cpu().numpy(), acc_ref)
    c2 = hr.w4a8_gemm(_t(gi.a_codes), _t(sa), _t(gi.w_codes), _t(sw), group)
    assert torch.equal(c2, c)


@pytest.mark.parametrize("M,N,K,group,scale_mode", [
    (130, 256, 1024, 128, "f16"),    # prefill tiles, ragged M
    (300, 512, 768, 128, "f16"),
    (257, 256, 512, 64, "f16"),      # 64-code stages
    (200, 512, 1024, 256, "f16"),    # two stages per group
    (1024, 2048, 512, 128, "f16"),
    (160, 256, 512, 128, "f32"),     # fp32 scales
    (140, 512, 768, 64, "f32"),
    (100, 192, 1024, 128, "f16"),    # N not a multiple of 128: the simple kernel
    (70, 64, 512, 256, "f32"),
])
def test_w4a8_gemm_prefill(M, N, K, group, scale_mode):
    _gemm_case(M, N, K, group, scale_mode, seed=1000 + M)


@pytest.mark.parametrize("M,N,K,group,scale_mode", [
    (16, 256, 512, 128, "f16"),
    (1, 64, 256, 256, "f16"),
    (16, 128, 768, 256, "f16"),
    (12, 128, 2560, 128, "f16"),
    (7, 192, 4096, 64, "f32"),
    (16, 64, 16384, 64, "f16"),
    (3, 256, 1536, 256, "f32"),
])
def test_w4a8_gemm_decode(M, N, K, group, scale_mode):
    _gemm_case(M, N, K, group, scale_mode, seed=1100 + K + M)


@pytest.mark.parametrize("M", [16, 160])
def test_w4a8_gemm_extreme_codes(M):
    """-128 and 127 activations against -8 and 7 weights over whole groups."""
    hr = _hr()
    N, K, group = 128, 512, 256
    rng = np.random.default_rng(35 + M)
    a = rng.choice(np.array([-128, -127, 127], dtype=np.int8), size=(M, K))
    w = rng.choice(np.array([-8, 7]), size=(N, K))
    wp = oracle.quant.pack_int4(w)
    sa = rng.uniform(0.0001, 0.005, size=(M, K // group)).astype(np.float16)
    sw = rng.uniform(0.001, 0.05, size=(N, K // group)).astype(np.float16)
    c, acc = hr.w4a8_gemm(_t(a), _t(sa), _t(wp), _t(sw), group, group_acc=True)
    c_ref, acc_ref, bound = oracle.gemm.w4a8_gemm(a, sa, wp, sw, group, return_sums=True)
    check_gemm(c.cpu().numpy(), c_ref, bound, acc.cpu().numpy(), acc_ref)


def test_w4a8_pipeline_beats_w4a4():
    """Rotated activations quantized to int8 (W4A8) against int4 (W4A4), same
    int4 weights: the experiment page's third finding, that int8 activations
    carry most of the accuracy back."""
    hr = _hr()
    M, N, K, group = 64, 128, 2048, 128
    rng = np.random.default_rng(36)
    a = rng.standard_normal((M, K)).astype(np.float32)
    a[:, rng.choice(K, 8, replace=False)] *= 20
    w = rng.standard_normal((N, K)).astype(np.float32)
    dd = _t(hr_inputs.sign_vector(rng, K))
    wc, ws = hr.rotate_quant_int4(_t(w), group, dd)
    a8, s8 = hr.rotate_quant_int8(_t(a), group, dd)
    a4, s4 = hr.rotate_quant_int4(_t(a), group, dd)
    c8 = hr.w4a8_gemm(a8, s8, wc, ws, group).cpu().numpy()
    c4 = hr.w4a4_gemm(a4, s4, wc, ws, group).cpu().numpy()
    c8_ref, _, b8 = oracle.gemm.w4a8_gemm(a8.cpu().numpy(), s8.cpu().numpy(), wc.cpu().numpy(),
                                          ws.cpu().numpy(), group, return_sums=True)
    check_gemm(c8, c8_ref, b8)
    exact = a.astype(np.float64) @ w.astype(np.float64).T
    e8 = np.linalg.norm(c8 - exact) / np.linalg.norm(exact)
    e4 = np.linalg.norm(c4 - exact) / np.linalg.norm(exact)
    assert e8 < 0.8 * e4 and e8 < 0.15, (e8, e4)


# ---------------------------------------------------------------- full sizes

def test_rotate_quant_int8_65536x2048():
    hr = _hr()
    inp = hr_inputs.rht_inputs()
    codes, scales = hr.rotate_quant_int8(inp.x.to(DEV), 128, _t(inp.signs))
    rows = np.unique(np.concatenate([np.random.default_rng(37).choice(inp.rows, 128, replace=False),
                                     [0, inp.rows - 1]]))
    ri = torch.from_numpy(rows).to(DEV)
    y64 = oracle.hadamard.rht(inp.x[rows].float().numpy(), inp.signs)
    check_quant(codes[ri].cpu().numpy(), scales[ri].cpu().numpy(), y64, 128, "f16", bits=8)


@pytest.mark.parametrize("M", [4096, 16])
def test_w4a8_gemm_4096(M):
    hr = _hr()
    gi = hr_inputs.gemm_w4a8_inputs(M=M)
    c, acc = hr.w4a8_gemm(_t(gi.a_codes), _t(gi.a_scales), _t(gi.w_codes), _t(gi.w_scales), 128,
                          group_acc=True)
    rows = np.unique(np.concatenate([np.random.default_rng(38).choice(M, min(M, 24), replace=False),
                                     [0, M - 1]]))
    c_ref, acc_ref, bound = oracle.gemm.w4a8_gemm(gi.a_codes, gi.a_scales, gi.w_codes, gi.w_scales,
                                                  128, rows=rows, return_sums=True)
    ri = torch.from_numpy(rows).to(DEV)
    check_gemm(c[ri].cpu().numpy(), c_ref, bound, acc[ri].cpu().numpy(), acc_ref)
