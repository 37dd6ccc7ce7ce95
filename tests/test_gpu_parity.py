"""GPU parity of every entry point against the oracle, at sizes the oracle
finishes in seconds that still span several workgroups and a ragged tail.
All calls go through the C ABI (the ctypes binding)."""
import math

import numpy as np
import pytest
import torch

import hr_inputs
import oracle
from parity import check_gemm, check_quant, check_rotated

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _hr():
    import hadamard_rotation_int4_amd as hr
    return hr


def _bf16_rows(rows, n, seed, outlier_scale=50.0):
    inp = hr_inputs.rht_inputs(rows=rows, n=n, seed=seed, outlier_scale=outlier_scale)
    return inp.x, inp.signs


# ---------------------------------------------------------------- rotation

@pytest.mark.parametrize("n", [64, 128, 512, 2048, 4096, 8192, 16384])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_rotate_pow2(n, dtype):
    hr = _hr()
    rows = 37
    inp = hr_inputs.rht_inputs(rows=rows, n=n, seed=100 + n, dtype=dtype)
    x, d = inp.x, inp.signs
    y = hr.rotate(x.to(DEV), torch.from_numpy(d).to(DEV)).cpu().numpy()
    y64 = oracle.hadamard.rht(x.float().numpy(), d)
    check_rotated(y, y64)


def test_rotate_without_signs_and_in_place():
    hr = _hr()
    x = torch.from_numpy(np.random.default_rng(1).standard_normal((19, 1024)).astype(np.float32))
    xd = x.to(DEV)
    y = hr.rotate(xd, None, out=xd).cpu().numpy()  # in place
    check_rotated(y, oracle.hadamard.rht(x.numpy(), None))


def test_rotate_closed_forms():
    hr = _hr()
    n = 2048
    d = hr_inputs.sign_vector(np.random.default_rng(5), n)
    x = np.zeros((2, n), dtype=np.float32)
    x[0, 0] = 1.0                 # delta: every output d_0 / sqrt(n)
    x[1] = d                      # sign vector: sqrt(n) e_0, exact zeros elsewhere
    y = hr.rotate(torch.from_numpy(x).to(DEV), torch.from_numpy(d).to(DEV)).cpu().numpy()
    np.testing.assert_allclose(y[0], d[0] / math.sqrt(n), rtol=1e-6)
    assert abs(y[1, 0] - math.sqrt(n)) <= 1e-6 * math.sqrt(n)
    assert np.all(y[1, 1:] == 0.0)


@pytest.mark.parametrize("rows", [1, 2, 3])
def test_rotate_closed_forms_bf16(rows):
    """bf16 input (the matrix-core path at n = 2048): a delta row gives d_0 / sqrt(n)
    everywhere, the sign vector itself gives sqrt(n) e_0 with exact zeros; one to
    three rows exercise the odd tail of the two-row step."""
    hr = _hr()
    n = 2048
    d = hr_inputs.sign_vector(np.random.default_rng(6), n)
    x = np.zeros((3, n), dtype=np.float32)
    x[0, 0] = 1.0
    x[1] = d
    x[2, 5] = -2.0
    xb = torch.from_numpy(x[:rows]).to(torch.bfloat16)
    y = hr.rotate(xb.to(DEV), torch.from_numpy(d).to(DEV)).cpu().numpy()
    np.testing.assert_allclose(y[0], d[0] / math.sqrt(n), rtol=1e-6)
    if rows > 1:
        assert abs(y[1, 0] - math.sqrt(n)) <= 1e-6 * math.sqrt(n)
        assert np.all(y[1, 1:] == 0.0)
    if rows > 2:
        h5 = np.array([(-1) ** bin(i & 5).count("1") for i in range(n)], dtype=np.float64)
        np.testing.assert_allclose(y[2], -2.0 * d[5] * h5 / math.sqrt(n), rtol=1e-6)


def test_rotate_zero_rows():
    hr = _hr()
    x = torch.empty((0, 2048), dtype=torch.bfloat16, device=DEV)
    assert hr.rotate(x).shape == (0, 2048)


# ------------------------------------------------------- rotate + quantize

@pytest.mark.parametrize("n,group", [(2048, 128), (2048, 32), (2048, 64), (2048, 256), (64, 32),
                                     (256, 64), (1024, 256), (4096, 128), (16384, 128), (4096, 256),
                                     (8192, 32)])
@pytest.mark.parametrize("scale_mode", ["f16", "f32"])
def test_rotate_quant(n, group, scale_mode):
    hr = _hr()
    rows = 301
    x, d = _bf16_rows(rows, n, seed=200 + n + group)
    sd = torch.float16 if scale_mode == "f16" else torch.float32
    codes, scales = hr.rotate_quant_int4(x.to(DEV), group, torch.from_numpy(d).to(DEV),
                                         scale_dtype=sd)
    y64 = oracle.hadamard.rht(x.float().numpy(), d)
    check_quant(codes.cpu().numpy(), scales.cpu().numpy(), y64, group, scale_mode)


@pytest.mark.parametrize("group,scale_mode,bits", [(128, "f16", 4), (32, "f32", 4), (64, "f16", 4),
                                                  (256, "f32", 4), (128, "f16", 8), (32, "f32", 8)])
def test_rotate_quant_4096_wave_per_row(group, scale_mode, bits):
    """n = 4096 with enough rows for the one-wave-per-row kernel (two
    2048-point chunks per wave, H_2 across them); some waves take two rows."""
    hr = _hr()
    rows, n = 2100, 4096
    x, d = _bf16_rows(rows, n, seed=4096 + group + bits)
    sd = torch.float16 if scale_mode == "f16" else torch.float32
    fn = hr.rotate_quant_int4 if bits == 4 else hr.rotate_quant_int8
    codes, scales = fn(x.to(DEV), group, torch.from_numpy(d).to(DEV), scale_dtype=sd)
    sample = np.unique(np.concatenate([np.random.default_rng(group).choice(rows, 40, replace=False),
                                       [0, 2047, 2048, rows - 1]]))
    y64 = oracle.hadamard.rht(x[sample].float().numpy(), d)
    check_quant(codes.cpu().numpy()[sample], scales.cpu().numpy()[sample], y64, group, scale_mode, bits)


def test_rotate_4096_wave_per_row_fp32_out():
    hr = _hr()
    rows, n = 2100, 4096
    x, d = _bf16_rows(rows, n, seed=4097)
    y = hr.rotate(x.to(DEV), torch.from_numpy(d).to(DEV)).cpu().numpy()
    sample = np.unique(np.concatenate([np.random.default_rng(5).choice(rows, 40, replace=False),
                                       [0, 2047, 2048, rows - 1]]))
    check_rotated(y[sample], oracle.hadamard.rht(x[sample].float().numpy(), d))


def test_rotate_quant_fp32_input_and_zero_rows():
    hr = _hr()
    n, group = 2048, 128
    x = np.random.default_rng(9).standard_normal((70, n)).astype(np.float32)
    x[3] = 0.0                         # an all-zero row: codes 0, scales 0
    x[4, :] = 1e-30                    # tiny values: fp16 scale underflows to 0
    d = hr_inputs.sign_vector(np.random.default_rng(10), n)
    codes, scales = hr.rotate_quant_int4(torch.from_numpy(x).to(DEV), group,
                                         torch.from_numpy(d).to(DEV))
    codes, scales = codes.cpu().numpy(), scales.cpu().numpy()
    assert np.all(codes[3] == 0) and np.all(scales[3] == 0)
    assert np.all(codes[4] == 0) and np.all(scales[4] == 0)
    check_quant(codes, scales, oracle.hadamard.rht(x, d), group, "f16")


def test_rotate_quant_large_dynamic_range():
    """Rows spanning many binades, including fp16-subnormal scales."""
    hr = _hr()
    n, group = 2048, 32
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((64, n)) * np.exp2(rng.integers(-30, 10, size=(64, 1)))).astype(np.float32)
    d = hr_inputs.sign_vector(rng, n)
    codes, scales = hr.rotate_quant_int4(torch.from_numpy(x).to(DEV), group,
                                         torch.from_numpy(d).to(DEV))
    check_quant(codes.cpu().numpy(), scales.cpu().numpy(), oracle.hadamard.rht(x, d), group, "f16")


@pytest.mark.parametrize("group", [32, 128, 256])
def test_rotate_quant_large_dynamic_range_bf16(group):
    """bf16 rows spanning many binades (matrix-core path), zero and tiny rows."""
    hr = _hr()
    n = 2048
    rng = np.random.default_rng(13 + group)
    x = (rng.standard_normal((67, n)) * np.exp2(rng.integers(-30, 10, size=(67, 1)))).astype(np.float32)
    x[7] = 0.0
    x[8] = 1e-30
    xb = torch.from_numpy(x).to(torch.bfloat16)
    d = hr_inputs.sign_vector(rng, n)
    codes, scales = hr.rotate_quant_int4(xb.to(DEV), group, torch.from_numpy(d).to(DEV))
    codes, scales = codes.cpu().numpy(), scales.cpu().numpy()
    assert np.all(codes[7] == 0) and np.all(scales[7] == 0)
    assert np.all(codes[8] == 0) and np.all(scales[8] == 0)
    check_quant(codes, scales, oracle.hadamard.rht(xb.float().numpy(), d), group, "f16")


# ---------------------------------------------------------------- mixed radix

@pytest.mark.parametrize("m,p,group", [(7, 2048, 128), (3, 64, 32), (5, 256, 64), (16, 1024, 128),
                                       (2, 2048, 32), (3, 2048, 256), (8, 2048, 64)])
def test_mixed_radix(m, p, group):
    hr = _hr()
    rows = 23
    mi = hr_inputs.mixed_inputs(rows=rows, m=m, p=p, seed=300 + m)
    xd = mi.x.to(DEV)
    dd = torch.from_numpy(mi.signs).to(DEV)
    od = torch.from_numpy(mi.block).to(DEV)
    y64 = oracle.mixed_radix.mixed_radix(mi.x.float().numpy(), mi.signs, mi.block, p)
    y = hr.rotate(xd, dd, od).cpu().numpy()
    check_rotated(y, y64)
    codes, scales = hr.rotate_quant_int4(xd, group, dd, od)
    check_quant(codes.cpu().numpy(), scales.cpu().numpy(), y64, group, "f16")


@pytest.mark.parametrize("m,group,with_signs,scale_mode", [(7, 128, True, "f16"), (4, 64, False, "f32"),
                                                          (6, 256, True, "f32"), (5, 32, True, "f32"),
                                                          (8, 128, True, "f16"), (3, 64, True, "f16")])
def test_mixed_radix_many_rows(m, group, with_signs, scale_mode):
    """More rows than resident workgroups (each workgroup loops over rows),
    with and without the sign diagonal, fp16 and fp32 scales."""
    hr = _hr()
    rows, p = 600, 2048
    mi = hr_inputs.mixed_inputs(rows=rows, m=m, p=p, seed=350 + m)
    signs = mi.signs if with_signs else np.ones_like(mi.signs)
    xd = mi.x.to(DEV)
    dd = torch.from_numpy(mi.signs).to(DEV) if with_signs else None
    od = torch.from_numpy(mi.block).to(DEV)
    y64 = oracle.mixed_radix.mixed_radix(mi.x.float().numpy(), signs, mi.block, p)
    check_rotated(hr.rotate(xd, dd, od).cpu().numpy(), y64)
    sd = torch.float16 if scale_mode == "f16" else torch.float32
    codes, scales = hr.rotate_quant_int4(xd, group, dd, od, scale_dtype=sd)
    check_quant(codes.cpu().numpy(), scales.cpu().numpy(), y64, group, scale_mode)


@pytest.mark.parametrize("m,scale_mode", [(2, "f16"), (3, "f32"), (7, "f16"), (7, "f32")])
def test_mixed_radix_rows_per_wave(m, scale_mode):
    """G = 128 codes with a dense block over 2125 rows: every workgroup of the
    persistent grid takes four or five rows in turn, and the last round is
    partial.  Sampled rows from every round against the oracle."""
    hr = _hr()
    rows, p = 2125, 2048
    mi = hr_inputs.mixed_inputs(rows=rows, m=m, p=p, seed=360 + m)
    xd = mi.x.to(DEV)
    dd = torch.from_numpy(mi.signs).to(DEV)
    od = torch.from_numpy(mi.block).to(DEV)
    sd = torch.float16 if scale_mode == "f16" else torch.float32
    codes, scales = hr.rotate_quant_int4(xd, 128, dd, od, scale_dtype=sd)
    rng = np.random.default_rng(m)
    sample = np.unique(np.concatenate([rng.choice(rows, 24, replace=False),
                                       [0, 1, 1023, 1024, 1025, 2047, 2048, 2049, rows - 1]]))
    y64 = oracle.mixed_radix.mixed_radix(mi.x[sample].float().numpy(), mi.signs, mi.block, p)
    check_quant(codes.cpu().numpy()[sample], scales.cpu().numpy()[sample], y64, 128, scale_mode)


@pytest.mark.parametrize("group", [32, 64, 128, 256])
@pytest.mark.parametrize("m", [2, 3, 4, 5, 6, 7, 8])
def test_mixed_radix_grid(m, group):
    """Every block size of the bf16 matrix-core kernel against every group
    size: the waves split the m output chunks into halves of (m + 1) // 2 and
    m // 2, and the group absmax takes 2 to 5 lane-reduction steps."""
    hr = _hr()
    rows, p = 5, 2048
    mi = hr_inputs.mixed_inputs(rows=rows, m=m, p=p, seed=700 + 10 * m + group)
    xd = mi.x.to(DEV)
    dd = torch.from_numpy(mi.signs).to(DEV)
    od = torch.from_numpy(mi.block).to(DEV)
    y64 = oracle.mixed_radix.mixed_radix(mi.x.float().numpy(), mi.signs, mi.block, p)
    codes, scales = hr.rotate_quant_int4(xd, group, dd, od)
    check_quant(codes.cpu().numpy(), scales.cpu().numpy(), y64, group, "f16")
    if group == 128:
        check_rotated(hr.rotate(xd, dd, od).cpu().numpy(), y64)


@pytest.mark.parametrize("group", [32, 64, 128, 256])
@pytest.mark.parametrize("n", [4096, 8192, 16384])
def test_sylvester_chunks_grid(n, group):
    """n = 4096 (few rows), 8192 and 16384 as H_{n/2048} kron H_2048 in the
    mixed-radix kernel (each wave's half of the outputs by one +- stage, then
    add/sub stages), every group size."""
    hr = _hr()
    rows = 7
    x, d = _bf16_rows(rows, n, seed=900 + n // 1024 + group)
    dd = torch.from_numpy(d).to(DEV)
    y64 = oracle.hadamard.rht(x.float().numpy(), d)
    codes, scales = hr.rotate_quant_int4(x.to(DEV), group, dd)
    check_quant(codes.cpu().numpy(), scales.cpu().numpy(), y64, group, "f16")
    if group == 128:
        check_rotated(hr.rotate(x.to(DEV), dd).cpu().numpy(), y64)


def test_mixed_radix_fp32_input_fp32_scales():
    hr = _hr()
    m, p, group = 5, 2048, 128
    mi = hr_inputs.mixed_inputs(rows=17, m=m, p=p, seed=333)
    x = mi.x.float()
    xd = x.to(DEV)
    dd = torch.from_numpy(mi.signs).to(DEV)
    od = torch.from_numpy(mi.block).to(DEV)
    y64 = oracle.mixed_radix.mixed_radix(x.numpy(), mi.signs, mi.block, p)
    check_rotated(hr.rotate(xd, dd, od).cpu().numpy(), y64)
    codes, scales = hr.rotate_quant_int4(xd, group, dd, od, scale_dtype=torch.float32)
    check_quant(codes.cpu().numpy(), scales.cpu().numpy(), y64, group, "f32")


# ---------------------------------------------------------------- butterfly

@pytest.mark.parametrize("n", [64, 1024, 4096, 8192])
@pytest.mark.parametrize("precondition", [False, True])
def test_butterfly_forward_inverse(n, precondition):
    hr = _hr()
    bi = hr_inputs.butterfly_inputs(rows=29, n=n, seed=400 + n)
    xd = torch.from_numpy(bi.x).to(DEV)
    co = hr.butterfly_coeffs(torch.from_numpy(bi.angles).to(DEV), precondition)
    pd = torch.from_numpy(bi.perm).to(DEV)
    y = hr.butterfly_apply(xd, co, precondition, pd)
    y64 = oracle.butterfly.butterfly(bi.x, bi.angles, bi.perm, precondition)
    check_rotated(y.cpu().numpy(), y64)
    # norm preservation and inverse round trip on the GPU
    yn = np.linalg.norm(y.cpu().numpy().astype(np.float64), axis=1)
    np.testing.assert_allclose(yn, np.linalg.norm(bi.x.astype(np.float64), axis=1), rtol=1e-5)
    back = hr.butterfly_apply(y, co, precondition, pd, inverse=True).cpu().numpy()
    check_rotated(back, bi.x.astype(np.float64))
    inv64 = oracle.butterfly.butterfly(bi.x, bi.angles, bi.perm, precondition, inverse=True)
    check_rotated(hr.butterfly_apply(xd, co, precondition, pd, inverse=True).cpu().numpy(), inv64)


def test_butterfly_zero_angles_is_hadamard():
    hr = _hr()
    n = 4096
    x = np.random.default_rng(3).standard_normal((9, n)).astype(np.float32)
    ang = torch.zeros((12, n // 2), dtype=torch.float32, device=DEV)
    co = hr.butterfly_coeffs(ang, True)
    y = hr.butterfly_apply(torch.from_numpy(x).to(DEV), co, True, None).cpu().numpy()
    check_rotated(y, oracle.hadamard.rht(x, None))


@pytest.mark.parametrize("group,scale_mode", [(64, "f16"), (128, "f32")])
def test_butterfly_quant(group, scale_mode):
    hr = _hr()
    bi = hr_inputs.butterfly_inputs(rows=33, n=4096, seed=450)
    co = hr.butterfly_coeffs(torch.from_numpy(bi.angles).to(DEV), False)
    sd = torch.float16 if scale_mode == "f16" else torch.float32
    y, codes, scales = hr.butterfly_apply(torch.from_numpy(bi.x).to(DEV), co, False,
                                          torch.from_numpy(bi.perm).to(DEV), group=group,
                                          scale_dtype=sd)
    y64 = oracle.butterfly.butterfly(bi.x, bi.angles, bi.perm)
    check_rotated(y.cpu().numpy(), y64)
    check_quant(codes.cpu().numpy(), scales.cpu().numpy(), y64, group, scale_mode)


@pytest.mark.parametrize("precondition", [False, True])
def test_butterfly_4096_many_rows_identity_perm(precondition):
    """About five rows per workgroup (the input ring wraps and reaches its
    steady-state waits), no permutation (the vector gather and scatter), and
    both outputs at once; sampled rows against the oracle."""
    hr = _hr()
    rows, n = 1300, 4096
    bi = hr_inputs.butterfly_inputs(rows=rows, n=n, seed=460 + int(precondition))
    co = hr.butterfly_coeffs(torch.from_numpy(bi.angles).to(DEV), precondition)
    xd = torch.from_numpy(bi.x).to(DEV)
    y, codes, scales = hr.butterfly_apply(xd, co, precondition, None, group=64)
    yi = hr.butterfly_apply(xd, co, precondition, None, inverse=True)
    sample = np.unique(np.concatenate([np.random.default_rng(5).choice(rows, 40, replace=False),
                                       [0, 255, 256, 767, 768, rows - 1]]))
    xs = bi.x[sample]
    y64 = oracle.butterfly.butterfly(xs, bi.angles, None, precondition)
    check_rotated(y.cpu().numpy()[sample], y64)
    check_quant(codes.cpu().numpy()[sample], scales.cpu().numpy()[sample], y64, 64, "f16")
    inv64 = oracle.butterfly.butterfly(xs, bi.angles, None, precondition, inverse=True)
    check_rotated(yi.cpu().numpy()[sample], inv64)


# ---------------------------------------------------------------- dequant

@pytest.mark.parametrize("group,scale_mode", [(32, "f16"), (128, "f16"), (256, "f32")])
def test_dequant_bit_exact(group, scale_mode):
    hr = _hr()
    rows, n = 55, 2048
    rng = np.random.default_rng(group)
    q = rng.integers(-7, 8, size=(rows, n)).astype(np.int8)
    sd = np.float16 if scale_mode == "f16" else np.float32
    s = rng.uniform(0.001, 0.05, size=(rows, n // group)).astype(sd)
    packed = oracle.quant.pack_int4(q)
    out = hr.dequant_int4(torch.from_numpy(packed).to(DEV), torch.from_numpy(s).to(DEV), group)
    ref = oracle.quant.dequant(q, s, group)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


# ---------------------------------------------------------------- GEMM

@pytest.mark.parametrize("M,N,K,group", [(16, 256, 512, 128), (100, 128, 1024, 128),
                                         (256, 192, 4096, 128), (5, 64, 256, 64),
                                         (130, 64, 512, 256), (64, 128, 768, 128)])
def test_gemm(M, N, K, group):
    hr = _hr()
    gi = hr_inputs.gemm_inputs(M=M, N=N, K=K, group=group, seed=500 + M)
    t = lambda a: torch.from_numpy(a).to(DEV)  # noqa: E731
    c, acc = hr.w4a4_gemm(t(gi.a_codes), t(gi.a_scales), t(gi.w_codes), t(gi.w_scales), group,
                          group_acc=True)
    c_ref, acc_ref, bound = oracle.gemm.w4a4_gemm(gi.a_codes, gi.a_scales, gi.w_codes, gi.w_scales,
                                                  group, return_sums=True)
    check_gemm(c.cpu().numpy(), c_ref, bound, acc.cpu().numpy(), acc_ref)
    c2 = hr.w4a4_gemm(t(gi.a_codes), t(gi.a_scales), t(gi.w_codes), t(gi.w_scales), group)
    assert torch.equal(c2, c)


@pytest.mark.parametrize("M,N,K,group,scale_mode", [
    (130, 256, 1024, 128, "f16"),    # two tiles of 128 x 256, ragged M
    (300, 512, 768, 128, "f16"),     # ragged M over three tile rows
    (257, 256, 512, 64, "f16"),      # 64-code stages
    (200, 512, 1024, 256, "f16"),    # two stages per group
    (1024, 2048, 512, 128, "f16"),   # 64 tiles: tile ranges per XCD
    (1100, 1024, 256, 128, "f16"),   # 9 tile rows: a partial group of tile rows
    (160, 256, 512, 128, "f32"),     # fp32 scales
    (140, 512, 768, 64, "f32"),
])
def test_gemm_wide_tiles(M, N, K, group, scale_mode):
    """N a multiple of 256 and M > 16: the 128 x 256 tile kernel."""
    hr = _hr()
    gi = hr_inputs.gemm_inputs(M=M, N=N, K=K, group=group, seed=700 + M)
    sd = np.float16 if scale_mode == "f16" else np.float32
    sa, sw = gi.a_scales.astype(sd), gi.w_scales.astype(sd)
    t = lambda a: torch.from_numpy(a).to(DEV)  # noqa: E731
    c, acc = hr.w4a4_gemm(t(gi.a_codes), t(sa), t(gi.w_codes), t(sw), group, group_acc=True)
    c_ref, acc_ref, bound = oracle.gemm.w4a4_gemm(gi.a_codes, sa, gi.w_codes, sw, group,
                                                  return_sums=True)
    check_gemm(c.cpu().numpy(), c_ref, bound, acc.cpu().numpy(), acc_ref)
    c2 = hr.w4a4_gemm(t(gi.a_codes), t(sa), t(gi.w_codes), t(sw), group)
    assert torch.equal(c2, c)


@pytest.mark.parametrize("M,N,K,group,scale_mode", [
    (1, 64, 256, 256, "f16"),       # one group: a single wave of eight has work
    (16, 128, 768, 256, "f16"),     # three groups over eight waves
    (12, 128, 2560, 128, "f16"),    # 20 groups: two or three per wave
    (7, 192, 4096, 64, "f32"),      # eight 32-byte runs per wave, fp32 scales
    (16, 64, 16384, 64, "f16"),     # 32 groups per wave: four load chunks
    (3, 256, 1536, 256, "f32"),     # two loads per group
])
def test_gemm_decode_shapes(M, N, K, group, scale_mode):
    """M <= 16: the decode kernel over group counts that do not divide evenly."""
    hr = _hr()
    gi = hr_inputs.gemm_inputs(M=M, N=N, K=K, group=group, seed=900 + K + M)
    sd = np.float16 if scale_mode == "f16" else np.float32
    sa, sw = gi.a_scales.astype(sd), gi.w_scales.astype(sd)
    t = lambda a: torch.from_numpy(a).to(DEV)  # noqa: E731
    c, acc = hr.w4a4_gemm(t(gi.a_codes), t(sa), t(gi.w_codes), t(sw), group, group_acc=True)
    c_ref, acc_ref, bound = oracle.gemm.w4a4_gemm(gi.a_codes, sa, gi.w_codes, sw, group,
                                                  return_sums=True)
    check_gemm(c.cpu().numpy(), c_ref, bound, acc.cpu().numpy(), acc_ref)
    c2 = hr.w4a4_gemm(t(gi.a_codes), t(sa), t(gi.w_codes), t(sw), group)
    assert torch.equal(c2, c)


@pytest.mark.parametrize("M,N,group", [(3, 64, 256), (17, 128, 128), (40, 192, 64)])
def test_gemm_max_k(M, N, group):
    """K = 65536, the largest the library accepts: decode, prefill and simple kernels."""
    hr = _hr()
    K = 65536
    gi = hr_inputs.gemm_inputs(M=M, N=N, K=K, group=group, seed=1200 + M)
    t = lambda a: torch.from_numpy(a).to(DEV)  # noqa: E731
    c, acc = hr.w4a4_gemm(t(gi.a_codes), t(gi.a_scales), t(gi.w_codes), t(gi.w_scales), group,
                          group_acc=True)
    c_ref, acc_ref, bound = oracle.gemm.w4a4_gemm(gi.a_codes, gi.a_scales, gi.w_codes, gi.w_scales,
                                                  group, return_sums=True)
    check_gemm(c.cpu().numpy(), c_ref, bound, acc.cpu().numpy(), acc_ref)


def test_gemm_fp32_scales_and_minus_eight():
    hr = _hr()
    M, N, K, group = 33, 128, 512, 128
    rng = np.random.default_rng(77)
    a = rng.integers(-8, 8, size=(M, K)).astype(np.int8)
    w = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
    sa = rng.uniform(0.001, 0.05, size=(M, K // group)).astype(np.float32)
    sw = rng.uniform(0.001, 0.05, size=(N, K // group)).astype(np.float32)
    ap, wp = oracle.quant.pack_int4(a), oracle.quant.pack_int4(w)
    t = lambda v: torch.from_numpy(v).to(DEV)  # noqa: E731
    c, acc = hr.w4a4_gemm(t(ap), t(sa), t(wp), t(sw), group, group_acc=True)
    c_ref, acc_ref, bound = oracle.gemm.w4a4_gemm(ap, sa, wp, sw, group, return_sums=True)
    check_gemm(c.cpu().numpy(), c_ref, bound, acc.cpu().numpy(), acc_ref)


def test_pipeline_rotate_quant_then_gemm():
    """Quantized rotated activations and weights feed the GEMM; the result
    approximates the unrotated product (rotation is exact before quantizing)."""
    hr = _hr()
    M, N, K, group = 64, 128, 2048, 128
    rng = np.random.default_rng(8)
    a = rng.standard_normal((M, K)).astype(np.float32)
    a[:, rng.choice(K, 4, replace=False)] *= 20
    w = rng.standard_normal((N, K)).astype(np.float32)
    d = hr_inputs.sign_vector(rng, K)
    dd = torch.from_numpy(d).to(DEV)
    ac, as_ = hr.rotate_quant_int4(torch.from_numpy(a).to(DEV), group, dd)
    wc, ws = hr.rotate_quant_int4(torch.from_numpy(w).to(DEV), group, dd)
    c = hr.w4a4_gemm(ac, as_, wc, ws, group).cpu().numpy()
    c_ref, _, bound = oracle.gemm.w4a4_gemm(ac.cpu().numpy(), as_.cpu().numpy(), wc.cpu().numpy(),
                                            ws.cpu().numpy(), group, return_sums=True)
    check_gemm(c, c_ref, bound)
    exact = a.astype(np.float64) @ w.astype(np.float64).T
    rel = np.linalg.norm(c - exact) / np.linalg.norm(exact)
    assert rel < 0.25
