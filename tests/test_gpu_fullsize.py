"""GPU parity at the full workload sizes, in the launch configuration the
bench times (the same entry points on the full arrays).  The oracle computes
a seeded sample of rows (plus the first and last row) one by one."""
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


def _sample(rows, k, seed=0):
    idx = np.random.default_rng(seed).choice(rows, size=k, replace=False)
    return np.unique(np.concatenate([idx, [0, rows - 1]]))


@pytest.fixture(scope="module")
def rht_full():
    inp = hr_inputs.rht_inputs()          # bf16 65536 x 2048, x50 outliers, seed 2
    return inp, inp.x.to(DEV), torch.from_numpy(inp.signs).to(DEV)


@pytest.mark.parametrize("group", [128, 32])
def test_rotate_quant_65536x2048(rht_full, group):
    hr = _hr()
    inp, xd, dd = rht_full
    codes, scales = hr.rotate_quant_int4(xd, group, dd)
    rows = _sample(inp.rows, 256, seed=group)
    y64 = oracle.hadamard.rht(inp.x[rows].float().numpy(), inp.signs)
    check_quant(codes.cpu().numpy()[rows], scales.cpu().numpy()[rows], y64, group, "f16")


def test_rotate_65536x2048_fp32_out(rht_full):
    hr = _hr()
    inp, xd, dd = rht_full
    y = hr.rotate(xd, dd)
    rows = _sample(inp.rows, 256, seed=7)
    y64 = oracle.hadamard.rht(inp.x[rows].float().numpy(), inp.signs)
    check_rotated(y[torch.from_numpy(rows).to(DEV)].cpu().numpy(), y64)
    del y


def test_mixed_radix_16384x14336():
    hr = _hr()
    mi = hr_inputs.mixed_inputs()         # bf16 16384 x (7*2048), seed 3
    xd = mi.x.to(DEV)
    dd = torch.from_numpy(mi.signs).to(DEV)
    od = torch.from_numpy(mi.block).to(DEV)
    codes, scales = hr.rotate_quant_int4(xd, 128, dd, od)
    rows = _sample(mi.rows, 48, seed=3)
    y64 = oracle.mixed_radix.mixed_radix(mi.x[rows].float().numpy(), mi.signs, mi.block, mi.p)
    check_quant(codes.cpu().numpy()[rows], scales.cpu().numpy()[rows], y64, 128, "f16")
    y = hr.rotate(xd, dd, od)
    check_rotated(y[torch.from_numpy(rows).to(DEV)].cpu().numpy(), y64)


def test_butterfly_32768x4096():
    hr = _hr()
    bi = hr_inputs.butterfly_inputs()     # fp32 32768 x 4096, seed 4
    xd = torch.from_numpy(bi.x).to(DEV)
    co = hr.butterfly_coeffs(torch.from_numpy(bi.angles).to(DEV), False)
    pd = torch.from_numpy(bi.perm).to(DEV)
    y, codes, scales = hr.butterfly_apply(xd, co, False, pd, group=64)
    rows = _sample(bi.rows, 96, seed=4)
    rd = torch.from_numpy(rows).to(DEV)
    y64 = oracle.butterfly.butterfly(bi.x[rows], bi.angles, bi.perm)
    check_rotated(y[rd].cpu().numpy(), y64)
    check_quant(codes.cpu().numpy()[rows], scales.cpu().numpy()[rows], y64, 64, "f16")
    # orthogonality and inverse round trip at full size
    yn = torch.linalg.vector_norm(y.double(), dim=1)
    xn = torch.linalg.vector_norm(xd.double(), dim=1)
    assert torch.allclose(yn, xn, rtol=1e-5)
    back = hr.butterfly_apply(y, co, False, pd, inverse=True)
    check_rotated(back[rd].cpu().numpy(), bi.x[rows].astype(np.float64))


def test_butterfly_32768x4096_bench_variants():
    """The two launches the bench times: fp32 output only, and codes only
    (G = 64); they are other kernel instances than the combined call above."""
    hr = _hr()
    bi = hr_inputs.butterfly_inputs()
    xd = torch.from_numpy(bi.x).to(DEV)
    co = hr.butterfly_coeffs(torch.from_numpy(bi.angles).to(DEV), False)
    pd = torch.from_numpy(bi.perm).to(DEV)
    rows = _sample(bi.rows, 64, seed=44)
    rd = torch.from_numpy(rows).to(DEV)
    y64 = oracle.butterfly.butterfly(bi.x[rows], bi.angles, bi.perm)
    y = hr.butterfly_apply(xd, co, False, pd)
    check_rotated(y[rd].cpu().numpy(), y64)
    del y
    none, codes, scales = hr.butterfly_apply(xd, co, False, pd, want_y=False, group=64)
    assert none is None
    check_quant(codes.cpu().numpy()[rows], scales.cpu().numpy()[rows], y64, 64, "f16")


def test_dequant_65536x2048(rht_full):
    """Dequantization of the headline codes at full size (grid-stride loop
    over 33.5 M quads), bit-exact on sampled rows."""
    hr = _hr()
    inp, xd, dd = rht_full
    codes, scales = hr.rotate_quant_int4(xd, 128, dd)
    out = hr.dequant_int4(codes, scales, 128)
    rows = _sample(inp.rows, 256, seed=12)
    q = oracle.quant.unpack_int4(codes.cpu().numpy()[rows])
    ref = oracle.quant.dequant(q, scales.cpu().numpy()[rows], 128)
    assert np.array_equal(out.cpu().numpy()[rows].view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("M", [4096, 16])
def test_gemm_4096(M):
    hr = _hr()
    gi = hr_inputs.gemm_inputs(M=M)
    t = lambda a: torch.from_numpy(a).to(DEV)  # noqa: E731
    ad, sad, wd, swd = t(gi.a_codes), t(gi.a_scales), t(gi.w_codes), t(gi.w_scales)
    c = hr.w4a4_gemm(ad, sad, wd, swd, 128)
    rows = _sample(M, min(M, 24), seed=M) if M > 16 else np.arange(M)
    c_ref, acc_ref, bound = oracle.gemm.w4a4_gemm(gi.a_codes, gi.a_scales, gi.w_codes, gi.w_scales,
                                                  128, rows=rows, return_sums=True)
    check_gemm(c.cpu().numpy()[rows], c_ref, bound)
    c2, acc = hr.w4a4_gemm(ad, sad, wd, swd, 128, group_acc=True)
    assert torch.equal(c2, c)
    rd = torch.from_numpy(rows).to(DEV)
    check_gemm(c.cpu().numpy()[rows], c_ref, bound, acc[rd].cpu().numpy(), acc_ref)
