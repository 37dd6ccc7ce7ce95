"""GPU parity of HARP's general mixed-radix processor (hr_harp_blocks,
hr_harp_apply) against the oracle (oracle/harp.py), through the C ABI."""
import numpy as np
import pytest
import torch

import hr_inputs
import oracle
from parity import check_quant, check_rotated

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
H = oracle.harp


def _hr():
    import hadamard_rotation_int4_amd as hr
    return hr


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _gpu_blocks(hi):
    hr = _hr()
    fb = _t(np.concatenate([f.ravel() for f in hi.fallbacks])) if hi.fallbacks else None
    return hr.harp_blocks(hi.radices, _t(hi.theta), fb)


def _split(flat, radices):
    """The library's quad-major table ([ceil(b^2/4)][d/b][4] per stage, the
    last quad zero-padded) as the oracle's per-block list ([d/b][b][b] per
    stage); the padding is checked to be zero."""
    d = int(np.prod(radices))
    assert flat.size == _hr().harp_table_size(radices)
    out, off = [], 0
    for b in radices:
        k4 = (b * b + 3) // 4
        stage = flat[off:off + 4 * k4 * (d // b)].reshape(k4, d // b, 4).transpose(1, 0, 2).reshape(d // b, 4 * k4)
        assert not stage[:, b * b:].any()
        out.append(stage[:, :b * b].reshape(d // b, b, b))
        off += 4 * k4 * (d // b)
    return out


SCHEDULES = [(8, 8, 8, 5, 2), (4, 5, 3, 2), (2,) * 6, (7, 4, 2), (6, 4), (3, 3, 4), (8, 8, 8, 8),
             (2, 2)]


def _oracle_blocks(hi):
    """The oracle's own blocks from theta (fp64 throughout)."""
    return H.blocks(hi.radices, hi.theta, hi.fallbacks)


def _oracle_blocks_stored(hi):
    """The oracle's blocks rounded once to fp32: what hr_harp_blocks documents
    it stores (each block formed in double precision, stored as fp32)."""
    return [b.astype(np.float32).astype(np.float64) for b in _oracle_blocks(hi)]


@pytest.mark.parametrize("radices", SCHEDULES)
def test_harp_blocks(radices):
    hi = hr_inputs.harp_inputs(rows=1, radices=radices, seed=60 + len(radices))
    got = np.concatenate([b.ravel() for b in _split(_gpu_blocks(hi).cpu().numpy(), radices)])
    got = got.astype(np.float64)
    ref = np.concatenate([b.ravel() for b in H.blocks(hi.radices, hi.theta, hi.fallbacks)])
    # double-precision construction rounded once to fp32: within one fp32 ulp
    np.testing.assert_allclose(got, ref, rtol=1.2e-7, atol=1e-9)


@pytest.mark.parametrize("radices,rows", [((8, 8, 8, 5, 2), 301), ((4, 5, 3, 2), 97), ((2,) * 6, 64),
                                          ((7, 4, 2), 33), ((8, 8, 8, 8), 21), ((2, 2), 9),
                                          ((3, 3, 4), 50)])
def test_harp_apply_forward_inverse(radices, rows):
    hr = _hr()
    hi = hr_inputs.harp_inputs(rows=rows, radices=radices, seed=70 + rows)
    blk = _gpu_blocks(hi)
    stage_blocks = _split(blk.cpu().numpy(), hi.radices)
    y = hr.harp_apply(_t(hi.x), hi.radices, blk)
    check_rotated(y.cpu().numpy(), H.apply(hi.x, hi.radices, stage_blocks))
    yi = hr.harp_apply(_t(hi.x), hi.radices, blk, inverse=True)
    check_rotated(yi.cpu().numpy(), H.apply(hi.x, hi.radices, stage_blocks, inverse=True))


@pytest.mark.parametrize("group,scale_mode", [(128, "f16"), (32, "f32"), (256, "f16")])
def test_harp_apply_quant(group, scale_mode):
    hr = _hr()
    hi = hr_inputs.harp_inputs(rows=130, seed=80 + group)
    blk = _gpu_blocks(hi)
    sd = torch.float16 if scale_mode == "f16" else torch.float32
    y, codes, scales = hr.harp_apply(_t(hi.x), hi.radices, blk, group=group, scale_dtype=sd)
    y64 = H.apply(hi.x, hi.radices, _split(blk.cpu().numpy(), hi.radices))
    check_rotated(y.cpu().numpy(), y64)
    check_quant(codes.cpu().numpy(), scales.cpu().numpy(), y64, group, scale_mode)
    _, c2, s2 = hr.harp_apply(_t(hi.x), hi.radices, blk, want_y=False, group=group, scale_dtype=sd)
    assert torch.equal(c2, codes) and torch.equal(s2, scales)


@pytest.mark.parametrize("group", [128, 32])
def test_harp_quant_tiny_fp32_scales(group):
    """Rows scaled by 2^-120: every fp32 group scale is below 2^-100, where
    its reciprocal would overflow; the quantizer takes values and scale
    x 2^64 (exact) and the codes still match the oracle's."""
    hr = _hr()
    hi = hr_inputs.harp_inputs(rows=9, seed=84 + group)
    x = (hi.x.astype(np.float64) * 2.0 ** -120).astype(np.float32)
    blk = _gpu_blocks(hi)
    _, codes, scales = hr.harp_apply(_t(x), hi.radices, blk, want_y=False, group=group,
                                     scale_dtype=torch.float32)
    y64 = H.apply(x.astype(np.float64), hi.radices, _split(blk.cpu().numpy(), hi.radices))
    s = scales.cpu().numpy()
    assert np.all(s < 2.0 ** -100) and np.all(s > 0)
    check_quant(codes.cpu().numpy(), s, y64, group, "f32")


def test_harp_zero_theta_is_hadamard():
    hr = _hr()
    radices = (4, 8, 2, 8)
    d = 512
    th = np.zeros(sum((d // b) * H.n_params(b) for b in radices), dtype=np.float32)
    blk = hr.harp_blocks(radices, _t(th))
    x = np.random.default_rng(81).standard_normal((40, d)).astype(np.float32)
    y = hr.harp_apply(_t(x), radices, blk)
    check_rotated(y.cpu().numpy(), oracle.hadamard.rht(x))


def test_harp_radix_two_matches_butterfly_kernel():
    hr = _hr()
    bi = hr_inputs.butterfly_inputs(rows=37, n=1024, seed=82)
    blk = hr.harp_blocks((2,) * 10, _t(bi.angles.ravel()))
    y = hr.harp_apply(_t(bi.x), (2,) * 10, blk).cpu().numpy()
    ref = oracle.butterfly.butterfly(bi.x, bi.angles, None, precondition=True)
    check_rotated(y, ref)
    co = hr.butterfly_coeffs(_t(bi.angles), precondition=True)
    yb = hr.butterfly_apply(_t(bi.x), co, precondition=True).cpu().numpy()
    assert np.abs(y - yb).max() <= 2e-5 * np.abs(ref).max()


def test_harp_round_trip_in_place_and_zero_rows():
    hr = _hr()
    hi = hr_inputs.harp_inputs(rows=64, seed=83)
    blk = _gpu_blocks(hi)
    xd = _t(hi.x)
    y = hr.harp_apply(xd, hi.radices, blk)
    back = hr.harp_apply(y, hi.radices, blk, inverse=True, out=y)      # in place
    assert back.data_ptr() == y.data_ptr()
    err = np.abs(back.cpu().numpy() - hi.x).max()
    assert err <= 2e-5 * np.abs(hi.x).max(), err
    z = hr.harp_apply(torch.empty((0, hi.d), dtype=torch.float32, device=DEV), hi.radices, blk)
    assert z.shape == (0, hi.d)


def test_harp_4096x5120_sampled():
    """The bench workload: 4096 rows of d = 5120 = (8, 8, 8, 5, 2), G = 128."""
    hr = _hr()
    hi = hr_inputs.harp_inputs()
    blk = _gpu_blocks(hi)
    y, codes, scales = hr.harp_apply(_t(hi.x), hi.radices, blk, group=128)
    rows = np.unique(np.concatenate([np.random.default_rng(84).choice(hi.rows, 64, replace=False),
                                     [0, hi.rows - 1]]))
    y64 = H.apply(hi.x[rows], hi.radices, _split(blk.cpu().numpy(), hi.radices))
    ri = torch.from_numpy(rows).to(DEV)
    check_rotated(y[ri].cpu().numpy(), y64)
    check_quant(codes[ri].cpu().numpy(), scales[ri].cpu().numpy(), y64, 128, "f16")
    # the codes-only call the bench times computes the same codes and scales
    none, codes2, scales2 = hr.harp_apply(_t(hi.x), hi.radices, blk, want_y=False, group=128)
    assert none is None
    assert torch.equal(codes2, codes) and torch.equal(scales2, scales)


# ---- end to end from theta: the GPU's block table and application against
# the oracle's own blocks (no GPU data enters the reference)

@pytest.mark.parametrize("radices,rows", [((8, 8, 8, 5, 2), 131), ((4, 5, 3, 2), 97), ((2,) * 6, 64),
                                          ((7, 4, 2), 33), ((6, 4), 40), ((3, 3, 4), 50),
                                          ((8, 8, 8, 8), 21), ((2, 2), 9),
                                          ((8, 8, 8, 8, 4), 5)])   # d = 16384: 2 rows a group, one ragged
def test_harp_theta_to_output(radices, rows):
    """Forward and inverse output from theta, against the oracle's fp64 blocks
    at 2e-5 x row max; the oracle's fp32-stored blocks at the same bound."""
    hr = _hr()
    hi = hr_inputs.harp_inputs(rows=rows, radices=radices, seed=90 + rows)
    blk = _gpu_blocks(hi)
    y = hr.harp_apply(_t(hi.x), hi.radices, blk).cpu().numpy()
    yi = hr.harp_apply(_t(hi.x), hi.radices, blk, inverse=True).cpu().numpy()
    for ob in (_oracle_blocks(hi), _oracle_blocks_stored(hi)):
        check_rotated(y, H.apply(hi.x, hi.radices, ob))
        check_rotated(yi, H.apply(hi.x, hi.radices, ob, inverse=True))


@pytest.mark.parametrize("radices,group,scale_mode", [((8, 8, 8, 5, 2), 128, "f16"),
                                                      ((8, 8, 8, 5, 2), 32, "f32"),
                                                      ((5, 8, 8), 64, "f16"),
                                                      ((3, 8, 8, 2), 128, "f32"),
                                                      ((8, 8, 8, 8), 256, "f16"),
                                                      ((2,) * 6, 64, "f32")])
def test_harp_theta_to_codes(radices, group, scale_mode):
    """Quantized output from theta: rotated values against the oracle's fp64
    blocks; codes and scales against the oracle's quantization of its own
    application of the stored (fp32-rounded) blocks."""
    hr = _hr()
    hi = hr_inputs.harp_inputs(rows=77, radices=radices, seed=95 + group)
    blk = _gpu_blocks(hi)
    sd = torch.float16 if scale_mode == "f16" else torch.float32
    y, codes, scales = hr.harp_apply(_t(hi.x), hi.radices, blk, group=group, scale_dtype=sd)
    check_rotated(y.cpu().numpy(), H.apply(hi.x, hi.radices, _oracle_blocks(hi)))
    y64 = H.apply(hi.x, hi.radices, _oracle_blocks_stored(hi))
    check_rotated(y.cpu().numpy(), y64)
    check_quant(codes.cpu().numpy(), scales.cpu().numpy(), y64, group, scale_mode)


def test_harp_two_sided():
    """HARP's two-sided use (abstract: a two-sided orthogonal processor with
    exact full-precision equivalence): with x' = Q_i x, W' = Q_o W Q_i^T, the
    product W' x' equals Q_o (W x).  Q_i (d_in = 5120, (8, 8, 8, 5, 2)) is
    applied on the GPU to the rows of X and of W, Q_o (d_out = 1152,
    (8, 8, 3, 6)) to the columns of W Q_i^T; the product of the transformed
    operands is checked against the oracle's Q_o applied to X W^T."""
    hr = _hr()
    hi = hr_inputs.harp_inputs(rows=48, radices=(8, 8, 8, 5, 2), seed=97)
    ho = hr_inputs.harp_inputs(rows=1, radices=(8, 8, 3, 6), seed=98)
    W = np.random.default_rng(99).standard_normal((ho.d, hi.d)).astype(np.float32)
    bi, bo = _gpu_blocks(hi), _gpu_blocks(ho)
    xp = hr.harp_apply(_t(hi.x), hi.radices, bi)                       # rows x -> Q_i x
    wqi = hr.harp_apply(_t(W), hi.radices, bi)                          # rows of W Q_i^T
    wp = hr.harp_apply(wqi.t().contiguous(), ho.radices, bo).t()        # Q_o on its columns
    yp = xp.cpu().numpy().astype(np.float64) @ wp.cpu().numpy().astype(np.float64).T
    y_ref = H.apply(hi.x.astype(np.float64) @ W.astype(np.float64).T, ho.radices, _oracle_blocks(ho))
    check_rotated(yp, y_ref)
    # and undoing Q_o on the GPU gives back the original product W x
    back = hr.harp_apply(_t(yp.astype(np.float32)), ho.radices, bo, inverse=True).cpu().numpy()
    check_rotated(back, hi.x.astype(np.float64) @ W.astype(np.float64).T)
