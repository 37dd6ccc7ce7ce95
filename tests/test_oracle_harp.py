"""Pins for the oracle of HARP's general mixed-radix processor (oracle/harp.py)."""
import math

import numpy as np
import pytest
import scipy.linalg

import hr_inputs
import oracle

H = oracle.harp


def _zero_theta(radices):
    d = int(np.prod(radices))
    return np.zeros(sum((d // b) * H.n_params(b) for b in radices))


@pytest.mark.parametrize("radices", [(2,) * 6, (4, 8, 2), (16, 4), (8, 8), (2, 16, 2)])
def test_zero_theta_power_of_two_is_normalised_hadamard(radices):
    """theta = 0 with Sylvester mixers recovers the fixed Hadamard transform H_d / sqrt(d)."""
    d = int(np.prod(radices))
    blk = H.blocks(radices, _zero_theta(radices))
    q = H.matrix(radices, blk)
    np.testing.assert_allclose(q, scipy.linalg.hadamard(d) / math.sqrt(d), atol=1e-14)


def test_shared_blocks_are_a_kronecker_product():
    """Equal blocks within each stage: the processor is B_{m-1} kron ... kron B_0."""
    rng = np.random.default_rng(1)
    radices = (3, 4, 2, 5)
    d = int(np.prod(radices))
    mats = [np.linalg.qr(rng.standard_normal((b, b)))[0] for b in radices]
    blk = [np.repeat(m[None], d // b, axis=0) for m, b in zip(mats, radices)]
    ref = mats[-1]
    for m in reversed(mats[:-1]):
        ref = np.kron(ref, m)
    np.testing.assert_allclose(H.matrix(radices, blk), ref, atol=1e-13)


def test_radix_two_schedule_is_the_butterfly():
    """All radices 2 with Givens factors and the G_2 mixer is the butterfly oracle
    with preconditioning (an independent implementation of the same stages)."""
    bi = hr_inputs.butterfly_inputs(rows=5, n=64, seed=3)
    radices = (2,) * 6
    blk = H.blocks(radices, bi.angles.ravel())
    y = H.apply(bi.x, radices, blk)
    ref = oracle.butterfly.butterfly(bi.x, bi.angles, None, precondition=True)
    np.testing.assert_allclose(y, ref, atol=1e-12)
    yi = H.apply(bi.x, radices, blk, inverse=True)
    refi = oracle.butterfly.butterfly(bi.x, bi.angles, None, precondition=True, inverse=True)
    np.testing.assert_allclose(yi, refi, atol=1e-12)


def test_cayley_three_by_three_closed_form():
    rng = np.random.default_rng(2)
    p = rng.normal(size=3)
    a = np.array([[0, p[0], p[1]], [-p[0], 0, p[2]], [-p[1], -p[2], 0]])
    ref = np.eye(3) + 2 * (a + a @ a) / (1 + np.sum(p * p))
    np.testing.assert_allclose(H.block_q(p, 3), ref, atol=1e-14)


@pytest.mark.parametrize("b", [3, 5, 8, 16])
def test_cayley_properties(b):
    rng = np.random.default_rng(b)
    p = rng.normal(scale=0.7, size=b * (b - 1) // 2)
    q = H.block_q(p, b)
    np.testing.assert_allclose(q.T @ q, np.eye(b), atol=1e-12)
    assert abs(np.linalg.det(q) - 1.0) < 1e-10
    a = (q - np.eye(b)) @ np.linalg.inv(q + np.eye(b))     # the inverse Cayley map
    iu = np.triu_indices(b, k=1)
    np.testing.assert_allclose(a[iu], p, atol=1e-10)
    np.testing.assert_allclose(a, -a.T, atol=1e-10)
    np.testing.assert_allclose(H.block_q(np.zeros_like(p), b), np.eye(b), atol=0)


def test_givens_block():
    q = H.block_q([0.3], 2)
    np.testing.assert_allclose(q, [[math.cos(0.3), -math.sin(0.3)], [math.sin(0.3), math.cos(0.3)]])


def test_hand_indexed_d6():
    """d = 6 = (3, 2): stage 0 blocks {0,1,2}, {3,4,5}; stage 1 blocks {l, l+3}."""
    rng = np.random.default_rng(4)
    b0 = rng.standard_normal((2, 3, 3))
    b1 = rng.standard_normal((3, 2, 2))
    x = rng.standard_normal(6)
    z = x.copy()
    for c, idx in enumerate([[0, 1, 2], [3, 4, 5]]):
        z[idx] = b0[c] @ x[idx]
    y = z.copy()
    for c in range(3):
        idx = [c, c + 3]
        y[idx] = b1[c] @ z[idx]
    np.testing.assert_allclose(H.apply(x[None], (3, 2), [b0, b1])[0], y, atol=1e-14)


def test_mixed_schedule_orthogonal_and_inverse():
    """Orthogonal up to the fp32 rounding of the given QR fallbacks (about 1e-7);
    with the fallbacks made exactly orthogonal in fp64 it is exact."""
    hi = hr_inputs.harp_inputs(rows=3, radices=(4, 5, 3, 2), seed=5)
    blk = H.blocks(hi.radices, hi.theta, hi.fallbacks)
    q = H.matrix(hi.radices, blk)
    np.testing.assert_allclose(q.T @ q, np.eye(hi.d), atol=1e-6)
    y = H.apply(hi.x, hi.radices, blk)
    np.testing.assert_allclose(y, hi.x.astype(np.float64) @ q.T, atol=1e-10)
    exact_fb = [np.linalg.qr(f.astype(np.float64))[0] for f in hi.fallbacks]
    blk64 = H.blocks(hi.radices, hi.theta, exact_fb)
    q64 = H.matrix(hi.radices, blk64)
    np.testing.assert_allclose(q64.T @ q64, np.eye(hi.d), atol=1e-12)
    back = H.apply(H.apply(hi.x, hi.radices, blk64), hi.radices, blk64, inverse=True)
    np.testing.assert_allclose(back, hi.x, atol=1e-10)


def test_page_example_5120_norms_and_round_trip():
    hi = hr_inputs.harp_inputs(rows=4, seed=6)
    assert hi.d == 5120 and hi.radices == (8, 8, 8, 5, 2)
    exact_fb = [np.linalg.qr(f.astype(np.float64))[0] for f in hi.fallbacks]
    blk = H.blocks(hi.radices, hi.theta, exact_fb)
    y = H.apply(hi.x, hi.radices, blk)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(hi.x.astype(np.float64), axis=1),
                               rtol=1e-12)
    np.testing.assert_allclose(H.apply(y, hi.radices, blk, inverse=True), hi.x, atol=1e-9)


def test_rejects_bad_schedules():
    with pytest.raises(ValueError):
        H.apply(np.zeros((1, 10)), (3, 3), [np.zeros((3, 3, 3))] * 2)
    with pytest.raises(ValueError):
        H.blocks((5, 2), np.zeros(10 * 2))          # radix 5 without a fallback
