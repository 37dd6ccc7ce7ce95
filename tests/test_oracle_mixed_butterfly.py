"""Pins for the oracle's mixed-radix rotation and HARP-style butterfly."""
import math

import numpy as np
import pytest
import scipy.linalg

import hr_inputs
import oracle

MR = oracle.mixed_radix
BF = oracle.butterfly


def test_mixed_radix_m1_is_rht():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 256))
    d = rng.choice([-1, 1], size=256)
    np.testing.assert_allclose(MR.mixed_radix(x, d, np.ones((1, 1)), 256),
                               oracle.hadamard.rht(x, d), atol=1e-12)


def test_mixed_radix_identity_block_is_blockwise_rht():
    rng = np.random.default_rng(2)
    m, p = 5, 64
    x = rng.standard_normal((2, m * p))
    d = rng.choice([-1, 1], size=m * p)
    y = MR.mixed_radix(x, d, np.eye(m), p)
    for i in range(m):
        sl = slice(i * p, (i + 1) * p)
        np.testing.assert_allclose(y[:, sl], oracle.hadamard.rht(x[:, sl], d[sl]), atol=1e-12)


def test_mixed_radix_matches_library_kron():
    rng = np.random.default_rng(3)
    m, p = 3, 8
    o = hr_inputs.random_orthogonal_f32(rng, m)
    d = rng.choice([-1, 1], size=m * p)
    x = rng.standard_normal((4, m * p))
    q = np.kron(o.astype(np.float64), scipy.linalg.hadamard(p).astype(np.float64)) \
        * d[None, :] / math.sqrt(p)
    np.testing.assert_allclose(MR.mixed_radix(x, d, o, p), x @ q.T, atol=1e-12)
    np.testing.assert_allclose(MR.mixed_radix_matrix(d, o, p), q, atol=1e-15)


def test_mixed_radix_orthogonal_and_norm():
    rng = np.random.default_rng(4)
    m, p = 7, 32
    g = rng.standard_normal((m, m))
    o, _ = np.linalg.qr(g)
    d = rng.choice([-1, 1], size=m * p)
    q = MR.mixed_radix_matrix(d, o, p)
    np.testing.assert_allclose(q @ q.T, np.eye(m * p), atol=1e-12)
    x = rng.standard_normal((3, m * p))
    np.testing.assert_allclose(np.linalg.norm(MR.mixed_radix(x, d, o, p), axis=1),
                               np.linalg.norm(x, axis=1), rtol=1e-12)


def test_orthogonal_block_input_is_orthogonal_fp32():
    o = hr_inputs.random_orthogonal_f32(np.random.default_rng(5), 7).astype(np.float64)
    np.testing.assert_allclose(o @ o.T, np.eye(7), atol=1e-6)


# ---------------------------------------------------------------- butterfly

def _angles(n, rng):
    L = int(math.log2(n))
    return rng.uniform(0, 2 * math.pi, size=(L, n // 2)).astype(np.float32)


def test_zero_angles_is_permutation():
    n = 64
    rng = np.random.default_rng(6)
    x = rng.standard_normal((3, n))
    perm = rng.permutation(n)
    y = BF.butterfly(x, np.zeros((6, n // 2)), perm)
    assert np.array_equal(y, x[:, perm])


@pytest.mark.parametrize("n", [2, 16, 4096])
def test_zero_angles_with_preconditioner_is_normalised_hadamard(n):
    """HARP's initialisation: theta = 0 recovers the fixed Hadamard processor."""
    x = np.random.default_rng(7).standard_normal((2, n))
    L = int(math.log2(n))
    y = BF.butterfly(x, np.zeros((L, n // 2)), None, precondition=True)
    np.testing.assert_allclose(y, oracle.hadamard.rht(x, None), atol=1e-12)


def test_n2_single_givens():
    th = 0.3
    x = np.array([[2.0, -1.0]])
    y = BF.butterfly(x, np.array([[th]], dtype=np.float32), None)
    t = float(np.float32(th))
    assert y[0, 0] == pytest.approx(math.cos(t) * 2 - math.sin(t) * -1, abs=1e-15)
    assert y[0, 1] == pytest.approx(math.sin(t) * 2 + math.cos(t) * -1, abs=1e-15)


def test_pair_indexing_by_hand():
    n = 8  # 3 stages, 4 pairs each
    x = np.arange(1.0, 9.0)[None, :]
    ang = np.zeros((3, 4))
    # stage 1 (stride 2): pairs (0,2),(1,3),(4,6),(5,7) -> pair indices 0,1,2,3
    ang[1, 2] = math.pi / 2      # rotates pair (4, 6): (a, b) -> (-b, a)
    y = BF.butterfly(x, ang, None)
    ref = x.copy()
    ref[0, 4], ref[0, 6] = -x[0, 6], x[0, 4]
    np.testing.assert_allclose(y, ref, atol=1e-15)
    ang = np.zeros((3, 4))
    ang[2, 3] = math.pi / 2      # stage 2 (stride 4): pair index 3 is (3, 7)
    y = BF.butterfly(x, ang, None)
    ref = x.copy()
    ref[0, 3], ref[0, 7] = -x[0, 7], x[0, 3]
    np.testing.assert_allclose(y, ref, atol=1e-15)
    ang = np.zeros((3, 4))
    ang[0, 1] = math.pi          # stage 0: pair index 1 is (2, 3); rotation by pi negates
    y = BF.butterfly(x, ang, None)
    ref = x.copy()
    ref[0, 2], ref[0, 3] = -x[0, 2], -x[0, 3]
    np.testing.assert_allclose(y, ref, atol=1e-15)


@pytest.mark.parametrize("precondition", [False, True])
def test_butterfly_orthogonal_inverse_norm(precondition):
    n = 256
    rng = np.random.default_rng(8)
    ang = _angles(n, rng)
    perm = rng.permutation(n)
    q = BF.butterfly_matrix(ang, perm, precondition)
    np.testing.assert_allclose(q.T @ q, np.eye(n), atol=1e-12)
    x = rng.standard_normal((4, n))
    y = BF.butterfly(x, ang, perm, precondition)
    np.testing.assert_allclose(y, x @ q.T, atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)
    back = BF.butterfly(y, ang, perm, precondition, inverse=True)
    np.testing.assert_allclose(back, x, atol=1e-12)
    np.testing.assert_allclose(BF.butterfly(x, ang, perm, precondition, inverse=True),
                               x @ q, atol=1e-12)
