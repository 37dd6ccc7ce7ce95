"""Pins for the oracle's Sylvester matrix and randomized Hadamard transform.

Each check ties the oracle to something other than itself: exact integer
identities, a library routine (scipy's Sylvester construction), the fast
recursive transform written independently here, and closed forms."""
import numpy as np
import pytest
import scipy.linalg

import hr_inputs
import oracle


@pytest.mark.parametrize("n", [1, 2, 4, 8, 64, 256, 1024])
def test_hh_equals_n_identity(n):
    h = oracle.hadamard.sylvester(n).astype(np.int64)
    assert np.array_equal(h @ h, n * np.eye(n, dtype=np.int64))
    assert np.array_equal(h, h.T)


@pytest.mark.parametrize("n", [2, 16, 128, 2048])
def test_matches_scipy_sylvester(n):
    assert np.array_equal(oracle.hadamard.sylvester(n).astype(np.int64),
                          scipy.linalg.hadamard(n).astype(np.int64))


def test_kronecker_recursion():
    for n in (1, 2, 4, 32, 512):
        h = oracle.hadamard.sylvester(n).astype(np.int64)
        h2 = oracle.hadamard.sylvester(2 * n).astype(np.int64)
        assert np.array_equal(h2, np.block([[h, h], [h, -h]]))


def test_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        oracle.hadamard.sylvester(12)


def _fwht_recursive(v):
    """Textbook fast Walsh-Hadamard transform by recursion on halves."""
    n = len(v)
    if n == 1:
        return v.copy()
    a = _fwht_recursive(v[: n // 2])
    b = _fwht_recursive(v[n // 2:])
    return np.concatenate([a + b, a - b])


@pytest.mark.parametrize("n", [2, 8, 64, 2048])
def test_rht_matches_fast_transform(n):
    rng = np.random.default_rng(n)
    x = rng.standard_normal((3, n))
    d = rng.choice([-1, 1], size=n)
    y = oracle.hadamard.rht(x, d)
    for r in range(3):
        ref = _fwht_recursive(d * x[r]) / np.sqrt(n)
        np.testing.assert_allclose(y[r], ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_delta_and_sign_vector_closed_forms():
    n = 2048
    d = hr_inputs.sign_vector(np.random.default_rng(7), n)
    e0 = np.zeros(n)
    e0[0] = 1.0
    y = oracle.hadamard.rht(e0, d)
    # x = e_0: every output is d_0 / sqrt(n)
    assert np.all(y == d[0] / np.sqrt(n))
    # x = d: u = all ones, so y = sqrt(n) e_0 with every other entry exactly 0
    y = oracle.hadamard.rht(d.astype(np.float64), d)
    assert y[0] == pytest.approx(np.sqrt(n), rel=1e-15)
    assert np.all(y[1:] == 0.0)


def test_norm_preserved():
    x = np.random.default_rng(3).standard_normal((5, 1024)) * 10
    d = np.random.default_rng(4).choice([-1, 1], size=1024)
    y = oracle.hadamard.rht(x, d)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


def test_rotation_identity_two_sided():
    """(A Q^T)(W Q^T)^T = A W^T: exact in fp64 to rounding, ~1e-6 in fp32."""
    rng = np.random.default_rng(11)
    K = 2048
    a = rng.standard_normal((16, K)).astype(np.float32)
    a[:, rng.choice(K, 8, replace=False)] *= 20
    w = rng.standard_normal((64, K)).astype(np.float32)
    d = rng.choice([-1, 1], size=K)
    ref = a.astype(np.float64) @ w.astype(np.float64).T
    ar = oracle.hadamard.rht(a, d)
    wr = oracle.hadamard.rht(w, d)
    rel64 = np.abs(ar @ wr.T - ref).max() / np.abs(ref).max()
    assert rel64 < 1e-12
    rel32 = np.abs(ar.astype(np.float32) @ wr.astype(np.float32).T - ref).max() / np.abs(ref).max()
    assert rel32 < 5e-6


def test_dense_matrix_orthogonal():
    d = np.random.default_rng(5).choice([-1, 1], size=256)
    q = oracle.hadamard.rht_matrix(256, d)
    np.testing.assert_allclose(q.T @ q, np.eye(256), atol=1e-13)
    x = np.random.default_rng(6).standard_normal(256)
    np.testing.assert_allclose(q @ x, oracle.hadamard.rht(x, d), atol=1e-12)


def test_peak_amplitude_drops_with_outliers():
    """The model card's claim that rotation cuts the peak activation amplitude
    (How it Works), as a trend on bf16 rows with x50 outlier channels."""
    inp = hr_inputs.rht_inputs(rows=64, n=2048)
    x = inp.x.float().numpy()
    y = oracle.hadamard.rht(x, inp.signs)
    ratio = np.abs(x).max(axis=1) / np.abs(y).max(axis=1)
    assert np.median(ratio) > 5.0
