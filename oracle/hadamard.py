"""Oracle: explicit Sylvester-Hadamard matrix and the randomized Hadamard transform.

Test infrastructure only (see the package docstring).  fp64 throughout.

Sources:
* "Experiment -- Hadamard rotation for int4 (W4A4) accuracy", Hypothesis: the
  rotation is Q = H / sqrt(K), orthonormal and symmetric; Method: the probe
  rotates with a fast Walsh-Hadamard transform followed by x 1/sqrt(K).
* "Llama-3.2-1B-Instruct-HadamardSpin-4bits", How it Works: Hadamard of size
  n = 2048 with the 1/sqrt(n) scaling.
* HARP abstract and technical summary section 1: the fixed randomized Hadamard
  transform (RHT) of incoherence processing.

Reading (stated once, used everywhere): the RHT of a row x is
    y = H_n (d * x) / sqrt(n)
with d a +-1 sign diagonal applied first, Q = H D / sqrt(n) acting on column
vectors, and H_n the Sylvester matrix in natural order,
    H[i][j] = (-1)^popcount(i & j).
The plain-Hadamard variant that the experiment page measured is d = all ones.
The oracle multiplies by the explicit matrix (O(n^2) per row); the fast
transform is what the GPU path implements.
"""
from __future__ import annotations

import numpy as np


def sylvester(n: int) -> np.ndarray:
    """Sylvester-Hadamard matrix H_n in natural order as int8 [n][n]:
    H[i][j] = (-1)^popcount(i & j).  n must be a power of two."""
    if n < 1 or (n & (n - 1)) != 0:
        raise ValueError(f"n={n} is not a power of two")
    i = np.arange(n, dtype=np.uint32)
    parity = np.bitwise_count(np.bitwise_and.outer(i, i)) & 1
    return (1 - 2 * parity.astype(np.int8)).astype(np.int8)


def rht(x, signs=None) -> np.ndarray:
    """Randomized Hadamard transform of each row of x, in fp64.

    x: array-like [rows][n] (any float dtype; widened exactly to fp64).
    signs: int array [n] of +-1, or None for all +1 (the plain Hadamard).
    Returns y64 [rows][n] = ((H_n (d * x_r)) / sqrt(n)) for every row r."""
    x64 = np.asarray(x, dtype=np.float64)
    squeeze = x64.ndim == 1
    x64 = np.atleast_2d(x64)
    n = x64.shape[1]
    u = x64 if signs is None else x64 * np.asarray(signs, dtype=np.float64)[None, :]
    h = sylvester(n).astype(np.float64)
    y = (u @ h.T) / np.sqrt(np.float64(n))
    return y[0] if squeeze else y


def rht_matrix(n: int, signs=None) -> np.ndarray:
    """The dense fp64 rotation Q = H_n D / sqrt(n) (acts on column vectors)."""
    h = sylvester(n).astype(np.float64)
    d = np.ones(n) if signs is None else np.asarray(signs, dtype=np.float64)
    return h * d[None, :] / np.sqrt(np.float64(n))
