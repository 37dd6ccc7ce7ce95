"""Oracle: mixed-radix randomized rotation for n = m * p (p a power of two).

Test infrastructure only.  fp64.

Sources: HARP abstract (non-power-of-two dimensions through mixed-radix
schedules); HARP technical summary (gist.science) section 2.1 (a schedule of
radices whose product is the dimension; radices that are not powers of two use
a deterministic orthogonal block, the QR of a fixed Gaussian matrix) and
section 2.2 (block kernel = orthogonal factor times a fixed base mixer).

Reading: the single-odd-radix schedule n = m * p is the rotation
    Q = (O kron H_p) D / sqrt(p)
with O an m x m orthogonal block (given, fp32 values used exactly), H_p the
Sylvester matrix, D the sign diagonal, and Kronecker indexing
    (O kron H)[i*p + r][j*p + c] = O[i][j] * H[r][c],
i.e. chunk i of the row is elements [i*p, (i+1)*p).  Only 1/sqrt(p) is applied
because O is already orthogonal.
"""
from __future__ import annotations

import numpy as np

from .hadamard import sylvester


def mixed_radix(x, signs, block, p: int) -> np.ndarray:
    """y64 [rows][m*p] = ((O kron H_p) D x_r) / sqrt(p) for every row r.

    Computed as: u = d * x; U = u reshaped to m chunks of p; V = U H_p^T
    (each chunk through the explicit Hadamard); Y = O V (mix across chunks at
    each position); y = vec(Y) / sqrt(p)."""
    x64 = np.atleast_2d(np.asarray(x, dtype=np.float64))
    o = np.asarray(block, dtype=np.float64)
    m = o.shape[0]
    rows, n = x64.shape
    if n != m * p:
        raise ValueError("row length must be m * p")
    u = x64 if signs is None else x64 * np.asarray(signs, dtype=np.float64)[None, :]
    h = sylvester(p).astype(np.float64)
    v = u.reshape(rows, m, p) @ h.T                       # [rows][m][p]
    y = np.einsum("ij,rjc->ric", o, v) / np.sqrt(np.float64(p))
    return y.reshape(rows, n)


def mixed_radix_matrix(signs, block, p: int) -> np.ndarray:
    """Dense fp64 Q = (O kron H_p) D / sqrt(p), built entry by entry from the
    Kronecker index rule (small sizes only)."""
    o = np.asarray(block, dtype=np.float64)
    m = o.shape[0]
    h = sylvester(p).astype(np.float64)
    n = m * p
    q = np.empty((n, n))
    for i in range(m):
        for j in range(m):
            q[i * p:(i + 1) * p, j * p:(j + 1) * p] = o[i, j] * h
    d = np.ones(n) if signs is None else np.asarray(signs, dtype=np.float64)
    return q * d[None, :] / np.sqrt(np.float64(p))
