"""Oracle: HARP-style butterfly of 2x2 orthogonal blocks, then a gather permutation.

Test infrastructure only.  fp64.

Sources: HARP abstract (each rotation is a product of sparse butterfly-like
block-orthogonal stages; initialises to the RHT up to a fixed permutation);
HARP technical summary (gist.science) section 2.1 (stages of block-diagonal
orthogonal matrices on coordinate groups, separated by stride permutations),
section 2.2 (block kernel B(theta) = Q(theta) G_b, Q a Givens rotation for
b = 2, G_2 the normalised Sylvester-Hadamard, theta = 0 gives B = G) and
section 2.4 (O(d log d) application without materialised permutations).

Readings:
* Stages s = 0 .. L-1 (L = log2 n) in ascending order.  Stage s pairs the
  elements (i, i + 2^s) for every i whose bit s is clear; such a pair has index
      pair(i, s) = ((i >> (s+1)) << s) | (i & (2^s - 1))
  into the [L][n/2] angle table.  Addressing the pairs in place is the
  stride-permutation layout with the permutations folded into the indexing.
* The block acting on (a, b) = (x_i, x_{i+2^s}) is
      G_2:        (a, b) <- ((a + b)/sqrt 2, (a - b)/sqrt 2)   [precondition only]
      Q(theta):   (a, b) <- (c a - s b, s a + c b),  c = cos theta, s = sin theta
  so the block is Q(theta) G_2 with the preconditioner, and Q(theta) alone
  without it.  Coefficients are the fp64 cos / sin of the fp32 angle.
* After the last stage the row is gathered: out[i] = z[perm[i]].
* The inverse applies Q^T: scatter z[perm[i]] = x[i], then the stages in
  descending order with each block transposed.
"""
from __future__ import annotations

import math

import numpy as np

_R2 = 1.0 / math.sqrt(2.0)


def _stage_view(z: np.ndarray, s: int):
    rows, n = z.shape
    v = z.reshape(rows, n >> (s + 1), 2, 1 << s)
    return v[:, :, 0, :], v[:, :, 1, :]


def butterfly(x, angles, perm=None, precondition: bool = False, inverse: bool = False) -> np.ndarray:
    """Apply the butterfly (or its transpose) to every row of x in fp64.

    x: [rows][n]; angles: [L][n/2] (fp32 values used exactly); perm: int [n]
    gather permutation or None for identity."""
    z = np.array(np.atleast_2d(np.asarray(x, dtype=np.float64)), copy=True)
    rows, n = z.shape
    L = int(round(math.log2(n)))
    if 1 << L != n:
        raise ValueError("n must be a power of two")
    th = np.asarray(angles, dtype=np.float64)
    if th.shape != (L, n // 2):
        raise ValueError("angles must be [log2 n][n/2]")
    cos, sin = np.cos(th), np.sin(th)

    if not inverse:
        for s in range(L):
            a, b = _stage_view(z, s)
            if precondition:
                a, b = (a + b) * _R2, (a - b) * _R2
            c = cos[s].reshape(n >> (s + 1), 1 << s)[None]
            sn = sin[s].reshape(n >> (s + 1), 1 << s)[None]
            na, nb = c * a - sn * b, sn * a + c * b
            va, vb = _stage_view(z, s)
            va[...] = na
            vb[...] = nb
        if perm is not None:
            z = z[:, np.asarray(perm)]
        return z

    if perm is not None:
        zz = np.empty_like(z)
        zz[:, np.asarray(perm)] = z
        z = zz
    for s in reversed(range(L)):
        a, b = _stage_view(z, s)
        c = cos[s].reshape(n >> (s + 1), 1 << s)[None]
        sn = sin[s].reshape(n >> (s + 1), 1 << s)[None]
        na, nb = c * a + sn * b, -sn * a + c * b
        if precondition:
            na, nb = (na + nb) * _R2, (na - nb) * _R2
        va, vb = _stage_view(z, s)
        va[...] = na
        vb[...] = nb
    return z


def butterfly_matrix(angles, perm=None, precondition: bool = False) -> np.ndarray:
    """Dense fp64 Q (acting on column vectors), from pushing each basis vector
    through the stages: column j of Q is the butterfly of e_j."""
    n = np.asarray(angles).shape[1] * 2
    return butterfly(np.eye(n), angles, perm, precondition).T
