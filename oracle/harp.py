"""Oracle: HARP's general mixed-radix processor -- stages of dense b x b
orthogonal blocks B_{t,c} = Q_{t,c}(theta) G_{b_t}.

Test infrastructure only.  fp64.

Sources: HARP technical summary (gist.science), section 2.1 (a mixed-radix
schedule b = (b_0 .. b_{m-1}) with prod b_t = d; stage t applies a
block-diagonal orthogonal matrix to groups of coordinates, the stages
separated by stride permutations; radices that are not powers of two use a
fixed orthogonal fallback from the QR factorisation of a Gaussian matrix; the
example 5120 = (8, 8, 8, 5, 2)) and section 2.2 (B_{t,c}(theta) =
Q_{t,c}(theta) G_{b_t}; G the normalised Sylvester-Hadamard matrix for powers
of two, the QR fallback otherwise; Q a Givens rotation for b = 2 and the
Cayley map for b > 2; theta = 0 gives B = G, so the processor starts as the
fixed Hadamard transform).

Readings:
* Digits.  Write a coordinate as i = sum_t i_t S_t with S_t = b_0 ... b_{t-1}
  (digit 0 varies fastest).  Stage t acts along digit t: block
  c = lo + S_t * hi (lo < S_t, hi < d / (S_t b_t)) holds the coordinates
  i_r = lo + S_t (r + b_t hi), r = 0 .. b_t - 1, and maps x_{i_q} to
  y_{i_r} = sum_q B_{t,c}[r][q] x_{i_q}.  This is the stride-permutation
  layout with the permutations folded into the indexing; for b = 2 it is the
  butterfly's pair (i, i + 2^t) with pair index c.
* Stages run t = 0 .. m-1; the inverse runs them backwards with B^T.
* Parameters: Q for b = 2 is [[cos th, -sin th], [sin th, cos th]] (one angle);
  for b > 2, Q = (I - A)^(-1) (I + A) with A skew-symmetric, its b(b-1)/2
  upper-triangle entries A[i][j] (i < j, row-major order) the parameters and
  A[j][i] = -A[i][j].  theta of stage t is [d / b_t][P_t], P_t = 1 for b = 2
  and b(b-1)/2 otherwise; stages are concatenated in order.
* G_b: H_b / sqrt(b) (Sylvester, natural order) for b a power of two; for
  other radices the caller's fixed orthogonal matrix, one per such stage in
  stage order.
"""
from __future__ import annotations

import math

import numpy as np

from .hadamard import sylvester


def is_pow2(b: int) -> bool:
    return b >= 1 and (b & (b - 1)) == 0


def n_params(b: int) -> int:
    return 1 if b == 2 else b * (b - 1) // 2


def block_q(params, b: int) -> np.ndarray:
    """The learnable factor Q(theta) of one block (Givens for b = 2, Cayley otherwise)."""
    p = np.asarray(params, dtype=np.float64)
    if b == 2:
        c, s = math.cos(p[0]), math.sin(p[0])
        return np.array([[c, -s], [s, c]])
    a = np.zeros((b, b))
    iu = np.triu_indices(b, k=1)
    a[iu] = p
    a = a - a.T
    eye = np.eye(b)
    return np.linalg.solve(eye - a, eye + a)


def mixer(b: int, fallback=None) -> np.ndarray:
    if is_pow2(b):
        return sylvester(b).astype(np.float64) / math.sqrt(b)
    if fallback is None:
        raise ValueError(f"radix {b} needs a fallback matrix")
    return np.asarray(fallback, dtype=np.float64)


def blocks(radices, theta, fallbacks=()) -> list:
    """Dense blocks per stage: list of [d / b_t][b_t][b_t] fp64 arrays."""
    radices = [int(b) for b in radices]
    d = int(np.prod(radices))
    th = np.asarray(theta, dtype=np.float64).ravel()
    fb = list(fallbacks)
    out, off = [], 0
    for b in radices:
        g = mixer(b, None if is_pow2(b) or not fb else fb.pop(0))
        nb, P = d // b, n_params(b)
        pt = th[off:off + nb * P].reshape(nb, P)
        off += nb * P
        out.append(np.stack([block_q(pt[c], b) @ g for c in range(nb)]))
    if off != th.size:
        raise ValueError("theta has the wrong length")
    return out


def apply(x, radices, stage_blocks, inverse: bool = False) -> np.ndarray:
    """y = (stages of B_{t,c}) x for every row x (or the transpose with inverse)."""
    z = np.array(np.atleast_2d(np.asarray(x, dtype=np.float64)), copy=True)
    rows, d = z.shape
    radices = [int(b) for b in radices]
    if int(np.prod(radices)) != d:
        raise ValueError("radices do not multiply to the row length")
    strides = [int(np.prod(radices[:t])) for t in range(len(radices))]
    order = reversed(range(len(radices))) if inverse else range(len(radices))
    for t in order:
        b, S = radices[t], strides[t]
        H = d // (S * b)
        B = np.asarray(stage_blocks[t], dtype=np.float64).reshape(H, S, b, b)   # c = lo + S hi
        v = z.reshape(rows, H, b, S)
        if inverse:
            z = np.einsum("hlqr,nhql->nhrl", B, v).reshape(rows, d)
        else:
            z = np.einsum("hlrq,nhql->nhrl", B, v).reshape(rows, d)
    return z


def matrix(radices, stage_blocks) -> np.ndarray:
    """The dense d x d matrix Q of the forward processor (y = Q x)."""
    d = int(np.prod([int(b) for b in radices]))
    return apply(np.eye(d), radices, stage_blocks).T
