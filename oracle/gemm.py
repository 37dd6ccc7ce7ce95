"""Oracle: W4A4 and W4A8 GEMMs on int4 weight codes with per-group scales.

Test infrastructure only.

Source: "Experiment -- Hadamard rotation for int4 (W4A4) accuracy",
Hypothesis (W4A4 on a same-precision integer MAC: both operands int4 with
per-group absmax scales) and Verdict (splitting the K dimension into separate
per-group submissions is what made int4 slow, so the per-group scaling belongs
inside the GEMM).

Reading: C = A W^T with both operands K-contiguous packed int4 codes,
    acc[m][n][g] = sum_{k in group g} a[m][k] * w[n][k]      (exact integer)
    C[m][n]      = fl32( sum_g sA[m][g] * sW[n][g] * acc[m][n][g] )  (fp64 sum)
The integer sums are computed with an fp64 matrix product, which is exact here
(|a| <= 128, |w| <= 8 and G <= 4096 keep every partial sum far below 2^53).

W4A8 (same page, Method and Results: the "W4A8 (act8/wt4)" rows, int8
activations against int4 weights): the same two formulas with A held as one
int8 code per element instead of packed nibbles.  W8A8 (the W8A8 rows): both
operands held that way.
"""
from __future__ import annotations

import numpy as np

from .quant import unpack_int4


def group_sums(a_packed, w_packed, group: int, rows=None) -> np.ndarray:
    """Exact per-group integer sums, int64 [len(rows)][N][K/G].

    rows: optional index array of A rows to compute (all rows if None)."""
    return _group_sums(unpack_int4(a_packed), unpack_int4(w_packed), group, rows)


def _group_sums(a_codes, w_codes, group: int, rows=None) -> np.ndarray:
    a = np.asarray(a_codes).astype(np.float64)
    w = np.asarray(w_codes).astype(np.float64)
    if rows is not None:
        a = a[np.asarray(rows)]
    K = a.shape[1]
    if K % group or w.shape[1] != K:
        raise ValueError("bad K / group")
    G = K // group
    out = np.empty((a.shape[0], w.shape[0], G), dtype=np.int64)
    for g in range(G):
        sl = slice(g * group, (g + 1) * group)
        out[:, :, g] = np.rint(a[:, sl] @ w[:, sl].T).astype(np.int64)
    return out


def w4a4_gemm(a_packed, a_scales, w_packed, w_scales, group: int, rows=None,
              return_sums: bool = False):
    """C fp32 [len(rows)][N] (and optionally the exact per-group sums).

    Also returns, when return_sums, the fp64 per-element bound
    sum_g |sA sW acc_g| used to judge the fp32 result."""
    acc = group_sums(a_packed, w_packed, group, rows)
    return _scale_sum(acc, a_scales, w_scales, rows, return_sums)


def w4a8_gemm(a_codes, a_scales, w_packed, w_scales, group: int, rows=None,
              return_sums: bool = False):
    """W4A8: A int8 codes [M][K] (one per element), W packed int4 [N][K/2].
    Returns as w4a4_gemm."""
    a = np.asarray(a_codes)
    if a.dtype != np.int8:
        raise ValueError("a_codes must be int8")
    acc = _group_sums(a, unpack_int4(w_packed), group, rows)
    return _scale_sum(acc, a_scales, w_scales, rows, return_sums)


def w8a8_gemm(a_codes, a_scales, w_codes, w_scales, group: int, rows=None,
              return_sums: bool = False):
    """Both operands held one int8 code per element: A [M][K], W [N][K].

    Covers the W8A8 rows of the experiment page's Results (int8 activations
    and weights) and the W4A4 GEMM with its int4 codes held in int8 for an
    int8 MAC; the sums and the scale fusion are those of w4a4_gemm.  Returns
    as w4a4_gemm."""
    a = np.asarray(a_codes)
    w = np.asarray(w_codes)
    if a.dtype != np.int8 or w.dtype != np.int8:
        raise ValueError("a_codes and w_codes must be int8")
    acc = _group_sums(a, w, group, rows)
    return _scale_sum(acc, a_scales, w_scales, rows, return_sums)


def _scale_sum(acc, a_scales, w_scales, rows, return_sums):
    sa = np.asarray(a_scales).astype(np.float64)
    if rows is not None:
        sa = sa[np.asarray(rows)]
    sw = np.asarray(w_scales).astype(np.float64)
    terms = sa[:, None, :] * sw[None, :, :] * acc.astype(np.float64)
    c64 = terms.sum(axis=-1)
    c32 = c64.astype(np.float32)
    if return_sums:
        return c32, acc, np.abs(terms).sum(axis=-1)
    return c32
