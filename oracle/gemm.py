"""Oracle: W4A4 GEMM on packed int4 codes with per-group scales.

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
(|a|, |w| <= 8 and G <= 4096 keep every partial sum far below 2^53).
"""
from __future__ import annotations

import numpy as np

from .quant import unpack_int4


def group_sums(a_packed, w_packed, group: int, rows=None) -> np.ndarray:
    """Exact per-group integer sums, int64 [len(rows)][N][K/G].

    rows: optional index array of A rows to compute (all rows if None)."""
    a = unpack_int4(a_packed).astype(np.float64)
    w = unpack_int4(w_packed).astype(np.float64)
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
