"""Oracle: the matmul quantization-error probe.

Test infrastructure only.  fp64 matmuls.

Source: "Experiment -- Hadamard rotation for int4 (W4A4) accuracy", Method
(synthetic Gaussian A, B with injected activation outliers; RMS relative error
of the quantized matmul against the fp32 reference, plain vs Hadamard-rotated,
across bit widths) and Results (the synthetic table at M=16 K=2048 N=512,
outliers x20, G=128 and G=32; "W4A8" there means 8-bit activations with 4-bit
weights).

Readings:
* The page writes A.B = (A.Q)(Q.B), which needs a symmetric Q.  With the sign
  diagonal Q = H D / sqrt(K) is not symmetric, so the same row transform is
  applied to A's rows and to B's columns (the weights' K-vectors):
  (A Q^T)(Q B) = A B because Q^T Q = I.  With d = 1 (the page's plain
  Hadamard) this is exactly the page's form.
* Groups run along K for both operands; scales are fp32 (s = absmax / qmax).
* Error = ||C_hat - C||_F / ||C||_F with C = A B from the unrotated inputs.
"""
from __future__ import annotations

import numpy as np

from .hadamard import rht
from .quant import quant_dequant


def probe_error(a, b, signs, group: int, abits: int, bbits: int, rotate: str) -> float:
    """RMS relative error of the quantized product.

    rotate: "none", "rht" (with the given signs) or "plain" (signs all +1)."""
    a64 = np.asarray(a, dtype=np.float64)
    b64 = np.asarray(b, dtype=np.float64)
    c = a64 @ b64
    if rotate == "none":
        ar, br_t = a64, b64.T
    elif rotate in ("rht", "plain"):
        d = signs if rotate == "rht" else None
        ar = rht(a64, d)
        br_t = rht(b64.T, d)          # rotate every column of B (its K-vector)
    else:
        raise ValueError(rotate)
    ah = quant_dequant(ar, group, abits).astype(np.float64)
    bh = quant_dequant(br_t, group, bbits).astype(np.float64).T
    ch = ah @ bh
    return float(np.linalg.norm(ch - c) / np.linalg.norm(c))


ROWS = (("W8A8", 8, 8), ("W4A4", 4, 4), ("W4A8", 8, 4))


def probe_table(a, b, signs, groups=(128, 32)):
    """{(label, rotate, group): error} for the page's five rows plus the
    rotated W8A8 and the plain-Hadamard variants."""
    out = {}
    for label, ab, bb in ROWS:
        for rot in ("none", "rht", "plain"):
            for g in groups:
                out[(label, rot, g)] = probe_error(a, b, signs, g, ab, bb, rot)
    return out
