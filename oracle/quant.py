"""Oracle: per-group symmetric absmax quantization, int4 nibble packing, dequant.

Test infrastructure only.

Source: "Experiment -- Hadamard rotation for int4 (W4A4) accuracy", Method
(per-group symmetric integer quantize -> dequantize for any bit width) and
Hypothesis (outliers inflate the per-group absmax scale).  The symmetric rule
s = absmax / qmax with q = round-half-away(x / s) clamped to [-qmax, qmax],
qmax = 2^(bits-1) - 1 (7 for int4), is the plain reading of "symmetric".

Readings (where the pages are silent):
* A group is G consecutive rotated outputs of a row, aligned at multiples of G.
* Decisions are taken in fp32, the precision of the rotated values the GPU
  path produces: y32 = fl32(y64); a = max |y32| over the group;
  s32 = fl32(a / qmax) (IEEE fp32 division); the stored scale is fp16(s32)
  rounded to nearest even ("f16" mode) or s32 itself ("f32" mode); codes are
  taken against the stored scale: t = fl32(y32 / s), q = sign(t) * floor(|t| + 1/2)
  clamped to [-qmax, qmax].
* A group whose stored scale is 0 gets all-zero codes.
* Two codes per byte, two's complement nibbles, element 2j in the low nibble
  and element 2j+1 in the high nibble.  -8 is never produced.
"""
from __future__ import annotations

import numpy as np


def quantize_groups(y, group: int, scale_dtype: str = "f16", bits: int = 4):
    """Quantize each row of y in groups of ``group``.

    y: [rows][n] values (fp64 or fp32); they are rounded to fp32 first.
    Returns (codes int8 [rows][n], scales [rows][n/group] as float16 or float32,
    s_used fp32 [rows][n/group] -- the scale the codes were taken against)."""
    y32 = np.atleast_2d(np.asarray(y)).astype(np.float32)
    rows, n = y32.shape
    if n % group:
        raise ValueError("group must divide n")
    qmax = np.float32((1 << (bits - 1)) - 1)
    g = y32.reshape(rows, n // group, group)
    a = np.abs(g).max(axis=-1)
    s32 = (a / qmax).astype(np.float32)
    if scale_dtype == "f16":
        stored = s32.astype(np.float16)
        s_used = stored.astype(np.float32)
    elif scale_dtype == "f32":
        stored = s32
        s_used = s32
    else:
        raise ValueError(scale_dtype)
    codes = codes_for_scale(g, s_used, qmax)
    return codes.reshape(rows, n), stored, s_used


def codes_for_scale(g32: np.ndarray, s_used: np.ndarray, qmax) -> np.ndarray:
    """Codes of fp32 values g32 [..., G] against fp32 scales s_used [...]:
    t = fl32(y / s); q = sign(t) floor(|t| + 1/2), clamped; zero scale -> 0."""
    qmax = np.float32(qmax)
    s = s_used[..., None]
    zero = s == 0
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (g32 / np.where(zero, np.float32(1), s)).astype(np.float32)
    t64 = t.astype(np.float64)
    q = np.sign(t64) * np.floor(np.abs(t64) + 0.5)
    q = np.clip(q, -float(qmax), float(qmax))
    q = np.where(zero, 0.0, q)
    return q.astype(np.int8)


def t_values(y, s_used: np.ndarray, group: int) -> np.ndarray:
    """fl32(y32 / s) per element (the value whose rounding decides the code)."""
    y32 = np.atleast_2d(np.asarray(y)).astype(np.float32)
    rows, n = y32.shape
    g = y32.reshape(rows, n // group, group)
    s = s_used[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (g / np.where(s == 0, np.float32(1), s)).astype(np.float32)
    return t.reshape(rows, n)


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """int8 codes [rows][n] in [-8, 7] -> uint8 [rows][n/2]; even element in the
    low nibble, odd element in the high nibble, two's complement."""
    c = np.atleast_2d(np.asarray(codes)).astype(np.int16)
    lo = c[:, 0::2] & 0xF
    hi = c[:, 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """uint8 [rows][n/2] -> int8 codes [rows][n] (inverse of pack_int4)."""
    b = np.atleast_2d(np.asarray(packed)).astype(np.int16)
    rows, half = b.shape
    out = np.empty((rows, 2 * half), dtype=np.int16)
    lo = b & 0xF
    hi = (b >> 4) & 0xF
    out[:, 0::2] = np.where(lo >= 8, lo - 16, lo)
    out[:, 1::2] = np.where(hi >= 8, hi - 16, hi)
    return out.astype(np.int8)


def dequant(codes: np.ndarray, scales: np.ndarray, group: int) -> np.ndarray:
    """x_hat = q * s per element in fp32 (one IEEE fp32 product)."""
    q = np.atleast_2d(np.asarray(codes)).astype(np.float32)
    rows, n = q.shape
    s = np.asarray(scales).astype(np.float32).reshape(rows, n // group, 1)
    return (q.reshape(rows, n // group, group) * s).astype(np.float32).reshape(rows, n)


def quant_dequant(y, group: int, bits: int) -> np.ndarray:
    """Per-group symmetric quantize -> dequantize at ``bits`` with fp32 scales
    (the probe's operation)."""
    codes, scales, _ = quantize_groups(y, group, "f32", bits)
    return dequant(codes, scales, group)
