"""Comparison rules between the HIP path and the oracle.

* Rotated values: |y_gpu - fl32(y64)| <= 2e-5 * max_i |y64_i| per row.
* Scales, fp16 mode: bit-equal to the oracle's, except groups whose fp32 scale
  lies within 1e-6 relative of an fp16 rounding midpoint (either neighbour is
  accepted there, and that group's codes are re-derived with the GPU's scale).
  fp32 mode: within 1e-6 relative.
* Codes: bit-exact, except elements whose t = y / s lies within 1e-4 of a
  rounding midpoint (|frac(|t|) - 1/2| < 1e-4).
* GEMM: per-group int32 sums bit-exact; |C_gpu - C| <= 1e-5 * sum_g |sA sW acc_g|.
"""
import numpy as np

import oracle

ROT_TOL = 2e-5
SCALE_REL = 1e-6
MID_WIN = 1e-4
GEMM_REL = 1e-5


def check_rotated(y_gpu, y64, tol=ROT_TOL):
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    y32 = y64.astype(np.float32).astype(np.float64)
    bound = tol * np.abs(y64).max(axis=1, keepdims=True)
    err = np.abs(y_gpu - y32)
    bad = err > bound
    assert not bad.any(), (
        f"{bad.sum()} rotated values out of tolerance; worst ratio "
        f"{(err / np.maximum(bound, 1e-300)).max():.3g}")
    return float((err / np.maximum(bound, 1e-300)).max())


def _f16_ambiguous(s32):
    s = s32.astype(np.float64)
    lo = (s * (1 - SCALE_REL)).astype(np.float16)
    hi = (s * (1 + SCALE_REL)).astype(np.float16)
    return lo != hi


def check_quant(codes_gpu, scales_gpu, y64, group, scale_mode="f16", bits=4):
    """Compare codes (packed int4, or int8 when bits == 8) and scales from the
    GPU against the oracle's quantization of y64.  Returns a dict of counts."""
    codes_gpu = np.asarray(codes_gpu)
    scales_gpu = np.asarray(scales_gpu)
    rows, n = y64.shape
    G = n // group
    qmax = (1 << (bits - 1)) - 1
    codes_o, scales_o, s_used_o = oracle.quant.quantize_groups(y64, group, scale_mode, bits)
    q_gpu = oracle.quant.unpack_int4(codes_gpu) if bits == 4 else codes_gpu.view(np.int8)
    assert q_gpu.shape == codes_o.shape
    s_used = s_used_o.copy()
    n_amb = 0
    if scale_mode == "f16":
        assert scales_gpu.dtype == np.float16
        y32 = y64.astype(np.float32)
        s32 = (np.abs(y32.reshape(rows, G, group)).max(-1) / np.float32(qmax)).astype(np.float32)
        amb = _f16_ambiguous(s32)
        eq = scales_gpu.view(np.uint16) == scales_o.view(np.uint16)
        bad = ~eq & ~amb
        assert not bad.any(), f"{bad.sum()} fp16 scales differ outside the midpoint window"
        # ambiguous groups: the GPU's scale must be one of the two neighbours
        if amb.any():
            s = s32.astype(np.float64)[amb]
            lo = (s * (1 - SCALE_REL)).astype(np.float16).view(np.uint16)
            hi = (s * (1 + SCALE_REL)).astype(np.float16).view(np.uint16)
            g = scales_gpu.view(np.uint16)[amb]
            assert np.all((g == lo) | (g == hi))
            n_amb = int((~eq & amb).sum())
        s_used = scales_gpu.astype(np.float32)
    else:
        assert scales_gpu.dtype == np.float32
        rel = np.abs(scales_gpu.astype(np.float64) - scales_o.astype(np.float64))
        ok = rel <= SCALE_REL * np.abs(scales_o.astype(np.float64))
        assert ok.all(), f"{(~ok).sum()} fp32 scales differ by more than 1e-6 relative"
        s_used = scales_gpu.astype(np.float32)
    # codes against the scale the GPU stored (identical to the oracle's except
    # in the exempt cases above)
    y32 = y64.astype(np.float32).reshape(rows, G, group)
    ref = oracle.quant.codes_for_scale(y32, s_used, qmax).reshape(rows, n)
    t = oracle.quant.t_values(y64, s_used, group).astype(np.float64)
    frac = np.abs(t) - np.floor(np.abs(t))
    near_mid = np.abs(frac - 0.5) < MID_WIN
    diff = q_gpu != ref
    bad = diff & ~near_mid
    assert not bad.any(), (f"{bad.sum()} codes differ away from a rounding midpoint; "
                           f"first at {np.argwhere(bad)[:3].tolist()}")
    # a differing code near a midpoint may only be the other neighbour
    assert np.all(np.abs(q_gpu.astype(int) - ref.astype(int))[diff] <= 1)
    return {"codes_exempt_diff": int(diff.sum()), "near_mid": int(near_mid.sum()),
            "scale_ambiguous_diff": n_amb}


def check_gemm(c_gpu, c_ref, bound, acc_gpu=None, acc_ref=None):
    if acc_gpu is not None:
        a = np.asarray(acc_gpu, dtype=np.int64)
        bad = a != acc_ref
        assert not bad.any(), (f"{bad.sum()} of {bad.size} group sums differ; first "
                               f"[m, n, g] {np.argwhere(bad)[:4].tolist()}, gpu "
                               f"{a[bad][:4].tolist()} oracle {acc_ref[bad][:4].tolist()}; "
                               f"rows with errors {np.unique(np.argwhere(bad)[:, 0])[:12].tolist()}")
    err = np.abs(np.asarray(c_gpu, dtype=np.float64) - c_ref.astype(np.float64))
    ok = err <= GEMM_REL * bound + 1e-30
    assert ok.all(), f"{(~ok).sum()} outputs beyond 1e-5 relative; worst {(err / bound).max():.3g}"
    return float((err / np.maximum(bound, 1e-300)).max())
