"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This module draws random numbers and nothing else: it holds none of the
rotation, quantization or GEMM arithmetic.  Every draw uses numpy's PCG64 with
an explicit seed and a documented draw order, so the CPU oracle and the HIP
path see identical bytes.

Workloads (sizes follow the pages' Llama shapes):

* ``probe``      -- the matmul-error probe of "Experiment -- Hadamard rotation
  for int4 (W4A4) accuracy" (Method / Results, synthetic table): A fp32 16x2048
  N(0,1) with 8 channels scaled x20, B fp32 2048x512 N(0,1).
* ``rht``        -- bf16 activations, 65536 tokens x 2048 (the n=2048 Hadamard
  of the "Llama-3.2-1B-Instruct-HadamardSpin-4bits" card), N(0,1) plus 0.1% of
  channels scaled x50.
* ``mixed``      -- bf16 16384 x 14336 (14336 = 7*2048), N(0,1) plus 0.1% of
  channels scaled x20, a 7x7 orthogonal block and a sign diagonal.
* ``butterfly``  -- fp32 32768 x 4096 N(0,1), 12 stages of 2048 Givens angles
  U(0, 2*pi), and a seeded permutation of 4096.
* ``gemm``       -- packed int4 codes uniform over [-7, 7] for A (M x 4096) and
  W (4096 x 4096), fp16 group scales (group 128) uniform in [0.001, 0.05].
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

# Seeds per workload.  The probe uses seeds 1..10 (seed 1 is the headline).
SEED_PROBE = 1
SEED_RHT = 2
SEED_MIXED = 3
SEED_BUTTERFLY = 4
SEED_GEMM = 5


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _to_bf16(x32: np.ndarray):
    """Round an fp32 array to bfloat16 (round-to-nearest-even) as a torch CPU tensor."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)


def outlier_count(n: int, frac: float = 0.001) -> int:
    """Number of outlier channels: round(frac * n), at least 1."""
    return max(1, int(round(frac * n)))


def sign_vector(rng: np.random.Generator, n: int) -> np.ndarray:
    """A seeded +-1 diagonal as int8 [n]."""
    return (rng.integers(0, 2, size=n, dtype=np.int64) * 2 - 1).astype(np.int8)


def gaussian_rows_with_outliers(rng, rows: int, n: int, n_outliers: int, scale: float) -> np.ndarray:
    """fp32 [rows][n] N(0,1); every value of n_outliers channels (drawn without
    replacement) is multiplied by ``scale``.  Draw order: channels, then values."""
    chans = rng.choice(n, size=n_outliers, replace=False)
    x = rng.standard_normal(size=(rows, n), dtype=np.float32)
    x[:, chans] *= np.float32(scale)
    return x


@dataclass
class RhtInputs:
    x: "object"            # torch bf16 (or fp32) CPU tensor [rows][n]
    signs: np.ndarray      # int8 [n]
    n: int
    rows: int


def rht_inputs(rows: int = 65536, n: int = 2048, seed: int = SEED_RHT,
               outlier_scale: float = 50.0, dtype: str = "bf16") -> RhtInputs:
    """Activations for the power-of-two rotate(+quantize) path.

    Draw order: signs [n], outlier channels, values [rows][n] (fp32), then the
    outlier channels are scaled and the array is rounded to bf16."""
    rng = _rng(seed)
    signs = sign_vector(rng, n)
    x32 = gaussian_rows_with_outliers(rng, rows, n, outlier_count(n), outlier_scale)
    if dtype == "bf16":
        x = _to_bf16(x32)
    elif dtype == "fp32":
        import torch
        x = torch.from_numpy(x32)
    else:
        raise ValueError(dtype)
    return RhtInputs(x=x, signs=signs, n=n, rows=rows)


def random_orthogonal_f32(rng: np.random.Generator, m: int) -> np.ndarray:
    """A seeded m x m orthogonal block: QR of an fp64 Gaussian matrix with the
    columns of Q multiplied by sign(diag(R)), then cast to fp32.  This is the
    deterministic orthogonal fallback that the HARP summary describes for radices
    that are not powers of two (technical summary, section 2.1); here it is only
    an input, handed to both sides as the same fp32 matrix."""
    g = rng.standard_normal(size=(m, m))
    q, r = np.linalg.qr(g)
    q = q * np.sign(np.diag(r))[None, :]
    return q.astype(np.float32)


@dataclass
class MixedInputs:
    x: "object"            # torch bf16 CPU tensor [rows][m*p]
    signs: np.ndarray      # int8 [m*p]
    block: np.ndarray      # fp32 [m][m] row-major
    m: int
    p: int
    rows: int


def mixed_inputs(rows: int = 16384, m: int = 7, p: int = 2048, seed: int = SEED_MIXED,
                 outlier_scale: float = 20.0) -> MixedInputs:
    """Draw order: signs [m*p], outlier channels, values, then the m x m block."""
    rng = _rng(seed)
    n = m * p
    signs = sign_vector(rng, n)
    x32 = gaussian_rows_with_outliers(rng, rows, n, outlier_count(n), outlier_scale)
    block = random_orthogonal_f32(rng, m)
    return MixedInputs(x=_to_bf16(x32), signs=signs, block=block, m=m, p=p, rows=rows)


@dataclass
class ButterflyInputs:
    x: np.ndarray          # fp32 [rows][n]
    angles: np.ndarray     # fp32 [log2 n][n/2]
    perm: np.ndarray       # int32 [n]
    n: int
    rows: int


def butterfly_inputs(rows: int = 32768, n: int = 4096, seed: int = SEED_BUTTERFLY) -> ButterflyInputs:
    """Draw order: values [rows][n] N(0,1) fp32, angles U(0, 2*pi) fp32, permutation."""
    rng = _rng(seed)
    stages = int(math.log2(n))
    assert 1 << stages == n
    x = rng.standard_normal(size=(rows, n), dtype=np.float32)
    angles = rng.uniform(0.0, 2.0 * math.pi, size=(stages, n // 2)).astype(np.float32)
    perm = rng.permutation(n).astype(np.int32)
    return ButterflyInputs(x=x, angles=angles, perm=perm, n=n, rows=rows)


SEED_HARP = 6


@dataclass
class HarpInputs:
    x: np.ndarray          # fp32 [rows][d]
    radices: tuple         # the mixed-radix schedule, prod = d
    theta: np.ndarray      # fp32, per stage [d / b][P_b] concatenated (P_2 = 1, P_b = b(b-1)/2)
    fallbacks: list        # fp32 [b][b] orthogonal matrices, one per radix that is not a power of two
    d: int
    rows: int


def harp_inputs(rows: int = 4096, radices=(8, 8, 8, 5, 2), seed: int = SEED_HARP,
                theta_scale: float = 0.3, outlier_scale: float = 20.0) -> HarpInputs:
    """The HARP summary's 5120 = (8, 8, 8, 5, 2) schedule by default.
    Draw order: values (N(0,1) rows with round(0.001 d) channels scaled),
    then per stage its parameters (b = 2: angles U(0, 2 pi); b > 2: Cayley
    parameters N(0, theta_scale^2)), then one QR fallback per radix that is
    not a power of two, in stage order."""
    rng = _rng(seed)
    radices = tuple(int(b) for b in radices)
    d = int(np.prod(radices))
    x = gaussian_rows_with_outliers(rng, rows, d, outlier_count(d), outlier_scale)
    parts = []
    for b in radices:
        nb = d // b
        if b == 2:
            parts.append(rng.uniform(0.0, 2.0 * math.pi, size=nb))
        else:
            parts.append(rng.normal(0.0, theta_scale, size=nb * (b * (b - 1) // 2)))
    theta = np.concatenate(parts).astype(np.float32)
    fallbacks = [random_orthogonal_f32(rng, b) for b in radices if b & (b - 1)]
    return HarpInputs(x=np.ascontiguousarray(x, dtype=np.float32), radices=radices, theta=theta,
                      fallbacks=fallbacks, d=d, rows=rows)


# Two's-complement nibble patterns of the int4 codes -7..7 (pattern 0x8, i.e. -8,
# is never used by the symmetric quantizer).
_NIBBLES = np.array([0, 1, 2, 3, 4, 5, 6, 7, 9, 10, 11, 12, 13, 14, 15], dtype=np.uint8)


def random_packed_codes(rng: np.random.Generator, rows: int, k: int) -> np.ndarray:
    """uint8 [rows][k/2]: each byte holds two int4 codes drawn uniformly from
    -7..7 (low nibble = even k, high nibble = odd k, two's complement).
    Draw order: low nibbles [rows][k/2], then high nibbles."""
    lo = _NIBBLES[rng.integers(0, 15, size=(rows, k // 2))]
    hi = _NIBBLES[rng.integers(0, 15, size=(rows, k // 2))]
    return (lo | (hi << 4)).astype(np.uint8)


def random_scales_f16(rng: np.random.Generator, rows: int, groups: int,
                      lo: float = 0.001, hi: float = 0.05) -> np.ndarray:
    return rng.uniform(lo, hi, size=(rows, groups)).astype(np.float16)


@dataclass
class GemmInputs:
    a_codes: np.ndarray    # uint8 [M][K/2]
    a_scales: np.ndarray   # fp16 [M][K/G]
    w_codes: np.ndarray    # uint8 [N][K/2]
    w_scales: np.ndarray   # fp16 [N][K/G]
    M: int
    N: int
    K: int
    group: int


def gemm_inputs(M: int = 4096, N: int = 4096, K: int = 4096, group: int = 128,
                seed: int = SEED_GEMM) -> GemmInputs:
    """Draw order: W codes, W scales, A codes, A scales (W first, so the weight
    operand is the same for every M)."""
    rng = _rng(seed)
    w_codes = random_packed_codes(rng, N, K)
    w_scales = random_scales_f16(rng, N, K // group)
    a_codes = random_packed_codes(rng, M, K)
    a_scales = random_scales_f16(rng, M, K // group)
    return GemmInputs(a_codes, a_scales, w_codes, w_scales, M, N, K, group)


@dataclass
class GemmW4A8Inputs:
    a_codes: np.ndarray    # int8 [M][K], one code per element in -127..127
    a_scales: np.ndarray   # fp16 [M][K/G]
    w_codes: np.ndarray    # uint8 [N][K/2]
    w_scales: np.ndarray   # fp16 [N][K/G]
    M: int
    N: int
    K: int
    group: int


def gemm_w4a8_inputs(M: int = 4096, N: int = 4096, K: int = 4096, group: int = 128,
                     seed: int = SEED_GEMM) -> GemmW4A8Inputs:
    """Draw order: W codes, W scales (the same draws as gemm_inputs, so the
    weight operand matches the W4A4 workload), then A int8 codes uniform in
    -127..127, then A scales."""
    rng = _rng(seed)
    w_codes = random_packed_codes(rng, N, K)
    w_scales = random_scales_f16(rng, N, K // group)
    a_codes = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    a_scales = random_scales_f16(rng, M, K // group, 0.0001, 0.005)
    return GemmW4A8Inputs(a_codes, a_scales, w_codes, w_scales, M, N, K, group)


SEED_GEMM8 = 7


@dataclass
class GemmI8Inputs:
    a_codes: np.ndarray    # int8 [M][K], one code per element
    a_scales: np.ndarray   # fp16 [M][K/G]
    w_codes: np.ndarray    # int8 [N][K]
    w_scales: np.ndarray   # fp16 [N][K/G]
    M: int
    N: int
    K: int
    group: int


def gemm_i8_inputs(M: int = 4096, N: int = 4096, K: int = 4096, group: int = 128,
                   seed: int = SEED_GEMM8, code_max: int = 7) -> GemmI8Inputs:
    """GEMM operands with the codes held one per byte.  code_max = 7: the W4A4
    workload (codes uniform in -7..7, fp16 scales U(0.001, 0.05)) for an int8
    MAC; code_max = 127: W8A8.  Draw order: W codes, W scales, A codes, A
    scales."""
    rng = _rng(seed)
    w_codes = rng.integers(-code_max, code_max + 1, size=(N, K)).astype(np.int8)
    w_scales = random_scales_f16(rng, N, K // group)
    a_codes = rng.integers(-code_max, code_max + 1, size=(M, K)).astype(np.int8)
    a_scales = random_scales_f16(rng, M, K // group)
    return GemmI8Inputs(a_codes, a_scales, w_codes, w_scales, M, N, K, group)


@dataclass
class ProbeInputs:
    a: np.ndarray          # fp32 [M][K] activations with outlier channels
    b: np.ndarray          # fp32 [K][N] weights
    signs: np.ndarray      # int8 [K]


def probe_inputs(seed: int = SEED_PROBE, M: int = 16, K: int = 2048, N: int = 512,
                 n_outliers: int = 8, outlier_scale: float = 20.0) -> ProbeInputs:
    """Draw order: signs [K], outlier channels, A [M][K], B [K][N]."""
    rng = _rng(seed)
    signs = sign_vector(rng, K)
    a = gaussian_rows_with_outliers(rng, M, K, n_outliers, outlier_scale)
    b = rng.standard_normal(size=(K, N), dtype=np.float32)
    return ProbeInputs(a=a, b=b, signs=signs)
