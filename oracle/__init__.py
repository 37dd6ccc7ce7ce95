"""CPU oracle for the rotate / quantize / W4A4 path -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct fp64 implementation (numpy) of what the HIP
path computes.  It shares no code with the HIP library and never imports it.
Only the test suite, the smoke check and the bench's CPU-baseline leg may
import it; the product path must never route through it.

Modules and the passages they follow:

* ``hadamard``     -- explicit Sylvester-Hadamard matrix and the randomized
  Hadamard transform y = H (d * x) / sqrt(n).  "Experiment -- Hadamard rotation
  for int4 (W4A4) accuracy" (Hypothesis, Method); "Llama-3.2-1B-Instruct-
  HadamardSpin-4bits" (How it Works); HARP abstract.
* ``mixed_radix``  -- y = (O kron H_p) D x / sqrt(p) for n = m * p.  HARP
  technical summary (gist.science), sections 2.1-2.2; HARP abstract.
* ``butterfly``    -- HARP's stages of 2x2 blocks Q(theta) G_2 on pairs at
  stride 2^s, then a gather permutation.  HARP technical summary, 2.1-2.2, 2.4.
* ``quant``        -- per-group symmetric absmax quantize / dequantize and the
  int4 nibble packing.  "Experiment -- ..." (Method: per-group symmetric int
  quant -> dequant at any bit width).
* ``gemm``         -- W4A4 GEMM with exact per-group integer sums and fp64
  scale fusion.  "Experiment -- ..." (Hypothesis: the NPU's same-precision MAC
  needs int4 activations; Verdict: per-group work must not be split).
* ``probe``        -- the matmul RMS-error probe (Method; Results, synthetic
  table).
* ``harp``         -- HARP's general processor: mixed-radix stages of dense
  blocks Q(theta) G_b (Givens for b = 2, Cayley map for b > 2).  HARP
  technical summary, sections 2.1-2.2.

Readings of points the pages leave open are stated where they are used.
"""
from . import hadamard, mixed_radix, butterfly, quant, gemm, probe, harp  # noqa: F401
