"""Plain CPU oracle for the SVDQuant W4A4 linear layer (test infrastructure only).

This package is the slow, obviously-correct reference that the HIP path is
checked against.  Only the test-suite, the smoke check and the CPU-baseline leg
of the benchmark may import it; the product path never does, and this package
imports nothing from the product path.

What it computes (sources are the web pages the method is described on):

* "SVDQuant W4A4" (vLLM-Omni user guide), section "Checkpoint contract": the
  tensor set ``qweight (N, K/2)`` of packed FP4 pairs, ``wscales (K/16, N)`` in
  float8_e4m3fn, ``proj_down (K, R)``, ``proj_up (N, R)``, ``smooth_factor
  (K,)``, ``wcscales (N,)`` and ``wtscale (1,)``; section "Runtime support":
  BF16 input, an NVFP4 (E2M1 with one e4m3 scale per 16 values) GEMM, then the
  BF16 rank correction.
* "Rotate techniques in quantization and their vLLM implementation" (llx-08
  notes), section 2.1 (rotation maths, x' = x R^T, W' = R W), section 2.2
  (Sylvester Hadamard recursion, orthogonality, symmetry), section 1 (the
  signed/unsigned INT4 absmax quantizer and its worked examples), section 3.1
  (the Hadamard kernel's tests: equality with the dense product, involution).

Modules:

* ``formats``  -- E2M1 and float8_e4m3fn encode/decode, bf16 rounding.
* ``hadamard`` -- block Sylvester fast Walsh-Hadamard transform.
* ``quant``    -- per-16-group FP4 quantizer, activation and weight quantizers,
                  INT4 absmax quantizer of the worked examples.
* ``linear``   -- dequantize-then-matmul composition and the epilogue.
* ``svd``      -- the offline low-rank split of a smoothed weight (top-R SVD,
                  bf16 factors, residual for the 4-bit branch).
* ``mx``       -- the MXFP4 variant (rotate notes, section 3.3, FP-Quant: E2M1
                  in blocks of 32 with one E8M0 power-of-two scale, group-32
                  rotation) with the same epilogue.

Precision: every step whose result decides an integer (a code, a scale byte)
is done in IEEE float32, the precision the GPU kernels take that decision in;
the contraction and epilogue are done in float64 and rounded once to bf16.

Pins (what each function is checked against, in ``tests/test_oracle_*.py``):
formats against torch's float8_e4m3fn conversion and a brute-force nearest
search; the transform against the pages' worked example, a dense Sylvester
matrix built by the recursion, orthogonality and involution; the quantizers
against the pages' INT4 examples, reconstruction bounds and special cases; the
composition against a pure-Python block-scaled triple loop and the
identity-quantizer reduction to the unquantized linear.  Parity unpinned (by
the pages): the conventions the pages leave open -- nibble order, smoothing
direction, scale layout, zero-scale rule, sign of zero -- are fixed readings,
checked only for self-consistency.
"""

from . import formats, hadamard, quant, linear, mx, svd  # noqa: F401
