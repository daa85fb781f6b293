"""CPU oracle for fine-grained FP8 (1x128 / 128x128, E4M3) quantisation and the
block-scaled FP8 GEMM with per-128-K-chunk promotion into FP32.

This package is TEST INFRASTRUCTURE. Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it. It shares no code with the HIP
library (no common helpers, tables or constants) and imports nothing from it.

Everything here is plain, slow and written to be checked by eye against the
pages it follows:

* DeepSeek-V3 technical report, Chinese translation, chapter 3 "Infrastructure"
  (section 3.3 FP8 training; 3.3.1 mixed-precision framework and Figure 6;
  3.3.2 "fine-grained quantization", "increasing accumulation precision",
  "mantissa over exponents", "online quantization" and Figure 7).
* The tech note "DeepSeek-V3 FP8 dynamic quantisation" (Figure 7 walk-through:
  the "fine-grained quantization" implementation formulas and the
  "increasing accumulation precision" steps).
* The "parallelism summary" page, FP8 part (floating-point format table and
  the resolution bullets: e4m3 has 7 values inside [1, 2], e5m2 has 3).

Modules:
    e4m3   -- the E4M3 (OCP E4M3FN) codec: decode, round-to-nearest-even encode
              with saturation, and a brute-force nearest-value encoder.
    quant  -- online per-tile absmax, scale s = absmax / 448, cast to E4M3.
    gemm   -- per-128-K-chunk FP8 products summed exactly in fp64, rescaled by
              s_a * s_b and accumulated into fp32; the bf16 epilogue.

Parity status of each function is stated in its docstring ("pinned by ...").
The GPU's MFMA-internal summation order and its exact output bits are not
pinned by anything on the pages: the GEMM is compared within a tolerance.
"""

from . import e4m3, quant, gemm  # noqa: F401
