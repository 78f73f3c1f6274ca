"""CPU oracle for the NVFP4 frozen-projection path.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or execute anything in this package.  The GPU
library never routes through it, and it shares no code with the GPU library:
it is written from the format and precision tables of "PACT: NVFP4 Data-Flow
LoRA Fine-Tuning on Consumer GPUs" (Appendix Table 6, NVFP4 and MXFP4 formats;
Appendix Table 7, precision allocation) and the readings of those tables that the
design notes list.

It is deliberately slow and plain: numpy in float64 for every real-valued
result, exact comparisons (products of short-mantissa values are exact in
float64) for every rounding decision, and numpy float32 only where a reading
pins an FP32 operation sequence (the fused RMSNorm and SiLU-multiply
forward and backward).

Modules
  nvfp4     E2M1 / E4M3 value sets, quantize, dequantize, packing
  mxfp4     the MXFP4 variant (32-element blocks, E8M0 scales) and its GEMM
  gemm      float64 forward and input-gradient GEMMs of dequantized operands
  lora      the BF16 rank-r branch on the dequantized input
  fused     RMSNorm -> quantize and SiLU-multiply -> quantize forward
  backward  RMSNorm and SiLU-multiply backward from the saved NVFP4 state,
            their pinned FP32 sequences, the BF16 residual accumulation and the
            quantize-on-emit compositions
  tolerance the acceptance bounds for floating-point results

Parity status: every function here is pinned by tests in
``tests/test_oracle_*.py`` (closed forms, hand-worked vectors under
``tests/golden/``, exhaustive exact-rational checks, brute force on tiny
shapes, finite differences).  None is "parity unpinned".
"""

from . import nvfp4, mxfp4, gemm, lora, fused, backward, tolerance  # noqa: F401
