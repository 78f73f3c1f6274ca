"""Acceptance bounds for floating-point results (oracle side).

* GEMM outputs (frozen projections: FP32 accumulation, BF16 output, PACT
  Appendix Table 7 row "Frozen projections"):
  ``|y - y_ref| <= ulp_bf16(y_ref) + 1e-5 * sum_k |a_k b_k|``, with ``y_ref``
  the float64 GEMM of the dequantized operands.  A rank-r term adds its own
  share of the same bound, plus the BF16 rounding of the intermediate T that
  the branch's BF16 GEMMs consume (one BF16 ulp of T may legitimately differ
  between an FP32-accumulating kernel and the exact value).
* Gradients of the fused nonlinear kernels (FP32 reconstruction, BF16
  gradients, Table 7 rows "RMSNorm" and "SiLU-multiply"):
  ``2 * ulp_bf16(ref) + 2**-17 * cancel``, where ``cancel`` is the summed
  magnitude of the terms that cancel in the formula, so that an FP32
  evaluation of a result near zero is not rejected for its FP32 rounding.
"""

from __future__ import annotations

import numpy as np


def bf16_rne(x) -> np.ndarray:
    """Round float64 values to the nearest BF16 value (ties to even), as float64.

    Rounds directly from float64 (no intermediate float32 rounding).
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                     # x = m * 2**e, 0.5 <= |m| < 1
    q = np.maximum(e.astype(np.int64) - 8, -133)   # 8 significant bits; subnormal grid 2**-133
    return np.ldexp(np.rint(np.ldexp(x, -q)), q)


def ulp_bf16(x) -> np.ndarray:
    """BF16 unit in the last place at |x|: 2**(max(floor(log2|x|), -126) - 7)."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(x)                     # floor(log2|x|) = e - 1 for x != 0
    fl = np.where(x > 0, e.astype(np.int64) - 1, -126)
    return np.ldexp(1.0, np.maximum(fl, -126) - 7)


def gemm_bound(y_ref, abs_sum, extra=0.0) -> np.ndarray:
    return ulp_bf16(y_ref) + 1e-5 * np.asarray(abs_sum, dtype=np.float64) + extra


def grad_bound(ref, cancel) -> np.ndarray:
    return 2.0 * ulp_bf16(ref) + 2.0 ** -17 * np.asarray(cancel, dtype=np.float64)


def violations(got, ref, bound):
    """Return (count, worst_ratio) of |got - ref| > bound."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    bad = ~(err <= bound)                  # NaN counts as a violation
    ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.inf)
    worst = float(np.nanmax(ratio)) if ratio.size else 0.0
    return int(bad.sum()), worst
