"""The BF16 rank-r LoRA branch on the dequantized input (oracle).

PACT keeps the adapter path in BF16: its products run in BF16 on the
dequantized NVFP4 input, forward and backward, and backward keeps only that
NVFP4 input and the BF16 adapters (Appendix Table 7, row "LoRA branch";
Figure 3's caption draws the same split).

Readings (the pages give no formulas, rank or scale):
* X~ = deq(X_q) is the reconstructed input; it is exact in BF16.
* T = bf16(X~ A^T) is the branch's intermediate, A [r x K], rounded to BF16
  because it feeds a BF16 GEMM.
* Y = bf16(deq(X_q) deq(W_fwd)^T + s T B^T), B [N x r], one BF16 rounding
  of the FP32 sum; ``s`` (alpha / r) is the caller's.
* Backward, with the BF16 output gradient dY (not its NVFP4 copy):
  dT = bf16(s dY B), dB = bf16(s dY^T T) with T recomputed from X_q,
  dA = bf16(dT^T X~), and the input gradient gains dT A, summed into the
  frozen projection's dgrad output before its single BF16 rounding.
"""

from __future__ import annotations

import numpy as np

from .nvfp4 import NVFP4, dequantize
from .tolerance import bf16_rne, ulp_bf16


def lora_down(xq: NVFP4, a):
    """T = X~ A^T: returns (T_exact float64, T_bf16 float64, sum |X~||A|^T)."""
    xt = dequantize(xq)
    a = np.asarray(a, dtype=np.float64)
    t = xt @ a.T
    return t, bf16_rne(t), np.abs(xt) @ np.abs(a).T


def lora_term(t_bf16, u_rn, scale: float):
    """s * T U where U [r x Nout]; returns (term, s * sum |T||U|, s * sum ulp(T)|U|).

    The third value bounds the effect of a one-ulp difference in any T element.
    """
    t = np.asarray(t_bf16, dtype=np.float64)
    u = np.asarray(u_rn, dtype=np.float64)
    s = float(scale)
    return s * (t @ u), abs(s) * (np.abs(t) @ np.abs(u)), abs(s) * (ulp_bf16(t) @ np.abs(u))


def lora_bwd(xq: NVFP4, a, b, dy, scale: float):
    """Exact-then-rounded adapter gradients.

    Returns a dict with dT, dB, dA (float64 values of the BF16 results) and, for
    the acceptance bounds, the exact values and the absolute-product sums.
    """
    xt = dequantize(xq)
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    s = float(scale)
    t_exact = xt @ a.T
    t = bf16_rne(t_exact)
    dt_exact = s * (dy @ b)
    dt = bf16_rne(dt_exact)
    db_exact = s * (dy.T @ t)
    da_exact = dt.T @ xt
    return {
        "T": t,
        "dT_exact": dt_exact, "dT": dt, "dT_abs": abs(s) * (np.abs(dy) @ np.abs(b)),
        "dB_exact": db_exact, "dB": bf16_rne(db_exact),
        "dB_abs": abs(s) * (np.abs(dy).T @ np.abs(t)),
        "dB_tslack": abs(s) * (np.abs(dy).T @ ulp_bf16(t)),
        "dA_exact": da_exact, "dA": bf16_rne(da_exact),
        "dA_abs": np.abs(dt).T @ np.abs(xt),
        "dA_tslack": ulp_bf16(dt).T @ np.abs(xt),
    }
