"""RMSNorm and SiLU-multiply backward from the saved NVFP4 state (oracle).

PACT's backward for these operators reconstructs in FP32 from the NVFP4
state kept in forward and emits BF16 gradients (Appendix Table 7, rows
"RMSNorm": FP32 reconstruction and reduction, BF16 gradient; "SiLU-multiply":
FP32 reconstruction and derivatives, BF16 gradients).  The exact value of
such a gradient is the textbook derivative evaluated at the reconstructed
inputs, which is what these functions return, in float64.

RMSNorm.  Forward y = x * rstd * g with rstd = (mean(x^2) + eps)^(-1/2); the
saved state is y_q = Q(y) and rstd.  With y^ = deq(y_q):
    dx_i = rstd * (g_i dy_i - (y^_i / g_i) * (1/K) sum_j dy_j y^_j)
(the gain is frozen: no gain gradient).

SiLU-multiply.  Forward h = silu(a) * b; saved a_q = Q(a), b_q = Q(b).  With
a^ = deq(a_q), b^ = deq(b_q) and sigma = 1 / (1 + e^(-a^)):
    da = dh * b^ * sigma * (1 + a^ (1 - sigma)),   db = dh * a^ * sigma.

Each function also returns the summed magnitude of the terms that cancel,
which the acceptance bound uses.
"""

from __future__ import annotations

import numpy as np

from .nvfp4 import NVFP4, dequantize


def rmsnorm_bwd(yq: NVFP4, rstd, g, dy):
    yh = dequantize(yq)
    rstd = np.asarray(rstd, dtype=np.float64)[:, None]
    g = np.asarray(g, dtype=np.float64)[None, :]
    dy = np.asarray(dy, dtype=np.float64)
    K = yh.shape[1]
    xh = yh / g
    mean_dot = (dy * yh).sum(axis=1, keepdims=True) / K
    mean_abs = np.abs(dy * yh).sum(axis=1, keepdims=True) / K
    dx = rstd * (g * dy - xh * mean_dot)
    cancel = rstd * (np.abs(g * dy) + np.abs(xh) * mean_abs)
    return dx, cancel


def _sigmoid(x):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def silu_mul_bwd(aq: NVFP4, bq: NVFP4, dh):
    ah = dequantize(aq)
    bh = dequantize(bq)
    dh = np.asarray(dh, dtype=np.float64)
    sig = _sigmoid(ah)
    da = dh * bh * sig * (1.0 + ah * (1.0 - sig))
    db = dh * ah * sig
    cancel_da = np.abs(dh * bh * sig) * (1.0 + np.abs(ah) * (1.0 - sig))
    cancel_db = np.abs(db)
    return da, db, cancel_da, cancel_db
