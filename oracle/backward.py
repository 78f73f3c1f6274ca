"""RMSNorm and SiLU-multiply backward from the saved NVFP4 state (oracle).

PACT's backward for these operators rebuilds its inputs in FP32 from the
NVFP4 copies saved in forward and writes BF16 gradients (Appendix Table 7,
rows "RMSNorm" and "SiLU-multiply", backward column; RMSNorm's also reduces
over the row).  The exact value of
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

Pinned FP32 sequences (reading D14).  So that the BF16 gradients, and the
NVFP4 copies the quantize-on-emit kernels make of them, are reproducible bit
for bit, the kernels evaluate these formulas in a fixed FP32 sequence, every
operation rounded to nearest:
    sigma = 1 / (1 + E(-a^))            (E: the pinned exponential of fused.py)
    dgate = ((dh * b^) * sigma) * (1 + a^ * (1 - sigma)),  dup = (dh * a^) * sigma
    S = sum_j dy_j y^_j exactly, rounded once to float64;  mean = fp32(S / H)
    dx = rstd * ((g * dy) - ((y^ / g) * mean))
each rounded to BF16 (RNE).  ``*_f32`` below are those sequences in numpy
float32; the float64 functions above are the exact values they approximate.
Residual gradients accumulate in BF16 (Table 7 row "Residuals"):
out = bf16(fp32(dx) + resid) with dx already BF16.
"""

from __future__ import annotations

import math

import numpy as np

from .fused import exp_f32
from .nvfp4 import NVFP4, dequantize, quantize
from .tolerance import bf16_rne


def rmsnorm_bwd(yq: NVFP4, rstd, g, dy):
    return rmsnorm_bwd_values(dequantize(yq), rstd, g, dy)


def rmsnorm_bwd_values(yh, rstd, g, dy):
    """float64 RMSNorm input gradient and its cancellation magnitude from the
    reconstructed output values yh (any format's dequantization)."""
    yh = np.asarray(yh, dtype=np.float64)
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
    return silu_mul_bwd_values(dequantize(aq), dequantize(bq), dh)


def silu_mul_bwd_values(ah, bh, dh):
    """float64 SiLU-multiply gradients and cancellation magnitudes from the
    reconstructed gate and up values (any format's dequantization)."""
    ah = np.asarray(ah, dtype=np.float64)
    bh = np.asarray(bh, dtype=np.float64)
    dh = np.asarray(dh, dtype=np.float64)
    sig = _sigmoid(ah)
    da = dh * bh * sig * (1.0 + ah * (1.0 - sig))
    db = dh * ah * sig
    cancel_da = np.abs(dh * bh * sig) * (1.0 + np.abs(ah) * (1.0 - sig))
    cancel_db = np.abs(db)
    return da, db, cancel_da, cancel_db


def to_bf16_f32(x) -> np.ndarray:
    """float32 values rounded to the nearest BF16 value (ties to even), as float32."""
    return bf16_rne(np.asarray(x, dtype=np.float32).astype(np.float64)).astype(np.float32)


def silu_mul_bwd_f32(aq: NVFP4, bq: NVFP4, dh):
    """(dgate, dup) as BF16 values (float32) from the pinned FP32 sequence."""
    return silu_mul_bwd_f32_values(dequantize(aq), dequantize(bq), dh)


def silu_mul_bwd_f32_values(ah, bh, dh):
    """The pinned FP32 sequence on reconstructed gate/up values (exact in FP32)."""
    a = np.asarray(ah, dtype=np.float64).astype(np.float32)      # exact: short-mantissa values
    b = np.asarray(bh, dtype=np.float64).astype(np.float32)
    d = np.asarray(dh, dtype=np.float32)
    one = np.float32(1.0)
    with np.errstate(over="ignore"):
        sig = one / (one + exp_f32(-a))
    da = ((d * b) * sig) * (one + a * (one - sig))
    db = (d * a) * sig
    return to_bf16_f32(da), to_bf16_f32(db)


def silu_mul_bwd_quant(aq: NVFP4, bq: NVFP4, dh):
    """(dgate, dup, Q(dgate), Q(dup)): the BF16 gradients and their NVFP4 copies."""
    da, db = silu_mul_bwd_f32(aq, bq, dh)
    return da, db, quantize(da.astype(np.float64)), quantize(db.astype(np.float64))


def rmsnorm_mean_f32(yq: NVFP4, dy) -> np.ndarray:
    """Per-row fp32(S / H) with S = sum_j dy_j y^_j rounded once to float64."""
    return rmsnorm_mean_f32_values(dequantize(yq), dy)


def rmsnorm_mean_f32_values(yh, dy) -> np.ndarray:
    y = np.asarray(yh, dtype=np.float64)
    d = np.asarray(dy, dtype=np.float32).astype(np.float64)
    prod = d * y                               # exact: 8 + 6 significant bits
    S = np.array([math.fsum(row) for row in prod], dtype=np.float64)
    return (S / np.float64(y.shape[1])).astype(np.float32)


def rmsnorm_bwd_f32(yq: NVFP4, rstd, g, dy) -> np.ndarray:
    """dx as BF16 values (float32) from the pinned FP32 sequence."""
    return rmsnorm_bwd_f32_values(dequantize(yq), rstd, g, dy)


def rmsnorm_bwd_f32_values(yh, rstd, g, dy) -> np.ndarray:
    y = np.asarray(yh, dtype=np.float64).astype(np.float32)
    d = np.asarray(dy, dtype=np.float32)
    gg = np.asarray(g, dtype=np.float32)[None, :]
    rs = np.asarray(rstd, dtype=np.float32)[:, None]
    mean = rmsnorm_mean_f32_values(yh, dy)[:, None]
    dx = rs * ((gg * d) - ((y / gg) * mean))
    return to_bf16_f32(dx)


def residual_add_bf16(dx_bf16, resid) -> np.ndarray:
    """bf16(fp32(dx) + resid) for BF16 operands given as float32 values."""
    return to_bf16_f32(np.asarray(dx_bf16, dtype=np.float32) + np.asarray(resid, dtype=np.float32))


def rmsnorm_bwd_residual(yq: NVFP4, rstd, g, dy, resid=None):
    """(out, Q(out)) with out = bf16(rmsnorm_bwd) [+ resid in BF16]."""
    dx = rmsnorm_bwd_f32(yq, rstd, g, dy)
    out = dx if resid is None else residual_add_bf16(dx, resid)
    return out, quantize(out.astype(np.float64))
