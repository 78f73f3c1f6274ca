"""Frozen-projection GEMMs of dequantized NVFP4 operands, in float64 (oracle).

PACT runs every frozen projection as an NVFP4 GEMM that sums in FP32 and
writes BF16, in both directions, each direction over its own cached NVFP4
copy of the weight (Appendix Table 7, row "Frozen projections").  The exact
result of such a GEMM is the product of the dequantized operands, which is
what this module computes:

* forward        Y[m, n]  = sum_k deq(X_q)[m, k] * deq(W_fwd)[n, k]
* input gradient dX[m, k] = sum_n deq(dY_q)[m, n] * deq(W_bwd)[k, n]
* single-layout input gradient (the variant that keeps W_fwd only)
                 dX[m, k] = sum_n deq(dY_q)[m, n] * deq(W_fwd)[n, k]

with W_fwd = Q(W) (blocks along K) and W_bwd = Q(W^T) (blocks along N), both
rounded to nearest from the same BF16 W.  Both are "A [M x Kr] times
B [Nout x Kr]^T", so one function serves both directions.
"""

from __future__ import annotations

import numpy as np

from .nvfp4 import NVFP4, dequantize, quantize


def weight_layouts(w):
    """(W_fwd, W_bwd) = (Q(W), Q(W^T)) for a BF16 weight W [N x K] given as real values."""
    w = np.asarray(w, dtype=np.float64)
    return quantize(w), quantize(w, transpose=True)


def gemm_nt(a: NVFP4, b: NVFP4):
    """(C, |A||B|^T) for C = deq(a) @ deq(b)^T in float64.

    The second result is sum_k |a_k b_k| per output, used by the acceptance bound.
    """
    da = dequantize(a)
    db = dequantize(b)
    return da @ db.T, np.abs(da) @ np.abs(db).T


def gemm_fwd(xq: NVFP4, w_fwd: NVFP4):
    return gemm_nt(xq, w_fwd)


def gemm_dgrad(dyq: NVFP4, w_bwd: NVFP4):
    return gemm_nt(dyq, w_bwd)


def gemm_dgrad_fwd_layout(dyq: NVFP4, w_fwd: NVFP4):
    """Single-layout input gradient: (dX, |dY||W|) for dX = deq(dY_q) @ deq(W_fwd).

    W_fwd = Q(W) [N x K] is the forward layout (blocks along K); the input
    gradient contracts over its rows, so forward and input gradient use the
    same effective weight deq(W_fwd) instead of deq(W_fwd) and deq(W_bwd)^T.
    """
    da = dequantize(dyq)
    dw = dequantize(w_fwd)
    return da @ dw, np.abs(da) @ np.abs(dw)


def gemm_dgrad_multi(segments):
    """Input gradient summed over projections that read one input (PACT,
    Appendix Table 7 row "Frozen projections"; every consumer's dY_i W_i adds
    into the same dX): sum_i deq(dY_i) deq(W_bwd,i)^T in float64, with the sum
    of |a||b| products for the acceptance bound.  ``segments``: list of
    (dY_i NVFP4 [M x N_i], W_bwd,i NVFP4 [K x N_i])."""
    ref, rabs = None, None
    for dyq, wb in segments:
        r, a = gemm_dgrad(dyq, wb)
        ref = r if ref is None else ref + r
        rabs = a if rabs is None else rabs + a
    return ref, rabs

