"""MXFP4 tensor format and its GEMM (oracle).  TEST INFRASTRUCTURE ONLY.

Format (PACT, Appendix Table 6, MXFP4 column): 32-element blocks along the
contraction axis, E2M1 elements, one E8M0 scale per block, 4.25 bits per
element, and no other scale.  The pages do not give the rule that picks a
block's scale; the reading taken is the OCP Microscaling (MX) one:

* E8M0 is an 8-bit biased exponent: byte b is the value 2**(b - 127),
  b = 255 is NaN (never produced).
* A block's shared exponent is ``e = floor(log2(amax)) - 2`` (2 is the
  exponent of the largest E2M1 value, 6 = 1.5 * 2**2), clamped to
  [-127, 127]; an all-zero block takes e = -127.  The scale byte is e + 127.
* Element code: round-to-nearest-even of ``|x| / 2**e`` onto the E2M1
  magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even code, saturating
  at 6 (``|x| / 2**e`` is below 8, so only (6, 8) saturates); the sign bit of
  ``x`` is kept (-0 encodes as 0x8).
* Layout: codes [R][C/2] bytes with element 2j in the low nibble of byte j
  (as for NVFP4); scales [R][C/32] bytes (the E8M0 bit pattern).

``|x| / 2**e`` is exact in float64 and the E2M1 midpoints are exact, so every
decision is an exact comparison.  The GEMM of two MXFP4 operands is the
float64 product of their dequantized values, as for NVFP4.
"""

from __future__ import annotations

import dataclasses

import numpy as np

from .nvfp4 import E2M1_ALL, e2m1_round_mag, unpack_codes

BLOCK = 32
E2M1_EMAX = 2          # exponent of 6 = 1.5 * 2**2


def e8m0_value(byte: int) -> float:
    """Value of an E8M0 scale byte: 2**(byte - 127); 255 is NaN."""
    if byte == 255:
        return float("nan")
    return float(np.ldexp(1.0, int(byte) - 127))


@dataclasses.dataclass
class MXFP4:
    """MXFP4 tensor of logical shape [rows x cols]."""
    codes: np.ndarray    # uint8 [rows, cols/2]
    scales: np.ndarray   # uint8 [rows, cols/32]

    @property
    def rows(self) -> int:
        return self.codes.shape[0]

    @property
    def cols(self) -> int:
        return self.codes.shape[1] * 2


def storage_bytes(rows: int, cols: int) -> int:
    """Bytes of one MXFP4 tensor: 4.25 bits per element."""
    return rows * cols // 2 + rows * cols // BLOCK


def shared_exponent(amax: np.ndarray) -> np.ndarray:
    """floor(log2(amax)) - 2 clamped to [-127, 127]; -127 where amax == 0 (exact, via frexp)."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)                      # amax = m * 2**ex, m in [0.5, 1): floor(log2) = ex - 1
    e = ex.astype(np.int64) - 1 - E2M1_EMAX
    e = np.where(amax > 0, e, -127)
    return np.clip(e, -127, 127)


def quantize(x, transpose: bool = False) -> MXFP4:
    """Quantize a real matrix X [R x C] (C % 32 == 0) to MXFP4 (X^T with ``transpose``)."""
    x = np.asarray(x, dtype=np.float64)
    if transpose:
        x = x.T
    if x.ndim != 2 or x.shape[1] % BLOCK != 0:
        raise ValueError("quantize expects [rows x cols] with cols % 32 == 0")
    R, C = x.shape
    nb = C // BLOCK
    blk = np.abs(x).reshape(R, nb, BLOCK)
    e = shared_exponent(blk.max(axis=2) if C else np.zeros((R, 0)))       # [R, nb]
    v = blk * np.ldexp(1.0, -e)[:, :, None]                               # |x| / 2**e, exact
    mu = e2m1_round_mag(v, np.ones_like(v))
    sign = np.signbit(x).reshape(R, nb, BLOCK).astype(np.int64)
    code = ((sign << 3) | mu).reshape(R, C)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return MXFP4(packed, (e + 127).astype(np.uint8))


def dequantize(q: MXFP4) -> np.ndarray:
    """Exact real values of an MXFP4 tensor, float64 [R, C]."""
    code = unpack_codes(q.codes)
    R, C = code.shape
    val = E2M1_ALL[code].reshape(R, C // BLOCK, BLOCK)
    s = np.ldexp(1.0, np.asarray(q.scales, dtype=np.int64) - 127)[:, :, None]
    return (val * s).reshape(R, C)


def weight_layouts(w):
    """(W_fwd, W_bwd) = (Q(W), Q(W^T)) in MXFP4 for a weight W [N x K] given as real values."""
    w = np.asarray(w, dtype=np.float64)
    return quantize(w), quantize(w, transpose=True)


def gemm_nt(a: MXFP4, b: MXFP4):
    """(C, |A||B|^T) for C = deq(a) @ deq(b)^T in float64 (forward and input gradient alike)."""
    da = dequantize(a)
    db = dequantize(b)
    return da @ db.T, np.abs(da) @ np.abs(db).T


def rmsnorm_quant(x, g, eps: float):
    """RMSNorm fused with MXFP4 quantization: (Q_mx(y), rstd, y) with y the
    RMSNorm output in the same pinned FP32 sequence as the NVFP4 path's
    (fused.rmsnorm_stats: exact sum of squares rounded once to float64,
    ms = fp32(S / K), v = ms + eps, rstd = 1 / sqrt(v), y = (x * rstd) * g),
    then the MXFP4 quantizer above.  Appendix Table 7 row "RMSNorm" with the
    Table 6 MXFP4 format in place of NVFP4."""
    from .fused import rmsnorm_stats
    x = np.asarray(x, dtype=np.float32)
    g = np.asarray(g, dtype=np.float32)
    rstd = rmsnorm_stats(x, eps)
    y = ((x * rstd[:, None]) * g[None, :]).astype(np.float32)
    return quantize(y.astype(np.float64)), rstd, y


def silu_mul_quant(a, b):
    """SiLU-multiply fused with MXFP4 quantization: (Q_mx(h), Q_mx(a), Q_mx(b), h)
    with h = (a * sigma(a)) * b in the pinned FP32 sequence of the NVFP4 path
    (fused.silu_f32).  Appendix Table 7 row "SiLU-multiply" with the Table 6
    MXFP4 format."""
    from .fused import silu_f32
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    h = (silu_f32(a) * b).astype(np.float32)
    return (quantize(h.astype(np.float64)), quantize(a.astype(np.float64)), quantize(b.astype(np.float64)), h)


def silu_mul_bwd_quant(aq: MXFP4, bq: MXFP4, dh):
    """SiLU-multiply backward from an MXFP4 state with MXFP4 copies:
    (dgate, dup, Q_mx(dgate), Q_mx(dup)).  The BF16 gradients follow the NVFP4
    path's pinned FP32 sequence (backward.silu_mul_bwd_f32_values) on the
    dequantized MXFP4 gate and up values.  Appendix Table 7 row
    "SiLU-multiply" with the Table 6 MXFP4 format."""
    from .backward import silu_mul_bwd_f32_values
    da, db = silu_mul_bwd_f32_values(dequantize(aq), dequantize(bq), dh)
    return da, db, quantize(da.astype(np.float64)), quantize(db.astype(np.float64))


def rmsnorm_bwd_residual(yq: MXFP4, rstd, g, dy, resid=None):
    """RMSNorm backward from an MXFP4 state (+ BF16 residual gradient) with an
    MXFP4 copy: (out, Q_mx(out)), out = bf16(bf16(dx) + resid), dx in the
    NVFP4 path's pinned FP32 sequence (backward.rmsnorm_bwd_f32_values) on the
    dequantized MXFP4 values.  Appendix Table 7 rows "RMSNorm" and "Residuals"
    with the Table 6 MXFP4 format."""
    from .backward import residual_add_bf16, rmsnorm_bwd_f32_values
    dx = rmsnorm_bwd_f32_values(dequantize(yq), rstd, g, dy)
    out = dx if resid is None else residual_add_bf16(dx, resid)
    return out, quantize(out.astype(np.float64))
