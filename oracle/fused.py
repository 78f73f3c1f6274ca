"""Fused RMSNorm -> NVFP4 and SiLU-multiply -> NVFP4 forward (oracle).

PACT fuses its nonlinear operators with quantization: RMSNorm takes a BF16
input, normalizes in FP32 and keeps its NVFP4 output plus an FP32 per-token
statistic for backward; SiLU-multiply takes BF16 gate/up inputs, computes in
FP32 and keeps separate NVFP4 copies of gate and up (Appendix Table 7, rows
"RMSNorm" and "SiLU-multiply"; the abstract adds that quantized RMSNorm
outputs are reused and that forward nonlinearities read BF16 inputs).

The NVFP4 codes of a fused kernel depend on every bit of the FP32 value it
quantizes, so the readings below pin the FP32 operation sequence; this module
evaluates it with numpy float32 arithmetic (each operation IEEE
round-to-nearest, no fused multiply-add):

RMSNorm, per row of K elements, for BF16 x, BF16 gain g, FP32 eps:
  S    = sum x_i^2, the exact sum rounded once to float64
  ms   = fp32(S / K)              (float64 division, then rounding to FP32)
  v    = ms + eps                 (FP32)
  rstd = 1 / sqrt(v)              (FP32 correctly rounded sqrt, then division)
  y_i  = (x_i * rstd) * g_i       (FP32)
  outputs Q(y) and rstd; the saved NVFP4 tensor is the projection input.

SiLU-multiply, elementwise for BF16 gate a and up b:
  sigma = 1 / (1 + E(-a)),  silu = a * sigma,  h = silu * b   (FP32)
  outputs Q(h) (the down-projection input), Q(a) and Q(b) (saved for backward)
with E the FP32 exponential below (Cody and Waite's two-constant argument
reduction, then the degree-7 Taylor polynomial of e^r in Horner form, each
reduction and Horner step one fused multiply-add, fma(a, b, c) = RN32(a*b + c)
with a single rounding):
  E(x) = 0 for x < -80; +inf for x > 89; otherwise
  n = rint(x * L2E)  (ties to even),
  r = fma(-n, LN2_LO, fma(-n, LN2_HI, x)),
  p = C7;  p = fma(p, r, C_k)  for k = 6..0,  E = ldexp(p, n)
where L2E = RN32(1/ln 2), LN2_HI = ln 2 rounded to 16 significant bits,
LN2_LO = RN32(ln 2 - LN2_HI) and C_k = RN32(1/k!).  numpy has no FP32 fused
multiply-add; fma32 below evaluates it exactly (the FP32 product is exact in
float64, the float64 sum's rounding error is recovered exactly, and the one
case where rounding twice differs from rounding once, an FP32 midpoint, is
decided by that error).
"""

from __future__ import annotations

import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

from .nvfp4 import quantize


# ---------------------------------------------------------------------------
# Constants of E, derived from ln 2 and 1/k! with exact rational rounding
# ---------------------------------------------------------------------------

def _round_sig(fr: Fraction, bits: int) -> Fraction:
    """Nearest value with `bits` significant bits (ties to even); fr > 0."""
    e = fr.numerator.bit_length() - fr.denominator.bit_length()
    while Fraction(2) ** e > fr:
        e -= 1
    while Fraction(2) ** (e + 1) <= fr:
        e += 1
    q = e - (bits - 1)
    m = fr / (Fraction(2) ** q)
    mi = m.numerator // m.denominator
    rem = m - mi
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and mi % 2 == 1):
        mi += 1
    return mi * Fraction(2) ** q


def _ln2_fraction() -> Fraction:
    getcontext().prec = 60
    return Fraction(Decimal(2).ln())


def _f32(fr: Fraction) -> np.float32:
    v = _round_sig(fr, 24)
    out = np.float32(float(v))           # v has 24 bits: exact in float64 and float32
    assert Fraction(float(out)) == v
    return out


_LN2 = _ln2_fraction()
L2E = _f32(1 / _LN2)
_LN2_HI_FR = _round_sig(_LN2, 16)
LN2_HI = np.float32(float(_LN2_HI_FR))
LN2_LO = _f32(_LN2 - _LN2_HI_FR)
COEF = [np.float32(1.0) if k < 2 else _f32(Fraction(1, math.factorial(k))) for k in range(8)]
EXP_LO = np.float32(-80.0)
EXP_HI = np.float32(89.0)


def fma32(a, b, c) -> np.ndarray:
    """RN32(a*b + c) for float32 a, b, c (finite, result in the FP32 range),
    elementwise: the fused multiply-add with a single rounding to nearest
    even."""
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    c = np.asarray(c, dtype=np.float32)
    p = a.astype(np.float64) * b.astype(np.float64)      # exact: 24 + 24 significant bits
    c64 = c.astype(np.float64)
    s = p + c64                                          # RN64(p + c)
    bb = s - p                                           # two-sum: p + c = s + e exactly
    e = (p - (s - bb)) + (c64 - bb)
    r = s.astype(np.float32)                             # RN32(s)
    # RN32(s) differs from RN32(p + c) only when s is an FP32 midpoint and e
    # pushes the exact sum off it (a midpoint has 25 significant bits, so it
    # is a float64 value the float64 rounding cannot cross)
    d = s - r.astype(np.float64)
    toward = np.where(d > 0, np.float32(np.inf), np.float32(-np.inf))
    nb = np.nextafter(r, toward)
    mid = (d != 0) & (np.abs(d) * 2 == np.abs(nb.astype(np.float64) - r.astype(np.float64)))
    # at a midpoint r is the even neighbour; the exact sum lies on nb's side when e has d's sign
    fix = mid & (e != 0) & (np.sign(e) == np.sign(d))
    return np.where(fix, nb, r).astype(np.float32)


def exp_f32(x) -> np.ndarray:
    """The pinned FP32 exponential E(x), elementwise on float32."""
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        xc = np.clip(x, EXP_LO, EXP_HI)
        t = xc * L2E
        n = np.rint(t)
        r = fma32(-n, LN2_LO, fma32(-n, LN2_HI, xc))
        p = np.full(x.shape, COEF[7], dtype=np.float32)
        for k in range(6, -1, -1):
            p = fma32(p, r, COEF[k])
        out = np.ldexp(p, n.astype(np.int32)).astype(np.float32)
    out = np.where(x < EXP_LO, np.float32(0.0), out)
    out = np.where(x > EXP_HI, np.float32(np.inf), out)
    return out.astype(np.float32)


def silu_f32(a) -> np.ndarray:
    """silu(a) = a * (1 / (1 + E(-a))) in the pinned FP32 sequence."""
    a = np.asarray(a, dtype=np.float32)
    with np.errstate(over="ignore"):
        sig = np.float32(1.0) / (np.float32(1.0) + exp_f32(-a))
        return (a * sig).astype(np.float32)


def silu_mul_quant(a, b):
    """(Q(h), Q(a), Q(b), h) for BF16 gate a and up b given as float32 values."""
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    h = (silu_f32(a) * b).astype(np.float32)
    return quantize(h), quantize(a), quantize(b), h


def rmsnorm_stats(x, eps: float) -> np.ndarray:
    """Per-row rstd of BF16 rows x [M x K] (float32 values)."""
    x = np.asarray(x, dtype=np.float32)
    M, K = x.shape
    xd = x.astype(np.float64)
    sq = xd * xd                               # exact: BF16 squares fit in 16 bits
    S = np.array([math.fsum(row) for row in sq], dtype=np.float64)
    ms = (S / np.float64(K)).astype(np.float32)
    v = ms + np.float32(eps)
    return (np.float32(1.0) / np.sqrt(v)).astype(np.float32)


def rmsnorm_quant(x, g, eps: float):
    """(Q(y), rstd, y) with y = (x * rstd) * g in FP32."""
    x = np.asarray(x, dtype=np.float32)
    g = np.asarray(g, dtype=np.float32)
    rstd = rmsnorm_stats(x, eps)
    y = ((x * rstd[:, None]) * g[None, :]).astype(np.float32)
    return quantize(y), rstd, y
