"""NVFP4 tensor format: value sets, quantization and dequantization (oracle).

Format (PACT, Appendix Table 6, NVFP4 column): 16-element blocks along the
contraction axis, E2M1 elements, one E4M3 scale per block, 4.50 bits per
element.  The pages fix only these parameters; the readings taken where they
are silent are:

* Row scale.  Every row also carries one power-of-two FP32 scale
  ``r = 2**e``, with ``e`` the smallest integer such that the row's largest
  magnitude ``A`` satisfies ``A <= 6 * 448 * 2**e``; ``e`` is clamped to
  [-126, 127] and is 0 for an all-zero row.  It keeps block scales of
  small-magnitude tensors (weights, output gradients) out of the E4M3
  subnormal range, costs 32 bits per row on top of Table 6's 4.50 bits per
  element, and is the only second-level scale.
* E4M3 is the OCP "FN" variant: bias 7, no infinities, 0x7F/0xFF NaN,
  largest finite 448, subnormals m * 2**-9.
* Block scale ``s = RNE_E4M3(amax_block / (6 r))``, ties to the even code,
  saturating at 448; a scale of zero is allowed.
* Element code: round-to-nearest-even of ``|x| / (s r)`` onto the E2M1
  magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even code, saturating
  at 6; the sign bit of ``x`` is kept (so -0 encodes as 0x8); every
  magnitude is 0 in a block whose scale is 0.
* Layout: codes [R][C/2] bytes with element 2j in the low nibble of byte j;
  scales [R][C/16] bytes (the E4M3 bit pattern); row scales float32 [R].

All decisions are taken with exact comparisons: ``|x| / r`` is exact in
float64 (``r`` is a power of two), and every threshold (a midpoint times a
scale) has at most 7 significant bits, so it too is exact in float64.

Recipe variant with a conventional FP32 tensor scale (the pages leave the
second-level scale open; this is the usual two-level reading, with every
rounding fixed so that the result is unique): for a tensor maximum ``amax``
(an FP32 value), the stored scale is ``S = RN32(amax / 2688)`` raised to
2**-126 if smaller (``S = 1`` when amax is 0), the encoding multiplier is
``R = RN32(1 / S)``, and every element's scaled magnitude is the FP32 product
``u = RN32(|x| * R)``.  Block scale and element code then follow the rules
above on ``u`` in place of ``|x| / r`` (``s = RNE_E4M3(max u / 6)``, code =
``RNE_E2M1(u / s)``), and every row's stored scale is ``S``.  ``u`` is an
FP32 number, so the decisions are again exact comparisons in float64.
"""

from __future__ import annotations

import dataclasses
import numpy as np

BLOCK = 16
E2M1_MAX = 6.0
E4M3_MAX = 448.0


# ---------------------------------------------------------------------------
# Value sets, derived from the bit-field definitions
# ---------------------------------------------------------------------------

def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code: 1 sign, 2 exponent (bias 1), 1 mantissa bit."""
    s = -1.0 if (code >> 3) & 1 else 1.0
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        return s * (m / 2.0)            # subnormal: 0.m * 2**(1-1)
    return s * (1.0 + m / 2.0) * 2.0 ** (e - 1)


def e4m3fn_value(code: int) -> float:
    """Value of an 8-bit E4M3FN code: 1 sign, 4 exponent (bias 7), 3 mantissa bits."""
    s = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> 3) & 15
    m = code & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** (1 - 7)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E2M1_MAG = np.array([e2m1_value(c) for c in range(8)], dtype=np.float64)
E2M1_ALL = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E4M3_POS = np.array([e4m3fn_value(c) for c in range(0x7F)], dtype=np.float64)  # codes 0..126
E4M3_MID = (E4M3_POS[:-1] + E4M3_POS[1:]) / 2.0          # exact (<= 5 significant bits)
E2M1_MID = (E2M1_MAG[:-1] + E2M1_MAG[1:]) / 2.0          # 0.25 .75 1.25 1.75 2.5 3.5 5


@dataclasses.dataclass
class NVFP4:
    """Canonical NVFP4 tensor of logical shape [rows x cols]."""
    codes: np.ndarray    # uint8 [rows, cols/2]
    scales: np.ndarray   # uint8 [rows, cols/16]
    rscale: np.ndarray   # float32 [rows]

    @property
    def rows(self) -> int:
        return self.codes.shape[0]

    @property
    def cols(self) -> int:
        return self.codes.shape[1] * 2

    def nbytes(self) -> int:
        return self.codes.nbytes + self.scales.nbytes + self.rscale.nbytes


def storage_bytes(rows: int, cols: int) -> int:
    """Bytes of one NVFP4 tensor: 4.5 bits/element plus a 4-byte row scale per row."""
    return rows * cols // 2 + rows * cols // BLOCK + 4 * rows


# ---------------------------------------------------------------------------
# Quantization
# ---------------------------------------------------------------------------

def row_exponent(amax: np.ndarray) -> np.ndarray:
    """Smallest integer e with amax <= 2688 * 2**e, clamped to [-126, 127]; 0 if amax == 0."""
    amax = np.asarray(amax, dtype=np.float64)
    lim = E2M1_MAX * E4M3_MAX                                  # 2688
    e = np.zeros(amax.shape, dtype=np.int64)
    nz = amax > 0
    with np.errstate(divide="ignore"):
        guess = np.ceil(np.log2(np.where(nz, amax, 1.0) / lim)).astype(np.int64)
    guess = np.clip(guess, -1100, 1100)
    # fix the estimate with exact comparisons (lim * 2**e is exact in float64)
    for _ in range(3):
        too_small = nz & (amax > np.ldexp(lim, guess))
        guess = guess + too_small
        too_big = nz & (amax <= np.ldexp(lim, guess - 1))
        guess = guess - too_big
    e[nz] = guess[nz]
    return np.clip(e, -126, 127)


def e4m3_round_code(t_times6: np.ndarray) -> np.ndarray:
    """E4M3FN code of RNE(t), given 6*t exactly; saturates at 448 (code 0x7E).

    ``idx`` counts the midpoints strictly below t; at an exact midpoint
    between codes j and j+1 the even code is chosen, i.e. j+1 when j is odd.
    """
    thr = 6.0 * E4M3_MID                                      # exact
    idx = np.searchsorted(thr, t_times6, side="left")
    tie = np.zeros(idx.shape, dtype=bool)
    inr = idx < thr.size
    tie[inr] = t_times6[inr] == thr[idx[inr]]
    idx = idx + (tie & (idx % 2 == 1))
    return idx.astype(np.uint8)


def e2m1_round_mag(v_num: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """E2M1 magnitude code of RNE(v_num / scale), ties to even code, saturating at 6.

    Works on exact comparisons ``v_num > m_q * scale``.
    """
    mu = np.zeros(v_num.shape, dtype=np.int64)
    for q, m in enumerate(E2M1_MID):
        thr = m * scale                                       # exact
        mu += v_num > thr
        if q % 2 == 1:                                        # tie between odd q and even q+1
            mu += v_num == thr
    return mu


def e4m3_round_up_code(t_times6: np.ndarray) -> np.ndarray:
    """E4M3FN code of the smallest E4M3 value >= t, given 6*t exactly (t <= 448)."""
    return np.searchsorted(6.0 * E4M3_POS, t_times6, side="left").astype(np.uint8)


def tensor_scale_fp32(amax):
    """(S, R) of the FP32 tensor-scale recipe for a tensor maximum ``amax``
    (an FP32 value >= 0): S = RN32(amax / 2688), at least 2**-126, or 1 when
    amax == 0; R = RN32(1 / S).  numpy's float32 division is IEEE division
    (correctly rounded to nearest even)."""
    a = np.float32(amax)
    if not np.isfinite(a) or a < 0:
        raise ValueError("amax must be finite and >= 0")
    if a == 0:
        return np.float32(1.0), np.float32(1.0)
    s = np.float32(a / np.float32(E2M1_MAX * E4M3_MAX))
    s = max(s, np.float32(2.0 ** -126))
    return np.float32(s), np.float32(np.float32(1.0) / s)


def quantize(x, transpose: bool = False, round_up: bool = False, tensor_amax=None,
             fp32_tensor_scale: bool = False) -> NVFP4:
    """Quantize a real matrix X [R x C] (C % 16 == 0) to canonical NVFP4.

    With ``transpose`` the input is X^T of the given matrix: rows of the result
    are columns of ``x``, blocked along the other axis.

    Recipe variants (reading D15): ``round_up`` takes each block scale as the
    smallest E4M3 value >= blockmax / (6 r) instead of the nearest (then no
    element saturates); ``tensor_amax`` (a real >= max |x|, or "auto" for
    max |x|) gives every row the one power-of-two scale the row rule assigns to
    that maximum.  With ``fp32_tensor_scale`` (and ``tensor_amax``) the
    tensor scale is instead the FP32 value S of ``tensor_scale_fp32`` and the
    elements are scaled by the FP32 multiplier R (module docstring); ``x``
    must then hold FP32-representable values.
    """
    x = np.asarray(x, dtype=np.float64)
    if transpose:
        x = x.T
    if x.ndim != 2 or x.shape[1] % BLOCK != 0:
        raise ValueError("quantize expects [rows x cols] with cols % 16 == 0")
    R, C = x.shape
    ax = np.abs(x)
    if fp32_tensor_scale and tensor_amax is None:
        raise ValueError("fp32_tensor_scale needs tensor_amax")
    if tensor_amax is None:
        e = row_exponent(ax.max(axis=1) if C else np.zeros(R))
    else:
        ta = (ax.max() if ax.size else 0.0) if isinstance(tensor_amax, str) else float(tensor_amax)
        e = np.full(R, int(row_exponent(np.array(ta))), dtype=np.int64)
    if fp32_tensor_scale:
        ax32 = ax.astype(np.float32)
        if not np.array_equal(ax32.astype(np.float64), ax):
            raise ValueError("fp32_tensor_scale needs FP32-representable inputs")
        S, Rm = tensor_scale_fp32(ta)
        xr = (ax32 * Rm).astype(np.float64)                   # u = RN32(|x| * R), exact in float64
    else:
        inv_r = np.ldexp(1.0, -e)[:, None]
        xr = ax * inv_r                                       # |x| / r, exact
    blk = xr.reshape(R, C // BLOCK, BLOCK)
    bmax = blk.max(axis=2) if C else np.zeros((R, 0))
    # compare against 6*mid (or 6*value) exactly
    scode = e4m3_round_up_code(bmax) if round_up else e4m3_round_code(bmax)
    s = E4M3_POS[scode]                                       # [R, C/16]
    mu = e2m1_round_mag(blk, s[:, :, None])
    mu = np.where(s[:, :, None] == 0, 0, mu)
    sign = np.signbit(x).reshape(R, C // BLOCK, BLOCK).astype(np.int64)
    code = (sign << 3) | mu
    code = code.reshape(R, C)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    if fp32_tensor_scale:
        rscale = np.full(R, S, dtype=np.float32)
    else:
        rscale = np.ldexp(np.float32(1.0), e.astype(np.int32)).astype(np.float32)
    return NVFP4(packed, scode.reshape(R, C // BLOCK), rscale)


def unpack_codes(codes: np.ndarray) -> np.ndarray:
    """uint8 [R, C/2] -> int [R, C] 4-bit codes (low nibble = even element)."""
    codes = np.asarray(codes, dtype=np.uint8)
    R, H = codes.shape
    out = np.empty((R, 2 * H), dtype=np.int64)
    out[:, 0::2] = codes & 0xF
    out[:, 1::2] = codes >> 4
    return out


def dequantize(q: NVFP4) -> np.ndarray:
    """Exact real values of an NVFP4 tensor, float64 [R, C]."""
    code = unpack_codes(q.codes)
    R, C = code.shape
    val = E2M1_ALL[code].reshape(R, C // BLOCK, BLOCK)
    s = E4M3_POS[np.asarray(q.scales, dtype=np.int64)][:, :, None]
    r = np.asarray(q.rscale, dtype=np.float64)[:, None, None]
    return (val * s * r).reshape(R, C)


def scale_values(q: NVFP4) -> np.ndarray:
    """Block scale values s [R, C/16] as float64."""
    return E4M3_POS[np.asarray(q.scales, dtype=np.int64)]
