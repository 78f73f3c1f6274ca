"""Pins of the oracle's pinned-FP32 backward sequences, the BF16 residual
accumulation and the quantize-on-emit compositions.

PACT, Appendix Table 7: RMSNorm and SiLU-multiply backward reconstruct in FP32
from the NVFP4 state and emit BF16 gradients; residual gradients accumulate in
BF16.  The pinned FP32 sequences are checked against the exact (float64)
derivatives they evaluate, the BF16 rounding and the residual add against
exact-rational round-to-nearest-even, the row mean against an exact rational
sum, and closed forms (a = 0, dh = 0, zero residual).
"""

from fractions import Fraction

import numpy as np

from oracle import backward as obwd
from oracle import nvfp4 as onv
from oracle import tolerance as tol
from synth import bf16_round


def _rne_bits(fr: Fraction, sig_bits: int, min_exp: int) -> Fraction:
    """Exact round-to-nearest-even of a rational onto a binary grid with
    sig_bits significant bits and smallest exponent min_exp (subnormals)."""
    if fr == 0:
        return Fraction(0)
    sgn = -1 if fr < 0 else 1
    a = abs(fr)
    e = 0
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    while Fraction(2) ** e > a:
        e -= 1
    q = max(e - (sig_bits - 1), min_exp)
    unit = Fraction(2) ** q
    n = a / unit
    lo = n.numerator // n.denominator
    rem = n - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sgn * lo * unit


def _rne_bf16(fr):
    return _rne_bits(Fraction(fr), 8, -133)


def _rne_f32(fr):
    return _rne_bits(Fraction(fr), 24, -149)


def test_bf16_rounding_matches_exact_rne():
    rng = np.random.default_rng(70)
    x = np.concatenate([rng.standard_normal(300).astype(np.float32),
                        (rng.standard_normal(100) * 2.0 ** -128).astype(np.float32),     # subnormal range
                        # exact ties between BF16 neighbours: (2k+1) * 2^(e-8) with 8-bit k
                        np.array([(2 * k + 1) * 2.0 ** (-8 - s) for k in range(0, 256, 37) for s in (0, 3, 9)],
                                 dtype=np.float32)])
    got = obwd.to_bf16_f32(x)
    for v, g in zip(x, got):
        assert Fraction(float(g)) == _rne_bf16(float(v)), v


def test_residual_add_matches_exact_rounding():
    rng = np.random.default_rng(71)
    a = bf16_round(rng.standard_normal(400).astype(np.float32))
    b = bf16_round((rng.standard_normal(400) * np.exp2(rng.integers(-20, 20, 400))).astype(np.float32))
    out = obwd.residual_add_bf16(a, b)
    for x, y, o in zip(a, b, out):
        want = _rne_bf16(_rne_f32(Fraction(float(x)) + Fraction(float(y))))   # FP32 add, then BF16
        assert Fraction(float(o)) == want
    # zero residual leaves a BF16 value unchanged
    assert np.array_equal(obwd.residual_add_bf16(a, np.zeros_like(a)), a)


def _state(rows, cols, seed, std=1.0):
    rng = np.random.default_rng(seed)
    x = bf16_round((rng.standard_normal((rows, cols)) * std).astype(np.float32)).astype(np.float64)
    return onv.quantize(x)


def test_silu_mul_bwd_f32_close_to_exact_derivative():
    aq, bq = _state(16, 256, 72), _state(16, 256, 73)
    dh = bf16_round((np.random.default_rng(74).standard_normal((16, 256)) * 0.01).astype(np.float32))
    da, db = obwd.silu_mul_bwd_f32(aq, bq, dh)
    ea, eb, ca, cb = obwd.silu_mul_bwd(aq, bq, dh)
    assert np.all(np.abs(da - ea) <= tol.grad_bound(ea, ca))
    assert np.all(np.abs(db - eb) <= tol.grad_bound(eb, cb))
    # the pinned sequence differs from the exact value by far less than one BF16 ulp beyond the final rounding
    assert np.all(np.abs(da - ea) <= 0.5 * tol.ulp_bf16(ea) * (1 + 2.0 ** -10) + 2.0 ** -20 * ca)


def test_silu_mul_bwd_f32_closed_forms():
    zero = onv.quantize(np.zeros((2, 32)))
    bq = _state(2, 32, 75)
    dh = bf16_round(np.random.default_rng(76).standard_normal((2, 32)).astype(np.float32))
    da, db = obwd.silu_mul_bwd_f32(zero, bq, dh)
    # a^ = 0: sigma = 1/2 exactly, dgate = bf16(dh b^ / 2), dup = 0
    b = onv.dequantize(bq)
    assert np.array_equal(da.astype(np.float64), tol.bf16_rne(dh.astype(np.float64) * b / 2))
    assert np.all(db == 0)
    da0, db0 = obwd.silu_mul_bwd_f32(_state(2, 32, 77), bq, np.zeros((2, 32), np.float32))
    assert np.all(da0 == 0) and np.all(db0 == 0)


def test_rmsnorm_mean_is_exactly_rounded():
    yq = _state(6, 64, 78)
    dy = bf16_round((np.random.default_rng(79).standard_normal((6, 64)) * 0.01).astype(np.float32))
    mean = obwd.rmsnorm_mean_f32(yq, dy)
    y = onv.dequantize(yq)
    for i in range(6):
        S = sum(Fraction(float(dy[i, j])) * Fraction(float(y[i, j])) for j in range(64))
        S64 = _rne_bits(S, 53, -1074)
        want = _rne_f32(_rne_bits(S64 / 64, 53, -1074))          # float64 division, then FP32
        assert Fraction(float(mean[i])) == want


def test_rmsnorm_bwd_f32_close_to_exact_derivative():
    yq = _state(12, 512, 80)
    rng = np.random.default_rng(81)
    g = bf16_round(rng.uniform(0.9, 1.1, 512).astype(np.float32))
    dy = bf16_round((rng.standard_normal((12, 512)) * 0.01).astype(np.float32))
    rstd = rng.uniform(0.5, 2.0, 12).astype(np.float32)
    dx = obwd.rmsnorm_bwd_f32(yq, rstd, g, dy)
    ref, cancel = obwd.rmsnorm_bwd(yq, rstd, g, dy)
    assert np.all(np.abs(dx - ref) <= tol.grad_bound(ref, cancel))


def test_rmsnorm_bwd_residual_composition():
    yq = _state(5, 128, 82)
    rng = np.random.default_rng(83)
    g = bf16_round(rng.uniform(0.9, 1.1, 128).astype(np.float32))
    dy = bf16_round((rng.standard_normal((5, 128)) * 0.01).astype(np.float32))
    resid = bf16_round((rng.standard_normal((5, 128)) * 0.01).astype(np.float32))
    rstd = rng.uniform(0.5, 2.0, 5).astype(np.float32)
    dx = obwd.rmsnorm_bwd_f32(yq, rstd, g, dy)
    out, q = obwd.rmsnorm_bwd_residual(yq, rstd, g, dy, resid)
    assert np.array_equal(out, obwd.residual_add_bf16(dx, resid))
    q2 = onv.quantize(out.astype(np.float64))
    assert np.array_equal(q.codes, q2.codes) and np.array_equal(q.scales, q2.scales)
    out0, _ = obwd.rmsnorm_bwd_residual(yq, rstd, g, dy, None)
    assert np.array_equal(out0, dx)


def test_silu_mul_bwd_quant_composition():
    aq, bq = _state(4, 64, 84), _state(4, 64, 85)
    dh = bf16_round((np.random.default_rng(86).standard_normal((4, 64)) * 0.01).astype(np.float32))
    da, db, qa, qb = obwd.silu_mul_bwd_quant(aq, bq, dh)
    a2, b2 = obwd.silu_mul_bwd_f32(aq, bq, dh)
    assert np.array_equal(da, a2) and np.array_equal(db, b2)
    # the NVFP4 copies dequantize to within the format's error of the BF16 gradients
    for v, q in ((da, qa), (db, qb)):
        d = onv.dequantize(q)
        assert np.all(np.abs(d - v) <= np.abs(v).max(axis=1, keepdims=True) * 0.25 + 1e-30)
