"""Pins of the oracle's fused RMSNorm / SiLU-multiply forward and backward.

PACT, Appendix Table 7, rows "RMSNorm" and "SiLU-multiply": RMSNorm
normalizes a BF16 row in FP32 and saves its NVFP4 result with one FP32
statistic per token; SiLU-multiply computes in FP32 from the BF16 gate and up
and saves an NVFP4 copy of each; backward rebuilds its inputs in FP32 from
those copies.  The tests check the pinned
FP32 exponential against math.exp, closed forms (constant rows, silu(0),
sigmoid(0)), invariances of the exact sum of squares, and the backward
formulas against finite differences of the float64 forward.
"""

import math
from fractions import Fraction

import numpy as np

from oracle import backward, fused, nvfp4
from synth import bf16_round


def test_exp_constants():
    assert abs(float(fused.L2E) * math.log(2) - 1.0) <= 2.0 ** -24
    assert abs(float(fused.LN2_HI) + float(fused.LN2_LO) - math.log(2)) <= 2.0 ** -40
    # LN2_HI has at most 16 significant bits, so n * LN2_HI is exact for |n| <= 256
    m, _ = math.frexp(float(fused.LN2_HI))
    assert (m * 2 ** 16) == int(m * 2 ** 16)
    for k in range(8):
        assert abs(float(fused.COEF[k]) * math.factorial(k) - 1.0) <= 2.0 ** -24


def _rn32_exact(v: Fraction) -> float:
    """Nearest FP32 value to the rational v (ties to even), v in the FP32 range."""
    if v == 0:
        return 0.0
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = Fraction(2) ** (max(e, -126) - 23)            # FP32 quantum at this binade (subnormals: 2^-149)
    m = a / q
    mi = m.numerator // m.denominator
    rem = m - mi
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and mi % 2 == 1):
        mi += 1
    out = float(mi * q)
    return -out if v < 0 else out


def _fma_exact(a, b, c) -> np.float32:
    return np.float32(_rn32_exact(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c))))


def test_fma32_single_rounding():
    rng = np.random.default_rng(5)
    a = rng.standard_normal(3000).astype(np.float32)
    b = (rng.standard_normal(3000) * np.exp2(rng.integers(-30, 30, 3000))).astype(np.float32)
    c = (rng.standard_normal(3000) * np.exp2(rng.integers(-40, 40, 3000))).astype(np.float32)
    c[:500] = (-(a[:500].astype(np.float64) * b[:500]) * (1 + 2.0 ** -20)).astype(np.float32)   # cancellation
    got = fused.fma32(a, b, c)
    want = np.array([_fma_exact(x, y, z) for x, y, z in zip(a, b, c)], dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # the float64 sum lands exactly on an FP32 midpoint, the exact sum just off it:
    # (1 + 2^-15)(1 - 2^-15) = 1 - 2^-30, and 2^24 + 3 - 2^-30 rounds down to 2^24 + 2
    # (rounding the float64 tie to even would give 2^24 + 4); 2^24 + 1 + 2^-30 rounds up
    u, d = np.float32(1 + 2.0 ** -15), np.float32(1 - 2.0 ** -15)
    assert fused.fma32(u, d, np.float32(2.0 ** 24 + 2)) == np.float32(2.0 ** 24 + 2)
    assert fused.fma32(-u, d, np.float32(2.0 ** 24 + 2)) == np.float32(2.0 ** 24 + 2)
    assert _fma_exact(u, d, np.float32(2.0 ** 24 + 2)) == np.float32(2.0 ** 24 + 2)
    # subnormal results, exact zeros (+0 for an exact cancellation, -0 + -0 = -0)
    t = np.float32(2.0 ** -140)
    assert fused.fma32(t, np.float32(1.5), t) == _fma_exact(t, np.float32(1.5), t)
    z = fused.fma32(np.float32(3.0), np.float32(2.0), np.float32(-6.0))
    assert z == 0.0 and not np.signbit(z)
    assert np.signbit(fused.fma32(np.float32(-0.0), np.float32(1.0), np.float32(-0.0)))


def test_exp_is_the_fma_sequence():
    """E(x) at sampled x against the same reduction and Horner steps evaluated
    with exact rational fused multiply-adds (each rounded once to FP32)."""
    xs = np.concatenate([np.linspace(-79.5, 88.5, 97, dtype=np.float32),
                         np.array([0.0, -0.0, 1e-8, -1e-8, 0.3466, -0.3466, 1.0, -1.0], dtype=np.float32)])
    got = fused.exp_f32(xs)
    for x, g in zip(xs, got):
        n = np.float32(np.rint(np.float32(x) * fused.L2E))
        r = _fma_exact(-n, fused.LN2_LO, _fma_exact(-n, fused.LN2_HI, x))
        p = fused.COEF[7]
        for k in range(6, -1, -1):
            p = _fma_exact(p, r, fused.COEF[k])
        want = np.float32(math.ldexp(float(p), int(n)))
        assert np.float32(g).view(np.uint32) == want.view(np.uint32), float(x)


def test_exp_accuracy_and_edges():
    x = np.linspace(-80, 88, 400001, dtype=np.float32)
    e = fused.exp_f32(x).astype(np.float64)
    ref = np.array([math.exp(float(v)) for v in x[::50]])
    ulp = np.array([np.spacing(np.float32(v)) for v in ref], dtype=np.float64)
    assert np.max(np.abs(e[::50] - ref) / ulp) <= 1.0
    assert fused.exp_f32(np.float32(0.0)) == 1.0
    assert fused.exp_f32(np.float32(-80.5)) == 0.0
    assert np.isinf(fused.exp_f32(np.float32(89.5)))
    assert np.isinf(fused.exp_f32(np.float32(88.9)))      # overflows inside ldexp
    assert np.all(np.diff(fused.exp_f32(np.linspace(-5, 5, 10001, dtype=np.float32))) >= 0)


def test_exp_range_selects_do_not_reach_the_sigmoid():
    """The sigmoid's denominator 1 + E(-a) is the same with or without E's two
    range selects: at the lower clamp E(-80) is about 2^-115, too small to move
    1 + E off 1 in FP32, and at the upper clamp the polynomial times 2^128
    already overflows to +inf.  (The GPU kernels form the denominator without
    the selects and rely on exactly these two facts.)"""
    lo = fused.exp_f32(np.float32(-80.0))
    assert 0.0 < float(lo) < 2.0 ** -110
    assert np.float32(1.0) + lo == np.float32(1.0)
    assert np.isinf(fused.exp_f32(np.float32(89.0)))
    # below and above the clamps the selects' values give the same denominators
    for x in (-80.25, -100.0, -1e30):
        assert np.float32(1.0) + fused.exp_f32(np.float32(x)) == np.float32(1.0) + lo
    for x in (89.25, 100.0, 1e30):
        assert np.isinf(fused.exp_f32(np.float32(x)))


def test_silu_closed_forms():
    a = np.array([0.0, -0.0, 1.0, -1.0, 100.0, -100.0, 3.0], dtype=np.float32)
    s = fused.silu_f32(a)
    assert s[0] == 0.0 and s[1] == 0.0
    assert np.signbit(s[5])                                   # -100 * 0 keeps the sign
    assert s[4] == 100.0
    sig1 = 1.0 / (1.0 + math.exp(-1.0))
    assert abs(s[2] - sig1) <= 2 * np.spacing(np.float32(sig1))
    # sigma(a) + sigma(-a) = 1  =>  silu(a) - silu(-a) = a
    assert abs((s[2] - s[3]) - 1.0) <= 4 * 2.0 ** -24
    # silu(a) ~ a/2 near zero
    assert abs(float(fused.silu_f32(np.float32(1e-3))) - 1e-3 / (1 + math.exp(-1e-3))) <= 1e-10


def test_silu_mul_quant_outputs():
    rng = np.random.default_rng(21)
    a = bf16_round(rng.standard_normal((4, 64)).astype(np.float32))
    b = bf16_round(rng.standard_normal((4, 64)).astype(np.float32))
    hq, aq, bq, h = fused.silu_mul_quant(a, b)
    ref = a.astype(np.float64) / (1 + np.exp(-a.astype(np.float64))) * b
    assert np.allclose(h, ref, rtol=1e-6, atol=1e-30)
    assert np.array_equal(nvfp4.dequantize(aq), nvfp4.dequantize(nvfp4.quantize(a)))
    assert np.array_equal(hq.codes, nvfp4.quantize(h).codes)


def test_rmsnorm_constant_row_closed_form():
    for c in [1.0, 0.5, 3.0, 1e-3, 17.25]:
        x = np.full((1, 256), bf16_round(np.float32(c)), dtype=np.float32)
        g = np.ones(256, dtype=np.float32)
        rstd = fused.rmsnorm_stats(x, 1e-5)[0]
        xc = float(x[0, 0])
        exact = 1.0 / math.sqrt(xc * xc + float(np.float32(1e-5)))
        assert abs(float(rstd) - exact) <= 1.5 * np.spacing(np.float32(exact))


def test_rmsnorm_sum_is_order_independent_and_accurate():
    rng = np.random.default_rng(22)
    x = bf16_round((rng.standard_normal((8, 1024)) * np.exp(rng.uniform(-8, 8, (8, 1024)))).astype(np.float32))
    perm = rng.permutation(1024)
    r1 = fused.rmsnorm_stats(x, 1e-5)
    r2 = fused.rmsnorm_stats(x[:, perm], 1e-5)
    assert np.array_equal(r1.view(np.uint32), r2.view(np.uint32))
    xd = x.astype(np.float64)
    ref = 1.0 / np.sqrt((xd * xd).mean(axis=1) + np.float32(1e-5))
    assert np.all(np.abs(r1 - ref) <= 2 * np.spacing(r1))


def test_rmsnorm_quant_output():
    rng = np.random.default_rng(23)
    x = bf16_round(rng.standard_normal((4, 128)).astype(np.float32))
    g = bf16_round(rng.uniform(0.9, 1.1, 128).astype(np.float32))
    yq, rstd, y = fused.rmsnorm_quant(x, g, 1e-5)
    ref = x.astype(np.float64) * rstd[:, None] * g
    assert np.allclose(y, ref, rtol=2 ** -22)
    assert np.array_equal(yq.codes, nvfp4.quantize(y).codes)


def _consistent_rmsnorm_state(rng, M, K):
    """y_q, rstd, g and the input x that they reconstruct exactly (eps derived)."""
    g = rng.uniform(0.9, 1.1, K)
    yq = nvfp4.quantize(rng.standard_normal((M, K)) * 0.5)
    yh = nvfp4.dequantize(yq)
    rstd = rng.uniform(0.3, 2.0, M)
    c = np.mean((yh / g) ** 2, axis=1)           # mean(x^2) * rstd^2
    # choose eps so that rstd = (mean(x^2) + eps)^-1/2 with x = y^ / (rstd g)
    eps = (1.0 - c) / rstd ** 2
    return yq, yh, rstd, g, eps


def test_rmsnorm_bwd_finite_differences():
    rng = np.random.default_rng(24)
    M, K = 3, 32
    yq, yh, rstd, g, eps = _consistent_rmsnorm_state(rng, M, K)
    assert np.all(eps > 0)
    x0 = yh / (rstd[:, None] * g)
    dy = rng.standard_normal((M, K))

    def loss(x):
        rs = 1.0 / np.sqrt(np.mean(x * x, axis=1) + eps)
        return float(np.sum(dy * x * rs[:, None] * g))

    h = 1e-6
    num = np.zeros_like(x0)
    for i in range(M):
        for k in range(K):
            E = np.zeros_like(x0)
            E[i, k] = h
            num[i, k] = (loss(x0 + E) - loss(x0 - E)) / (2 * h)
    dx, cancel = backward.rmsnorm_bwd(yq, rstd, g, dy)
    assert np.allclose(dx, num, rtol=1e-6, atol=1e-8)
    assert np.all(cancel >= np.abs(dx) * (1 - 1e-12))


def test_silu_mul_bwd_finite_differences_and_closed_form():
    rng = np.random.default_rng(25)
    a = rng.standard_normal((2, 32)) * 3
    b = rng.standard_normal((2, 32))
    aq, bq = nvfp4.quantize(a), nvfp4.quantize(b)
    ah, bh = nvfp4.dequantize(aq), nvfp4.dequantize(bq)
    dh = rng.standard_normal((2, 32))

    def h(a_, b_):
        return a_ / (1 + np.exp(-a_)) * b_

    eps = 1e-6
    num_da = (h(ah + eps, bh) - h(ah - eps, bh)) / (2 * eps) * dh
    num_db = (h(ah, bh + eps) - h(ah, bh - eps)) / (2 * eps) * dh
    da, db, cda, cdb = backward.silu_mul_bwd(aq, bq, dh)
    assert np.allclose(da, num_da, rtol=1e-6, atol=1e-9)
    assert np.allclose(db, num_db, rtol=1e-6, atol=1e-9)
    # silu'(0) = 1/2
    z = nvfp4.quantize(np.zeros((1, 16)))
    one = nvfp4.quantize(np.ones((1, 16)))
    da0, db0, _, _ = backward.silu_mul_bwd(z, one, np.ones((1, 16)))
    assert np.all(da0 == 0.5 * nvfp4.dequantize(one)) and np.all(db0 == 0.0)
