"""Pins of the oracle's single-layout input gradient dX = deq(dY_q) deq(W_fwd).

Checked against an exact-rational product on small shapes, against the
dual-layout gradient where both layouts are exact (weights whose every block
is exactly representable along both axes), and through the identity that
forward and single-layout input gradient use the same effective weight
(<dX, X> = <dY, Y> for the exact products).
"""

from fractions import Fraction

import numpy as np

from oracle import gemm as ogemm
from oracle import nvfp4 as onv


def test_matches_exact_rational_product():
    rng = np.random.default_rng(50)
    dyq = onv.quantize(rng.standard_normal((4, 32)) * 0.01)
    wf = onv.quantize(rng.standard_normal((32, 48)) * 0.02)
    dx, dabs = ogemm.gemm_dgrad_fwd_layout(dyq, wf)
    a, b = onv.dequantize(dyq), onv.dequantize(wf)
    for m in range(4):
        for k in range(48):
            exact = sum(Fraction(float(a[m, n])) * Fraction(float(b[n, k])) for n in range(32))
            absum = sum(abs(Fraction(float(a[m, n])) * Fraction(float(b[n, k]))) for n in range(32))
            assert abs(dx[m, k] - float(exact)) <= 2 ** -50 * float(absum)
            assert abs(dabs[m, k] - float(absum)) <= 2 ** -50 * float(absum)


def test_equals_dual_layout_when_both_layouts_are_exact():
    # W = E2M1 codes times one power of two per row: every 16-block along K has
    # block max 6 (an E4M3-exact scale), but along N the blocks mix rows, so make
    # the power of two the same for all rows; then both layouts reproduce W exactly
    rng = np.random.default_rng(51)
    vals = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    w = rng.choice(vals, size=(64, 64)) * rng.choice([-1, 1], size=(64, 64)) * 2.0 ** -6
    w[:, ::16] = 6 * 2.0 ** -6                    # every block along K and along N reaches the maximum
    w[::16, :] = 6 * 2.0 ** -6
    wf, wb = ogemm.weight_layouts(w)
    assert np.array_equal(onv.dequantize(wf), w) and np.array_equal(onv.dequantize(wb), w.T)
    dyq = onv.quantize(rng.standard_normal((8, 64)) * 0.01)
    d1, _ = ogemm.gemm_dgrad_fwd_layout(dyq, wf)
    d2, _ = ogemm.gemm_dgrad(dyq, wb)
    assert np.allclose(d1, d2, rtol=0, atol=1e-15)


def test_adjoint_of_the_forward_product():
    rng = np.random.default_rng(52)
    xq = onv.quantize(rng.standard_normal((6, 64)))
    wf = onv.quantize(rng.standard_normal((48, 64)) * 0.02)
    dyq = onv.quantize(rng.standard_normal((6, 48)) * 0.01)
    y, _ = ogemm.gemm_fwd(xq, wf)                   # Y = X W~^T
    dx, _ = ogemm.gemm_dgrad_fwd_layout(dyq, wf)    # dX = dY W~
    lhs = np.sum(onv.dequantize(dyq) * y)
    rhs = np.sum(dx * onv.dequantize(xq))
    assert abs(lhs - rhs) <= 1e-12 * (abs(lhs) + 1e-30)
