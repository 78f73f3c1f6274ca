"""Pins of the oracle's recipe variants of the NVFP4 quantizer.

The format table (PACT, Appendix Table 6) fixes the block format but not the
block-scale rounding or the second-level scale's extent.  Variants: block
scales rounded up (the smallest E4M3 value >= blockmax / (6 r), so no element
saturates) and one power-of-two scale for the whole tensor (the row-scale rule
applied to the tensor maximum).  Pinned by a hand-worked block, an
exact-rational brute force, the non-saturation property and the reductions
to the default recipe.
"""

from fractions import Fraction

import numpy as np

from oracle import nvfp4 as onv

E2M1 = [Fraction(v) for v in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
E4M3 = [Fraction(onv.e4m3fn_value(c)) for c in range(0x7F)]


def test_hand_worked_round_up_block():
    # row [7, 1, 0 x 14]: rowmax 7 -> e = ceil(log2(7 / 2688)) = -8, r = 2^-8;
    # blockmax / (6 r) = 7 * 256 / 6 = 298.67: nearest E4M3 is 288 (0x79,
    # 1.125 * 2^8), the next one up 320 (0x7A, 1.25 * 2^8).
    x = np.zeros((1, 16))
    x[0, 0], x[0, 1] = 7.0, 1.0
    q = onv.quantize(x)
    qu = onv.quantize(x, round_up=True)
    assert q.rscale[0] == qu.rscale[0] == 2.0 ** -8
    assert q.scales[0, 0] == 0x79 and qu.scales[0, 0] == 0x7A
    # 7 / (288 r) = 6.22 saturates to 6 (code 7); 7 / (320 r) = 5.6 rounds to 6 too;
    # 1 / (288 r) = 0.89 and 1 / (320 r) = 0.8 both round to 1 (code 2)
    c, cu = onv.unpack_codes(q.codes)[0], onv.unpack_codes(qu.codes)[0]
    assert c[0] == 7 and c[1] == 2 and cu[0] == 7 and cu[1] == 2


def _brute_round_up(row):
    fr = [Fraction(float(v)) for v in row]
    amax = max(abs(v) for v in fr)
    e = 0
    if amax > 0:
        e = -200
        while amax > 2688 * Fraction(2) ** e:
            e += 1
        e = max(-126, min(127, e))
    r = Fraction(2) ** e
    scales, codes = [], []
    for b in range(len(fr) // 16):
        blk = fr[16 * b:16 * b + 16]
        t = max(abs(v) for v in blk) / (6 * r)
        c = min(i for i, v in enumerate(E4M3) if v >= t)
        s = E4M3[c]
        scales.append(c)
        for v in blk:
            if s == 0:
                mu = 0
            else:
                u = abs(v) / (s * r)
                assert u <= 6                                     # never saturates
                mu = min(range(8), key=lambda k: (abs(E2M1[k] - u), k % 2))
            codes.append(mu | (8 if v < 0 or (v == 0 and np.signbit(float(v))) else 0))
    return e, scales, codes


def test_round_up_matches_exact_rational_brute_force():
    rng = np.random.default_rng(60)
    rows = []
    for i in range(60):
        v = rng.standard_normal(64) * 2.0 ** int(rng.integers(-30, 30))
        if i % 3 == 0:
            v[rng.integers(0, 64, 5)] *= 20.0
        rows.append(v.astype(np.float32).astype(np.float64))
    x = np.array(rows)
    q = onv.quantize(x, round_up=True)
    codes = onv.unpack_codes(q.codes)
    for i, row in enumerate(rows):
        e, sc, cd = _brute_round_up(row)
        assert q.rscale[i] == 2.0 ** e
        assert q.scales[i].tolist() == sc, i
        assert codes[i].tolist() == cd, i


def test_round_up_never_below_nearest_and_never_saturates():
    rng = np.random.default_rng(61)
    x = rng.standard_normal((40, 256)) * np.exp(rng.uniform(-8, 8, (40, 1)))
    q, qu = onv.quantize(x), onv.quantize(x, round_up=True)
    assert np.all(qu.scales >= q.scales) and np.all(qu.scales <= q.scales.astype(int) + 1)
    s = np.repeat(onv.scale_values(qu), 16, axis=1) * qu.rscale[:, None].astype(np.float64)
    assert np.all(np.abs(x) <= 6.0 * s)                          # block scale * row scale per element


def test_tensor_scale_reduces_to_the_row_rule():
    rng = np.random.default_rng(62)
    x = rng.standard_normal((24, 128)) * np.exp(rng.uniform(-3, 3, (24, 1)))
    qt = onv.quantize(x, tensor_amax="auto")
    e = onv.row_exponent(np.array(np.abs(x).max()))
    assert np.all(qt.rscale == np.float32(2.0 ** int(e)))
    # the row holding the tensor maximum is quantized exactly as by the default recipe
    i = int(np.argmax(np.abs(x).max(axis=1)))
    q = onv.quantize(x)
    assert np.array_equal(qt.codes[i], q.codes[i]) and np.array_equal(qt.scales[i], q.scales[i])
    # a one-row tensor: identical to the default recipe
    q1, qt1 = onv.quantize(x[:1]), onv.quantize(x[:1], tensor_amax="auto")
    assert np.array_equal(q1.codes, qt1.codes) and np.array_equal(q1.scales, qt1.scales)
    # a supplied maximum above the true one only moves the exponent up
    qs = onv.quantize(x, tensor_amax=4 * np.abs(x).max())
    assert np.all(qs.rscale >= qt.rscale)
    # every element still dequantizes within the format's error: half the E2M1
    # spacing at the value (<= 1 * s r), or below 2 s r where the block saturates
    d = onv.dequantize(qt)
    s = np.repeat(onv.scale_values(qt), 16, axis=1) * qt.rscale[:, None].astype(np.float64)
    assert np.all(np.abs(d - x) <= 2.0 * s)
