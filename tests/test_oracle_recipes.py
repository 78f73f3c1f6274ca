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


# ---------------------------------------------------------------------------
# FP32 tensor-scale recipe: S = RN32(amax / 2688) (>= 2^-126; 1 for a zero
# tensor), R = RN32(1 / S), u = RN32(|x| R), then the block rules on u.
# ---------------------------------------------------------------------------
def _f32_rne(q: Fraction) -> Fraction:
    """Nearest FP32 value to a non-negative rational (ties to even), normal or
    subnormal, by integer arithmetic on the exact value."""
    assert q >= 0
    if q == 0:
        return Fraction(0)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    while Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    step = Fraction(2) ** (max(e, -126) - 23)              # spacing of FP32 values at q
    n = q / step
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    out = fl * step
    assert out < Fraction(2) ** 128
    return out


def _brute_fp32_tensor(rows, amax):
    a = Fraction(float(amax))
    if a == 0:
        S, R = Fraction(1), Fraction(1)
    else:
        S = max(_f32_rne(a / 2688), Fraction(2) ** -126)
        R = _f32_rne(1 / S)
    out = []
    for row in rows:
        fr = [Fraction(float(v)) for v in row]
        u = [_f32_rne(abs(v) * R) for v in fr]
        scales, codes = [], []
        for b in range(len(fr) // 16):
            ub = u[16 * b:16 * b + 16]
            t = max(ub) / 6
            c = min(range(len(E4M3)), key=lambda k: (abs(E4M3[k] - t), k % 2))   # nearest, ties to even
            s = E4M3[c]
            scales.append(c)
            for v, uv in zip(row[16 * b:16 * b + 16], ub):
                mu = 0 if s == 0 else min(range(8), key=lambda k: (abs(E2M1[k] - uv / s), k % 2))
                codes.append(mu | (8 if np.signbit(float(v)) else 0))
        out.append((scales, codes))
    return S, R, out


def test_fp32_tensor_scale_constants_match_exact_rounding():
    rng = np.random.default_rng(63)
    amaxes = [0.0, 2688.0, 1.0, 3.0, 1e-3, 7.25, float(np.float32(3.3895314e38)), 2.0 ** -133, 2.0 ** -110,
              2688.0 * 2.0 ** -126, 2688.0 * 2.0 ** -127]
    amaxes += list(np.exp(rng.uniform(-60, 60, 200)))
    for a in [float(np.float32(v)) for v in amaxes]:                  # FP32 maxima
        S, R = onv.tensor_scale_fp32(a)
        if a == 0:
            assert S == 1 and R == 1
            continue
        S_ref = max(_f32_rne(Fraction(a) / 2688), Fraction(2) ** -126)
        assert Fraction(float(S)) == S_ref, a
        assert Fraction(float(R)) == _f32_rne(1 / S_ref), a


def test_fp32_tensor_scale_matches_exact_rational_brute_force():
    rng = np.random.default_rng(64)
    for trial in range(6):
        x = rng.standard_normal((5, 48)) * 2.0 ** int(rng.integers(-20, 20))
        x[rng.integers(0, 5), rng.integers(0, 48)] *= 30.0            # one outlier sets amax
        x = x.astype(np.float32).astype(np.float64)
        if trial == 1:
            x[2, :16] = 0.0                                            # an all-zero block
            x[3, 5] = -0.0
        amax = "auto" if trial % 2 == 0 else float(np.float32(np.abs(x).max() * 1.75))
        q = onv.quantize(x, tensor_amax=amax, fp32_tensor_scale=True)
        a = np.abs(x).max() if amax == "auto" else amax
        S, R, rows = _brute_fp32_tensor(x, a)
        assert np.all(q.rscale == np.float32(float(S)))
        codes = onv.unpack_codes(q.codes)
        for i, (sc, cd) in enumerate(rows):
            assert q.scales[i].tolist() == sc, (trial, i)
            assert codes[i].tolist() == cd, (trial, i)


def test_fp32_tensor_scale_with_power_of_two_scale_is_the_power_of_two_recipe():
    # amax = 2688 * 2^k gives S = 2^k exactly (and R = 2^-k): then u = |x| / r
    # as in the power-of-two tensor-scale recipe, which must agree bit for bit
    rng = np.random.default_rng(65)
    for k in (-20, -3, 0, 5):
        x = rng.standard_normal((12, 64)) * 2.0 ** k * 300.0
        x = x.astype(np.float32).astype(np.float64)
        amax = 2688.0 * 2.0 ** k
        assert np.abs(x).max() <= amax
        a = onv.quantize(x, tensor_amax=amax, fp32_tensor_scale=True)
        b = onv.quantize(x, tensor_amax=amax)
        assert np.all(a.rscale == np.float32(2.0 ** k)) and np.all(b.rscale == a.rscale)
        assert np.array_equal(a.codes, b.codes) and np.array_equal(a.scales, b.scales)
        for ru in (True,):
            a2 = onv.quantize(x, tensor_amax=amax, fp32_tensor_scale=True, round_up=ru)
            b2 = onv.quantize(x, tensor_amax=amax, round_up=ru)
            assert np.array_equal(a2.codes, b2.codes) and np.array_equal(a2.scales, b2.scales)


def test_fp32_tensor_scale_uses_the_top_of_the_scale_range():
    # the block holding amax gets scale ~448 (u_max = RN32(amax R) ~ 2688), so
    # the FP32 tensor scale leaves no E4M3 headroom unused, unlike the
    # power-of-two one; every element dequantizes within the format's error
    rng = np.random.default_rng(66)
    x = (rng.standard_normal((16, 128)) * 0.37).astype(np.float32).astype(np.float64)
    q = onv.quantize(x, tensor_amax="auto", fp32_tensor_scale=True)
    i, j = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert onv.scale_values(q)[i, j // 16] in (416.0, 448.0)
    d = onv.dequantize(q)
    s = np.repeat(onv.scale_values(q), 16, axis=1) * float(q.rscale[0])
    assert np.all(np.abs(d - x) <= np.maximum(1.0 * s, 2.0 * s * (np.abs(x) > 6 * s)))
    # a zero tensor: S = 1, every scale and code zero (signs kept)
    z = np.zeros((2, 32)); z[1, 3] = -0.0
    qz = onv.quantize(z, tensor_amax="auto", fp32_tensor_scale=True)
    assert np.all(qz.rscale == 1.0) and not qz.scales.any()
    assert onv.unpack_codes(qz.codes)[1, 3] == 8 and onv.unpack_codes(qz.codes).sum() == 8
