"""Pins of the oracle's NVFP4 format code against what the format fixes.

The NVFP4 format (PACT, Appendix Table 6): 16-element blocks, E2M1 elements,
E4M3 block scales, 4.50 bits per element.  These tests check the oracle
against the E2M1 and E4M3 bit-field definitions, hand-worked vectors
(tests/golden/nvfp4_vectors.txt), and an independent brute-force quantizer
written with exact rationals that picks nearest values by enumeration rather
than by counting thresholds.
"""

import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import nvfp4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "nvfp4_vectors.txt")


# ---------------------------------------------------------------------------
# Independent brute force: nearest-value search with exact rationals
# ---------------------------------------------------------------------------

def _e2m1_table():
    # magnitudes from the definition: sign | 2-bit exponent (bias 1) | 1-bit mantissa
    out = []
    for code in range(8):
        e, m = code >> 1, code & 1
        out.append(Fraction(m, 2) if e == 0 else Fraction(2 + m, 2) * Fraction(2) ** (e - 1))
    return out


def _e4m3_table():
    out = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        out.append(Fraction(m, 8) * Fraction(1, 64) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7))
    return out


E2 = _e2m1_table()
E4 = _e4m3_table()


def _nearest(table, t):
    """Index of the table value nearest t; ties to the even index; above max -> max."""
    best = None
    for i, v in enumerate(table):
        d = abs(v - t)
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
            best = (d, i)
    return best[1]


def brute_quantize_row(row):
    xs = [Fraction(float(v)) for v in row]
    signs = [1 if np.signbit(float(v)) else 0 for v in row]    # Fraction drops the sign of -0
    A = max(abs(v) for v in xs)
    if A == 0:
        e = 0
    else:
        e = -200
        while A > 2688 * Fraction(2) ** e:
            e += 1
        e = max(-126, min(127, e))
    r = Fraction(2) ** e
    codes, scales = [], []
    for b in range(0, len(xs), 16):
        blk = xs[b:b + 16]
        a = max(abs(v) for v in blk)
        si = _nearest(E4, a / (6 * r))
        s = E4[si]
        scales.append(si)
        for v, sign in zip(blk, signs[b:b + 16]):
            mu = 0 if s == 0 else _nearest(E2, abs(v) / (s * r))
            codes.append(sign << 3 | mu)
    return codes, scales, e


def _codes_of(q):
    return nvfp4.unpack_codes(q.codes)


# ---------------------------------------------------------------------------
# Value sets
# ---------------------------------------------------------------------------

def test_e2m1_value_set():
    vals = sorted(set(float(v) for v in nvfp4.E2M1_ALL))
    assert vals == [-6, -4, -3, -2, -1.5, -1, -0.5, 0, 0.5, 1, 1.5, 2, 3, 4, 6]
    # every code's value equals the definition's
    for c in range(16):
        sign = -1 if c >> 3 else 1
        assert nvfp4.E2M1_ALL[c] == sign * float(E2[c & 7])


def test_e4m3fn_value_set():
    pos = nvfp4.E4M3_POS
    assert pos.size == 127 and pos[0] == 0.0
    assert pos[-1] == 448.0 and pos[1] == 2.0 ** -9
    assert np.all(np.diff(pos) > 0)
    assert np.isnan(nvfp4.e4m3fn_value(0x7F)) and np.isnan(nvfp4.e4m3fn_value(0xFF))
    assert nvfp4.e4m3fn_value(0xFE) == -448.0
    for c in range(127):
        assert pos[c] == float(E4[c])
    # normal values have 4 significant bits, subnormals are multiples of 2**-9
    assert pos[8] == 2.0 ** -6 and pos[7] == 7 * 2.0 ** -9


def test_storage_is_4p5_bits_plus_row_scale():
    for R, C in [(1, 16), (64, 256), (4096, 3072), (7, 8192)]:
        bits = nvfp4.storage_bytes(R, C) * 8
        assert bits == R * C * 4.5 + 32 * R
        q = nvfp4.quantize(np.ones((min(R, 8), C)))
        assert q.nbytes() == nvfp4.storage_bytes(min(R, 8), C)


# ---------------------------------------------------------------------------
# Hand-worked vectors
# ---------------------------------------------------------------------------

def _load_golden():
    cases, cur = [], {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, _, val = line.partition(" ")
        if key == "end":
            cases.append(cur)
            cur = {}
        else:
            cur[key] = val
    return cases


@pytest.mark.parametrize("case", _load_golden(), ids=lambda c: c["name"])
def test_golden_vectors(case):
    x = np.array([float(v) for v in case["input"].split()])[None, :]
    q = nvfp4.quantize(x)
    assert q.rscale.view(np.uint32)[0] == int(case["rscale_bits"], 16)
    assert [int(v) for v in q.scales[0]] == [int(v, 16) for v in case["scales"].split()]
    assert [int(v) for v in q.codes[0]] == [int(v, 16) for v in case["codes"].split()]
    deq = nvfp4.dequantize(q)[0]
    assert list(deq) == [float(v) for v in case["dequant"].split()]
    # the brute force agrees on the same vector
    codes, scales, e = brute_quantize_row(x[0])
    assert codes == list(_codes_of(q)[0]) and scales == list(q.scales[0])


# ---------------------------------------------------------------------------
# Exhaustive and randomized checks against the brute force
# ---------------------------------------------------------------------------

def test_roundtrip_every_code_and_scale():
    """x = c * s * r quantizes back to exactly (c, s) for all 16 codes x 126 scales."""
    r = 2.0 ** -5
    rows = []
    for si in range(1, 127):
        s = float(E4[si])
        anchor = [6 * 448 * r] + [0.0] * 15                  # fixes the row scale at r
        blk = [float(nvfp4.E2M1_ALL[c]) * s * r for c in range(16)]
        blk[7] = 6 * s * r                                     # block max -> scale exactly s
        rows.append(anchor + blk)
    x = np.array(rows)
    q = nvfp4.quantize(x)
    assert np.all(q.rscale == np.float32(r))
    assert np.all(q.scales[:, 0] == 0x7E)
    assert np.array_equal(q.scales[:, 1], np.arange(1, 127, dtype=np.uint8))
    codes = _codes_of(q)[:, 16:]
    want = np.arange(16)
    want[7] = 7
    # +0 (code 0) and -0 (code 8) both survive with their sign bit
    for i in range(126):
        assert np.array_equal(codes[i], want), i
    assert np.array_equal(nvfp4.dequantize(q), x)


def _tie_row(rng):
    """A row whose blocks hit E2M1 and E4M3 midpoints exactly."""
    r = 2.0 ** int(rng.integers(-20, 4))
    row = []
    for _ in range(4):
        si = int(rng.integers(1, 126))
        s = float(E4[si])
        mids = nvfp4.E2M1_MID
        blk = rng.choice(np.concatenate([mids, nvfp4.E2M1_MAG]), size=16) * s * r
        blk *= rng.choice([-1.0, 1.0], size=16)
        if rng.random() < 0.5:       # make the block max an E4M3 midpoint times 6
            j = int(rng.integers(0, 125))
            blk[int(rng.integers(0, 16))] = float(nvfp4.E4M3_MID[j]) * 6 * r
        row.extend(blk)
    return np.array(row)


def test_matches_brute_force_random_and_ties():
    rng = np.random.default_rng(1234)
    rows = []
    for i in range(60):
        kind = i % 6
        if kind == 0:
            row = rng.standard_normal(64).astype(np.float32)
        elif kind == 1:
            row = (rng.standard_normal(64) * 10.0 ** rng.uniform(-30, 30)).astype(np.float32)
        elif kind == 2:
            row = _tie_row(rng)
        elif kind == 3:
            row = rng.standard_normal(64).astype(np.float32)
            row[rng.integers(0, 64, size=20)] = 0.0
            row[:16] = 0.0
            row[16:18] = -0.0
        elif kind == 4:
            row = rng.standard_t(3, size=64).astype(np.float32) * np.float32(1e-3)
            row[5] = 1e4                                # wide range within one row
        else:
            row = (rng.standard_normal(64) * 1e-38).astype(np.float32)   # subnormal-ish
        rows.append(np.asarray(row, dtype=np.float64))
    x = np.array(rows)
    q = nvfp4.quantize(x)
    codes = _codes_of(q)
    for i in range(x.shape[0]):
        bc, bs, be = brute_quantize_row(x[i])
        assert list(codes[i]) == bc, i
        assert list(q.scales[i]) == bs, i
        assert q.rscale[i] == np.float32(2.0 ** be), i


def test_zero_and_negative_zero():
    x = np.zeros((2, 32))
    x[1, :] = -0.0
    q = nvfp4.quantize(x)
    assert np.all(q.rscale == 1.0) and np.all(q.scales == 0)
    assert np.all(q.codes[0] == 0x00) and np.all(q.codes[1] == 0x88)


def test_sign_symmetry_and_power_of_two_invariance():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((16, 128))
    q = nvfp4.quantize(x)
    qn = nvfp4.quantize(-x)
    assert np.array_equal(qn.codes, q.codes ^ 0x88)
    assert np.array_equal(qn.scales, q.scales)
    q4 = nvfp4.quantize(x * 2.0 ** 9)
    assert np.array_equal(q4.codes, q.codes) and np.array_equal(q4.scales, q.scales)
    assert np.array_equal(q4.rscale, q.rscale * np.float32(2.0 ** 9))


def test_error_bound_and_idempotence():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((64, 256)) * np.exp(rng.uniform(-3, 3, size=(64, 1)))
    q = nvfp4.quantize(x)
    d = nvfp4.dequantize(q)
    sr = (nvfp4.scale_values(q) * q.rscale[:, None].astype(np.float64))
    bound = np.repeat(sr, 16, axis=1)
    assert np.all(np.abs(d - x) <= bound)
    # re-quantizing a dequantized tensor reproduces its values
    d2 = nvfp4.dequantize(nvfp4.quantize(d))
    assert np.array_equal(d2, d)


def test_transpose_flag_quantizes_the_transpose():
    rng = np.random.default_rng(3)
    w = rng.standard_normal((32, 48))
    a = nvfp4.quantize(w, transpose=True)
    b = nvfp4.quantize(np.ascontiguousarray(w.T))
    assert a.codes.shape == (48, 16) and np.array_equal(a.codes, b.codes)
    assert np.array_equal(a.scales, b.scales) and np.array_equal(a.rscale, b.rscale)
