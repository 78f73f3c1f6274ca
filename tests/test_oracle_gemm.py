"""Pins of the oracle's GEMMs, LoRA branch and tolerance helpers.

Frozen projections are NVFP4 GEMMs that sum in FP32 and write BF16 (PACT,
Appendix Table 7, row "Frozen projections"); the LoRA branch is a
BF16 GEMM on the reconstructed input (row "LoRA branch").  The oracle
computes both exactly in float64; these tests pin it with exact-rational
brute force on tiny shapes, an integer special case, finite differences of
the LoRA gradients, and closed forms of the BF16 rounding helpers.
"""

from fractions import Fraction

import numpy as np

from oracle import gemm, lora, nvfp4, tolerance


def _frac_deq(q):
    """Dequantize with exact rationals, element by element (independent of nvfp4.dequantize)."""
    R = q.codes.shape[0]
    C = q.codes.shape[1] * 2
    out = [[None] * C for _ in range(R)]
    for i in range(R):
        r = Fraction(float(q.rscale[i]))
        for j in range(C):
            byte = int(q.codes[i, j // 2])
            code = (byte >> 4) if j % 2 else (byte & 15)
            sc = int(q.scales[i, j // 16])
            e, m = sc >> 3, sc & 7
            s = Fraction(m, 512) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7)
            ee, mm = (code >> 1) & 3, code & 1
            v = Fraction(mm, 2) if ee == 0 else Fraction(2 + mm, 2) * Fraction(2) ** (ee - 1)
            out[i][j] = (-v if code & 8 else v) * s * r
    return out


def test_gemm_matches_rational_brute_force():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((5, 48)) * 3
    w = rng.standard_normal((7, 48)) * 0.02
    xq, wf = nvfp4.quantize(x), nvfp4.quantize(w)
    y, absy = gemm.gemm_fwd(xq, wf)
    fx, fw = _frac_deq(xq), _frac_deq(wf)
    for m in range(5):
        for n in range(7):
            exact = sum(a * b for a, b in zip(fx[m], fw[n]))
            abs_exact = sum(abs(a * b) for a, b in zip(fx[m], fw[n]))
            assert abs(Fraction(y[m, n]) - exact) <= abs_exact * Fraction(1, 2 ** 50)
            assert abs(Fraction(absy[m, n]) - abs_exact) <= abs_exact * Fraction(1, 2 ** 50)


def test_dgrad_uses_backward_layout():
    """dX = dY_q W_bwd^T with W_bwd = Q(W^T): brute force on a tiny case."""
    rng = np.random.default_rng(6)
    w = rng.standard_normal((32, 48)) * 0.02        # [N x K]
    dy = rng.standard_normal((3, 32)) * 0.01        # [M x N]
    wf, wb = gemm.weight_layouts(w)
    assert wf.codes.shape == (32, 24) and wb.codes.shape == (48, 16)
    dyq = nvfp4.quantize(dy)
    dx, _ = gemm.gemm_dgrad(dyq, wb)
    assert dx.shape == (3, 48)
    fd, fb = _frac_deq(dyq), _frac_deq(wb)
    for m in range(3):
        for k in range(48):
            exact = sum(a * b for a, b in zip(fd[m], fb[k]))
            assert abs(Fraction(dx[m, k]) - exact) <= Fraction(1, 2 ** 60)


def test_integer_special_case_is_exact():
    """Unit scales: every product is a multiple of 1/4, so the float64 GEMM is exact."""
    rng = np.random.default_rng(9)
    M, N, K = 8, 12, 512
    ca = rng.integers(0, 16, size=(M, K))
    cb = rng.integers(0, 16, size=(N, K))

    def mk(c):
        packed = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
        return nvfp4.NVFP4(packed, np.full((c.shape[0], c.shape[1] // 16), 0x38, np.uint8),
                           np.ones(c.shape[0], np.float32))

    y, _ = gemm.gemm_nt(mk(ca), mk(cb))
    # integer arithmetic: E2M1 value * 2 is an integer
    ia = np.round(nvfp4.E2M1_ALL[ca] * 2).astype(np.int64)
    ib = np.round(nvfp4.E2M1_ALL[cb] * 2).astype(np.int64)
    assert np.array_equal(y * 4, (ia @ ib.T).astype(np.float64))


def test_lora_down_and_term():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((6, 32))
    a = rng.standard_normal((4, 32)) * 0.01
    xq = nvfp4.quantize(x)
    t, tb, tabs = lora.lora_down(xq, a)
    fx = _frac_deq(xq)
    for m in range(6):
        for j in range(4):
            exact = sum(p * Fraction(float(q)) for p, q in zip(fx[m], a[j]))
            abs_exact = sum(abs(p * Fraction(float(q))) for p, q in zip(fx[m], a[j]))
            assert abs(Fraction(t[m, j]) - exact) <= abs_exact * Fraction(1, 2 ** 50)
            assert abs(Fraction(tabs[m, j]) - abs_exact) <= abs_exact * Fraction(1, 2 ** 50)
    assert np.all(np.abs(tb - t) <= tolerance.ulp_bf16(t) / 2)
    term, _, _ = lora.lora_term(tb, np.zeros((4, 9)), 2.0)
    assert np.all(term == 0)


def test_lora_gradients_by_finite_differences():
    """dA, dB, dT of L = sum(G * s T B^T), T = X~ A^T, before BF16 rounding."""
    rng = np.random.default_rng(13)
    M, K, N, r, s = 5, 32, 7, 3, 0.75
    xq = nvfp4.quantize(rng.standard_normal((M, K)))
    xt = nvfp4.dequantize(xq)
    A = rng.standard_normal((r, K))
    B = rng.standard_normal((N, r))
    G = rng.standard_normal((M, N))

    def loss(A_, B_):
        return float(np.sum(G * (s * (xt @ A_.T) @ B_.T)))

    h = 1e-6
    num_dA = np.zeros_like(A)
    for j in range(r):
        for k in range(K):
            E = np.zeros_like(A)
            E[j, k] = h
            num_dA[j, k] = (loss(A + E, B) - loss(A - E, B)) / (2 * h)
    num_dB = np.zeros_like(B)
    for n in range(N):
        for j in range(r):
            E = np.zeros_like(B)
            E[n, j] = h
            num_dB[n, j] = (loss(A, B + E) - loss(A, B - E)) / (2 * h)
    out = lora.lora_bwd(xq, A, B, G, s)
    # the oracle rounds T and dT to BF16 before the next BF16 GEMM; the exact
    # gradients differ from its results by at most half an ulp of those inputs
    assert np.all(np.abs(out["dA_exact"] - num_dA) <= out["dA_tslack"] / 2 + 1e-7)
    assert np.all(np.abs(out["dB_exact"] - num_dB) <= out["dB_tslack"] / 2 + 1e-7)
    assert np.all(np.abs(out["dT"] - out["dT_exact"]) <= tolerance.ulp_bf16(out["dT_exact"]) / 2)
    assert np.all(np.abs(out["dA"] - out["dA_exact"]) <= tolerance.ulp_bf16(out["dA_exact"]) / 2)


def test_bf16_rne_and_ulp_closed_forms():
    assert tolerance.ulp_bf16(1.0) == 2.0 ** -7
    assert tolerance.ulp_bf16(3.0) == 2.0 ** -6
    assert tolerance.ulp_bf16(-0.75) == 2.0 ** -8
    assert tolerance.ulp_bf16(0.0) == 2.0 ** -133
    assert tolerance.ulp_bf16(1e-39) == 2.0 ** -133
    one = 1.0
    u = 2.0 ** -7
    assert tolerance.bf16_rne(one + u / 2) == one                  # tie -> even (1.0)
    assert tolerance.bf16_rne(one + 1.5 * u) == one + 2 * u        # tie -> even (1 + 2u)
    assert tolerance.bf16_rne(one + u / 2 + 2.0 ** -40) == one + u # just above the tie
    assert tolerance.bf16_rne(-(one + u / 2 + 2.0 ** -40)) == -(one + u)
    assert tolerance.bf16_rne(255.5 * 2.0 ** -7) == 2.0             # carry into next binade
    # a value that double rounding through float32 would misround
    v = one + u / 2 + 2.0 ** -30                   # float32 rounds it to the tie point
    assert tolerance.bf16_rne(v) == one + u
    assert np.float32(v) == np.float32(one + u / 2)


def test_dgrad_multi_matches_rational_sum_over_segments():
    """Summed input gradient over segments of different widths and row-scale
    ranges equals the exact rational sum of every segment's products (rows of
    dY_i against rows of W_bwd,i = columns of W_i)."""
    rng = np.random.default_rng(140)
    M, K, widths = 3, 2, (16, 48, 32)
    segs = []
    for i, n in enumerate(widths):
        dy = rng.standard_normal((M, n)) * 2.0 ** (6 * i - 6)
        w = rng.standard_normal((n, K)) * 2.0 ** (-3 * i)
        segs.append((nvfp4.quantize(dy), nvfp4.quantize(w, transpose=True)))
    ref, rabs = gemm.gemm_dgrad_multi(segs)
    assert ref.shape == (M, K)
    exact = [[Fraction(0)] * K for _ in range(M)]
    absum = [[Fraction(0)] * K for _ in range(M)]
    for dyq, wb in segs:
        a, b = _frac_deq(dyq), _frac_deq(wb)
        for m in range(M):
            for k in range(K):
                for j in range(dyq.cols):
                    exact[m][k] += a[m][j] * b[k][j]
                    absum[m][k] += abs(a[m][j] * b[k][j])
    for m in range(M):
        for k in range(K):
            assert abs(Fraction(float(ref[m, k])) - exact[m][k]) <= Fraction(2) ** -50 * absum[m][k]
            assert abs(Fraction(float(rabs[m, k])) - absum[m][k]) <= Fraction(2) ** -50 * absum[m][k]
    # one segment is the plain input gradient
    r1, a1 = gemm.gemm_dgrad_multi(segs[:1])
    r0, a0 = gemm.gemm_dgrad(*segs[0])
    assert np.array_equal(r1, r0) and np.array_equal(a1, a0)


def _frac_bf16(x: Fraction) -> Fraction:
    """Round an exact rational to the nearest BF16 value, ties to the even
    significand (8 significant bits; subnormal spacing 2^-133), written with
    integer arithmetic only (independent of tolerance.bf16_rne)."""
    if x == 0:
        return Fraction(0)
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    q = Fraction(2) ** max(e - 7, -133)
    n = a / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return (fl * q) if x > 0 else -(fl * q)


def _frac_ulp_bf16(x: Fraction) -> Fraction:
    """BF16 unit in the last place at |x| by its definition: 2^(max(floor(log2|x|), -126) - 7)."""
    if x == 0:
        return Fraction(2) ** -133
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    return Fraction(2) ** (max(e, -126) - 7)


def test_lora_term_nonzero_against_rationals():
    """lora_term(T, U, s) = s T U with its two bound sums, checked against
    exact rationals on a non-square case (r = 3, Nout = 5) with nonzero U and
    scales that are not 1 or 2 (one not a power of two, one negative and not
    a binary fraction).  A dropped or doubled s, a sign error or a transposed
    U changes the term by far more than the 2^-50 relative slack."""
    rng = np.random.default_rng(141)
    M, r, N = 4, 3, 5
    t = tolerance.bf16_rne(rng.standard_normal((M, r)) * 0.3)
    u = tolerance.bf16_rne(rng.standard_normal((r, N)) * 0.01)
    for s in (0.75, -1.0 / 3.0):
        term, tabs, tslack = lora.lora_term(t, u, s)
        assert term.shape == (M, N) and tabs.shape == (M, N) and tslack.shape == (M, N)
        fs = Fraction(s)                       # the float the oracle was given
        for m in range(M):
            for n in range(N):
                prods = [Fraction(float(t[m, j])) * Fraction(float(u[j, n])) for j in range(r)]
                exact = fs * sum(prods)
                absum = abs(fs) * sum(abs(p) for p in prods)
                slack = abs(fs) * sum(_frac_ulp_bf16(Fraction(float(t[m, j]))) * abs(Fraction(float(u[j, n])))
                                      for j in range(r))
                assert absum > 0
                assert abs(Fraction(float(term[m, n])) - exact) <= absum * Fraction(1, 2 ** 50)
                assert abs(Fraction(float(tabs[m, n])) - absum) <= absum * Fraction(1, 2 ** 50)
                assert abs(Fraction(float(tslack[m, n])) - slack) <= slack * Fraction(1, 2 ** 50)
        # the transposed product is a different matrix here (and a different shape)
        with np.testing.assert_raises(ValueError):
            lora.lora_term(t, u.T, s)


def test_forward_with_lora_composed_against_rationals():
    """Y = X~ W~^T + s bf16(X~ A^T) B^T, composed from the oracle's pieces
    (gemm_fwd, lora_down, lora_term) exactly as the GPU tests compose their
    expected value, against an exact-rational evaluation of the same formula
    with its own BF16 rounding of T.  s = 0.75 and s = -1/3."""
    rng = np.random.default_rng(142)
    M, K, N, r = 3, 32, 5, 4
    x = rng.standard_normal((M, K))
    w = rng.standard_normal((N, K)) * 0.02
    a = tolerance.bf16_rne(rng.standard_normal((r, K)) * 0.05)
    b = tolerance.bf16_rne(rng.standard_normal((N, r)) * 0.05)
    xq, wf = nvfp4.quantize(x), nvfp4.quantize(w)
    fx, fw = _frac_deq(xq), _frac_deq(wf)
    ft = [[_frac_bf16(sum(fx[m][k] * Fraction(float(a[j, k])) for k in range(K))) for j in range(r)]
          for m in range(M)]
    y, yabs = gemm.gemm_fwd(xq, wf)
    _, t_bf16, _ = lora.lora_down(xq, a)
    for m in range(M):
        for j in range(r):
            assert Fraction(float(t_bf16[m, j])) == ft[m][j], "T must be the BF16 rounding of the exact X~ A^T"
    for s in (0.75, -1.0 / 3.0):
        term, tabs, _ = lora.lora_term(t_bf16, b.T, s)
        got = y + term
        fs = Fraction(s)
        for m in range(M):
            for n in range(N):
                base = [fx[m][k] * fw[n][k] for k in range(K)]
                lr = [ft[m][j] * Fraction(float(b[n, j])) for j in range(r)]
                exact = sum(base) + fs * sum(lr)
                absum = sum(abs(v) for v in base) + abs(fs) * sum(abs(v) for v in lr)
                assert abs(Fraction(float(got[m, n])) - exact) <= absum * Fraction(1, 2 ** 49)
                assert abs(Fraction(float(yabs[m, n] + tabs[m, n])) - absum) <= absum * Fraction(1, 2 ** 49)
        # the LoRA term is not negligible in this case: dropping it moves Y by
        # much more than the GPU acceptance bound
        bound = tolerance.gemm_bound(got, yabs + tabs)
        assert np.any(np.abs(term) > bound)
