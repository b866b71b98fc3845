"""Pins of the oracle's integer primitives against exact rational arithmetic,
library routines and closed-form error bounds (float appears only here, in
the checks, never in the oracle's forward path)."""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle as O


def half_up(x: Fraction) -> int:
    """floor(x + 1/2) on an exact rational."""
    return math.floor(x + Fraction(1, 2))


def test_round_shift_exhaustive_small():
    for s in range(-4, 25):
        for x in range(-4100, 4100, 7):
            want = half_up(Fraction(x, 2 ** s)) if s >= 0 else x * 2 ** (-s)
            assert O.rshift_round(x, s) == want, (x, s)


def test_round_shift_ties_and_negatives():
    # ties go up (towards +inf): -2.5 -> -2, 2.5 -> 3
    assert O.rshift_round(-5, 1) == -2
    assert O.rshift_round(5, 1) == 3
    assert O.rshift_round(-3, 1) == -1
    assert O.rshift_round(-1, 1) == 0
    assert O.rshift_round(-1, 2) == 0
    assert O.rshift_round(-2, 2) == 0
    assert O.rshift_round(-3, 2) == -1


def test_round_shift_random_64bit():
    rng = np.random.default_rng(1)
    for _ in range(3000):
        s = int(rng.integers(1, 62))
        x = int(rng.integers(-(1 << 62), 1 << 62))
        assert O.rshift_round(x, s) == half_up(Fraction(x, 1 << s))


def test_round_shift_overflow_raises():
    with pytest.raises(O.OracleError):
        O.rshift_round(1 << 40, -30)


def test_div_round():
    rng = np.random.default_rng(2)
    for a in range(0, 200):
        for b in range(1, 40):
            assert O.div_round(a, b) == half_up(Fraction(a, b))
    for _ in range(3000):
        a = int(rng.integers(0, 1 << 60))
        b = int(rng.integers(1, 1 << 40))
        assert O.div_round(a, b) == half_up(Fraction(a, b))


def test_isqrt():
    for n in range(0, 70000):
        assert O.isqrt(n) == math.isqrt(n)
    rng = np.random.default_rng(3)
    for _ in range(5000):
        n = int(rng.integers(0, 1 << 63, dtype=np.uint64))
        assert O.isqrt(n) == math.isqrt(n)
    assert O.isqrt((1 << 64) - 1) == math.isqrt((1 << 64) - 1)


def test_bitlen():
    for x in list(range(0, 3000)) + [(1 << k) + d for k in range(1, 63) for d in (-1, 0, 1)]:
        assert O.bitlen(x) == x.bit_length()


def test_dq_definition_and_error_bound():
    rng = np.random.default_rng(4)
    for trial in range(400):
        n = int(rng.integers(1, 300))
        mag = int(rng.integers(0, 46))
        y = rng.integers(-(1 << mag), (1 << mag) + 1, n, dtype=np.int64)
        q, e = O.dq(y)
        A = int(np.abs(y).max())
        # e is the smallest non-negative shift with A / 2^e < 128
        assert A < 2 ** (e + 7)
        assert e == 0 or A >= 2 ** (e + 6)
        for yi, qi in zip(y.tolist(), q.tolist()):
            r = half_up(Fraction(yi, 2 ** e))
            assert qi == max(-127, min(127, r))
            if abs(r) <= 127:
                assert abs(yi - qi * 2 ** e) <= 2 ** e / 2
    # zero row and tiny rows stay exact
    q, e = O.dq(np.zeros(5, np.int64))
    assert e == 0 and not q.any()
    q, e = O.dq(np.array([3, -100, 127], np.int64))
    assert e == 0 and q.tolist() == [3, -100, 127]


def test_irms_relative_error():
    rng = np.random.default_rng(5)
    for n in (1, 2, 64, 128, 256, 1024, 2048, 3072, 8192):
        for _ in range(300):
            b = int(rng.integers(1, 62))
            S = int(rng.integers(1 << (b - 1), 1 << b))
            m, sh = O.irms(S, n)
            assert (1 << 14) <= m < (1 << 15)
            approx = m * 2.0 ** -sh
            exact = 1.0 / math.sqrt(S / n)
            assert abs(approx / exact - 1) < 2 ** -14.5, (S, n, m, sh)


def test_irms_constant_row():
    # a row of n copies of c has 1/rms = 1/|c|
    for c in (1, 3, 1000, 12345, (1 << 25) - 1):
        for n in (64, 1024):
            m, sh = O.irms(c * c * n, n)
            assert abs(m * 2.0 ** -sh * c - 1) < 2 ** -14.5


def test_diexp_special_values_and_monotone():
    assert O.diexp(0) == 1 << 15
    assert O.diexp(-(1 << 15)) == 1 << 14
    assert O.diexp(-(2 << 15)) == 1 << 13
    assert O.diexp(-(40 << 15)) == 0
    prev = 1 << 15
    for u in range(0, -(18 << 15), -37):
        E = O.diexp(u)
        assert 0 <= E <= prev
        prev = E


def test_diexp_closed_form_bound():
    # linear 2^-x ~ 1 - x/2 on [0, 1) overestimates by at most the factor
    # max (1 - x/2) 2^x = 1.0615 (at x = 2 - 1/ln 2); rounding adds <= 1 unit
    cmax = (1 - (2 - 1 / math.log(2)) / 2) * 2 ** (2 - 1 / math.log(2))
    assert 1.0614 < cmax < 1.0615
    for u in range(0, -(17 << 15), -5):
        E = O.diexp(u)
        true = 2.0 ** 15 * 2.0 ** (u / 2.0 ** 15)
        assert true - 1.0 <= E <= cmax * true + 1.0, (u, E, true)


def test_softmax_and_swiglu_multipliers():
    # the dyadic constants represent their real values to 2^-15 relative
    for kq_m, kq_k, d in ((17027, 22, 64), (28857, 23, 128), (16384, 20, 128), (32767, 30, 64)):
        M, K = O.softmax_mult(kq_m, kq_k, d, 12)
        assert (1 << 14) <= M < (1 << 15)
        want = math.log2(math.e) / math.sqrt(d) * 2.0 ** 15 * 2.0 ** kq_k / kq_m * 2.0 ** -24
        assert abs(M * 2.0 ** -K / want - 1) < 2 ** -14.9
    M, K = O.swiglu_mult(12)
    assert abs(M * 2.0 ** -K / (math.log2(math.e) * 8) - 1) < 2 ** -14.9


def test_v_dequant_is_inverse():
    rng = np.random.default_rng(6)
    for _ in range(500):
        vq_m = int(rng.integers(1 << 14, 1 << 15))
        vq_k = int(rng.integers(10, 40))
        m, k = O.v_dequant(vq_m, vq_k)
        assert (1 << 14) <= m < (1 << 15)
        assert abs(vq_m * 2.0 ** -vq_k * m * 2.0 ** -k - 1) < 2 ** -14.4


def test_sigmoid_q15():
    Mg, Kg = O.swiglu_mult(12)
    assert O.sigmoid_q15(0, Mg, Kg) == 1 << 14
    rng = np.random.default_rng(7)
    gs = list(range(-70000, 70000, 97)) + rng.integers(-(1 << 23), 1 << 23, 2000).tolist()
    for g in gs:
        s = O.sigmoid_q15(g, Mg, Kg)
        assert 0 <= s <= 1 << 15
        # exact symmetry s(-g) = 1 - s(g)
        assert O.sigmoid_q15(-g, Mg, Kg) == (1 << 15) - s
        x = g / 4096.0
        sig = 1 / (1 + math.exp(-x)) if x >= 0 else math.exp(x) / (1 + math.exp(x))
        # closed form: DI-Exp overestimates e^-|x| by at most 1.0615 -> error
        # of 1/(1+t) vs 1/(1+1.0615 t) is <= 0.0149; rounding <= 2^-15 + E's unit
        assert abs(s / 2.0 ** 15 - sig) <= 0.0150 + 2 ** -14, (g, s)


def test_rope_tables_closed_form():
    for d, base in ((64, 1_000_000), (128, 1_000_000), (64, 500_000)):
        P = 300
        c, s = O.rope_tables(P, d, base)
        assert (c[0] == 16384).all() and (s[0] == 0).all()
        half = d // 2
        theta = np.array([base ** (-2 * i / d) for i in range(half)])
        for p in range(P):
            ang = p * theta
            assert np.all(np.abs(c[p] - 16384 * np.cos(ang)) <= 0.5 + 1e-9)
            assert np.all(np.abs(s[p] - 16384 * np.sin(ang)) <= 0.5 + 1e-9)
        r2 = c.astype(np.int64) ** 2 + s.astype(np.int64) ** 2
        assert np.all(np.abs(r2 - (1 << 28)) <= 2 * 16384 + 1)
