"""Pins of the oracle's exact mode (BitExact LLM blog, "Three execution
paths": exact mode keeps the bf16 weights and multiplies them with
fixed-point activations; "Fix the arithmetic": integer limbs, wide
accumulators) against what the bf16 format and exact rational arithmetic fix,
independently of the oracle's code:

* a bf16 pattern's value is the float32 whose upper 16 bits it is
  (IEEE 754 binary32 truncated), so the integer form times its row's power
  of two must equal that float exactly, for normals, subnormals, signed
  zeros and both ends of the exponent range;
* the product with int8 activations is the exact rational sum of a * w;
* the epilogue rounds that rational (scaled) to the nearest integer with
  halves up."""
from fractions import Fraction

import numpy as np
import pytest

import detint_synth as S
import oracle as O


def _bits(vals):
    return np.array(vals, np.uint16)


def test_weight_integers_are_the_bf16_values():
    rng = np.random.default_rng(1)
    rows = []
    # a row of normals over an exponent span of exactly 23, both signs
    e = rng.integers(100, 124, 64)
    f = rng.integers(0, 128, 64)
    sgn = rng.integers(0, 2, 64)
    e[0], e[1] = 100, 123
    rows.append((sgn << 15) | (e << 7) | f)
    # subnormals (exponent field 0), zeros, the smallest normal
    rows.append(np.array([0x0001, 0x807F, 0x0000, 0x8000, 0x0080, 0x0040] + [0x0003] * 58))
    # the largest finite exponents
    rows.append(np.array([0x7F7F, 0xFF00, 0x7E80, 0x7F00] * 16))
    # an all-zero row
    rows.append(np.zeros(64, np.int64))
    Wb = np.array(rows, np.uint16)
    W_int, row_exp = O.exact_weights(Wb)
    real = S.bf16_to_float64(Wb)
    for j in range(Wb.shape[0]):
        for k in range(Wb.shape[1]):
            assert Fraction(int(W_int[j, k])) * Fraction(2) ** int(row_exp[j]) == Fraction(real[j, k]), (j, k)
    assert np.abs(W_int).max() < 2 ** 31
    # a row's smallest nonzero magnitude has the row's scale, so its integer is the mantissa
    assert np.abs(W_int[0, 0]) in range(128, 256)


def test_weights_outside_the_format_are_errors():
    with pytest.raises(O.OracleError):
        O.exact_weights(_bits([[0x3F80, 0x7F80]]))          # infinity
    with pytest.raises(O.OracleError):
        O.exact_weights(_bits([[0x3F80, 0x7FC1]]))          # NaN
    with pytest.raises(O.OracleError):
        O.exact_weights(_bits([[0x3F80, 0x3300]]))          # exponents 127 and 102: span 25
    O.exact_weights(_bits([[0x3F80, 0x3400]]))              # span 23 is fine


def test_exact_product_is_the_rational_sum():
    rng = np.random.default_rng(2)
    M, N, K = 5, 7, 48
    Wb = S.make_bf16_weights(N, K, seed=3)
    W_int, row_exp = O.exact_weights(Wb)
    A = rng.integers(-128, 128, (M, K)).astype(np.int8)
    A[0] = -128
    acc = O.gemm_exact(A, W_int)
    real = S.bf16_to_float64(Wb)
    for i in range(M):
        for j in range(N):
            want = sum(Fraction(int(A[i, k])) * Fraction(real[j, k]) for k in range(K))
            assert Fraction(int(acc[i, j])) * Fraction(2) ** int(row_exp[j]) == want


def test_exact_epilogue_rounds_the_real_output():
    rng = np.random.default_rng(4)
    M, N, K = 6, 9, 64
    Wb = S.make_bf16_weights(N, K, seed=5)
    W_int, row_exp = O.exact_weights(Wb)
    A = rng.integers(-127, 128, (M, K)).astype(np.int8)
    rm = rng.integers(1 << 14, 1 << 15, M).astype(np.int32)
    rk = rng.integers(10, 20, M).astype(np.int32)
    acc = O.gemm_exact(A, W_int)
    real = S.bf16_to_float64(Wb)
    fix = O.exact_epilogue(acc, rm, rk, row_exp, 16, O.FIX)
    q = O.exact_epilogue(acc, rm, rk, row_exp, 0, O.REQ_I8)
    raw = O.exact_epilogue(acc, rm, rk, row_exp, 0, O.RAW)
    assert np.array_equal(raw, acc)
    half = Fraction(1, 2)
    for i in range(M):
        x = Fraction(int(rm[i]), 2 ** int(rk[i]))          # the activation row's scale
        for j in range(N):
            v = x * sum(Fraction(int(A[i, k])) * Fraction(real[j, k]) for k in range(K))
            f = v * 2 ** 16
            assert fix[i, j] == (f + half).__floor__(), (i, j)
            assert q[i, j] == max(-127, min(127, (v + half).__floor__())), (i, j)


def test_generated_bf16_weights_round_to_nearest_even():
    """The synthetic bf16 draw is round-to-nearest-even of the float32 draw:
    every pattern is within half a bf16 unit of some float32, and its value
    sits in the row's span."""
    Wb = S.make_bf16_weights(32, 256, seed=6)
    assert Wb.dtype == np.uint16
    E = (Wb >> 7) & 255
    assert (E != 255).all()
    nz = Wb & 0x7FFF != 0
    span = np.array([E[j][nz[j]].max() - E[j][nz[j]].min() for j in range(32)])
    assert span.max() <= 23
    v = S.bf16_to_float64(Wb)
    assert 0.015 < v.std() < 0.025
