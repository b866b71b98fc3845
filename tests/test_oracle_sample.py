"""Pins of the oracle's integer sampling (temperature + top-k) against what the
definition fixes independently: greedy selection at k = 1, closed forms for
equal logits, a cold temperature, monotonicity in the draw, the top-k support,
and the real-valued softmax distribution within DI-Exp's error bound."""
import math

import numpy as np
import pytest

import oracle as O

# log2(e) / 2 as a dyadic: logits carry 16 fractional bits and DI-Exp takes a
# base-2 exponent in Q15, so temperature 1 is t_m / 2^t_k = log2(e) / 2
T1_M, T1_K = 23637, 15


def _draws(rng, n):
    d = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
    d[:2] = [0, (1 << 32) - 1]
    return d


def test_top1_is_greedy():
    rng = np.random.default_rng(1)
    logits = rng.integers(-5, 5, (64, 50)).astype(np.int32) * 65536  # many ties
    got = O.sample(logits, 1, T1_M, T1_K, _draws(rng, 64))
    np.testing.assert_array_equal(got, np.argmax(logits, axis=1))  # first maximum


@pytest.mark.parametrize("V", [1, 7, 1000, 151936])
def test_equal_logits_uniform(V):
    rng = np.random.default_rng(V)
    r = _draws(rng, 16)
    logits = np.full((16, V), -123456, np.int32)
    want = (r.astype(object) * V) >> 32
    np.testing.assert_array_equal(O.sample(logits, 0, T1_M, T1_K, r), want.astype(np.int32))
    np.testing.assert_array_equal(O.sample(logits, V, T1_M, T1_K, r), want.astype(np.int32))


def test_top_k_takes_lowest_ids_among_ties():
    rng = np.random.default_rng(3)
    r = _draws(rng, 32)
    logits = np.full((32, 300), 7, np.int32)
    want = ((r.astype(object) * 5) >> 32).astype(np.int32)  # ids 0..4 kept, equal weight
    np.testing.assert_array_equal(O.sample(logits, 5, T1_M, T1_K, r), want)


def test_cold_temperature_picks_among_maxima():
    rng = np.random.default_rng(4)
    logits = rng.integers(-1000, 1000, (8, 200)).astype(np.int32)
    r = _draws(rng, 8)
    for o in range(8):
        logits[o, rng.choice(200, 3, replace=False)] = 5000  # three tied maxima
    got = O.sample(logits, 0, 1 << 23, 0, r)  # a gap of 1 already gives E = 0
    for o in range(8):
        ties = np.flatnonzero(logits[o] == 5000)
        assert got[o] == ties[(int(r[o]) * 3) >> 32]


def test_monotone_in_draw_and_inside_top_k():
    rng = np.random.default_rng(5)
    V, k = 40, 10
    row = rng.integers(-3 << 16, 3 << 16, V).astype(np.int32)
    row[[3, 17]] = row.max()  # a tie at the top
    r = np.sort(_draws(rng, 4096))
    got = O.sample(np.tile(row, (4096, 1)), k, T1_M, T1_K, r)
    assert np.all(np.diff(got) >= 0)
    order = np.lexsort((np.arange(V), -row.astype(np.int64)))  # logit desc, id asc
    assert set(got.tolist()) <= set(order[:k].tolist())
    assert {3, 17} <= set(got.tolist())


def test_distribution_matches_softmax():
    """Draws on a uniform grid: each token's share equals E_j / D up to the
    grid step, and E_j / E_max is within DI-Exp's linear-fraction bound
    (1 <= (1 - r/2) / 2^-r <= 1.0615) plus rounding of the real softmax at
    temperature 1 (logits with 16 fractional bits)."""
    rng = np.random.default_rng(6)
    V, N = 64, 1 << 16
    row = rng.integers(-4 << 16, 4 << 16, V).astype(np.int32)
    r = ((np.arange(N, dtype=np.uint64) * (1 << 32) + (1 << 31)) // N).astype(np.uint32)
    got = O.sample(np.tile(row, (N, 1)), 0, T1_M, T1_K, r)
    freq = np.bincount(got, minlength=V) / N
    x = row.astype(np.float64) / 65536.0
    p = np.exp(x - x.max())
    p /= p.sum()
    # each weight within [1, 1.0615] x its real value (plus the Q15 rounding),
    # so each normalised share within a factor 1.0615^(+-1) of the softmax
    big = p > 1e-3
    ratio = freq[big] / p[big]
    assert np.all(ratio > 1 / 1.07 - 2 / (N * p[big])) and np.all(ratio < 1.07 + 2 / (N * p[big]))
    assert math.isclose(freq.sum(), 1.0)


# ------------------------------------------------------------------ top-p

def test_top_p_smallest_is_greedy():
    rng = np.random.default_rng(21)
    logits = rng.integers(-5, 5, (64, 50)).astype(np.int32) * 65536
    got = O.sample(logits, 0, T1_M, T1_K, _draws(rng, 64), top_p=1)
    np.testing.assert_array_equal(got, np.argmax(logits, axis=1))


@pytest.mark.parametrize("top_p,kept", [(32768, 5), (32769, 6), (65535, 10), (6553, 1), (6554, 2)])
def test_top_p_equal_logits(top_p, kept):
    """Ten equal logits weigh 2^15 each: P = ceil(top_p * 10 * 2^15 / 2^16)
    keeps ceil(P / 2^15) of them, the lowest ids."""
    rng = np.random.default_rng(top_p)
    r = _draws(rng, 64)
    logits = np.full((64, 10), 99, np.int32)
    want = ((r.astype(object) * kept) >> 32).astype(np.int32)
    np.testing.assert_array_equal(O.sample(logits, 0, T1_M, T1_K, r, top_p=top_p), want)


def test_top_p_after_top_k():
    rng = np.random.default_rng(22)
    r = _draws(rng, 64)
    logits = np.full((64, 40), 5, np.int32)
    # top-3 first: D_k = 3 * 2^15; p just below 1 still needs all three
    want = ((r.astype(object) * 3) >> 32).astype(np.int32)
    np.testing.assert_array_equal(O.sample(logits, 3, T1_M, T1_K, r, top_p=65535), want)
    # P = ceil(21845 * 3 * 2^15 / 2^16) = 2^15: exactly one; one more unit of p needs two
    np.testing.assert_array_equal(O.sample(logits, 3, T1_M, T1_K, r, top_p=21845), np.zeros(64, np.int32))
    want2 = ((r.astype(object) * 2) >> 32).astype(np.int32)
    np.testing.assert_array_equal(O.sample(logits, 3, T1_M, T1_K, r, top_p=21846), want2)


def test_top_p_nucleus_is_a_rank_prefix_of_the_right_mass():
    rng = np.random.default_rng(23)
    V, N = 200, 1 << 14
    row = rng.normal(0, 2 * 65536, V).astype(np.int32)
    r = ((np.arange(N, dtype=np.uint64) * (1 << 32) + (1 << 31)) // N).astype(np.uint32)
    got = O.sample(np.tile(row, (N, 1)), 0, T1_M, T1_K, r, top_p=int(0.9 * 65536))
    order = np.lexsort((np.arange(V), -row.astype(np.int64)))  # rank order
    rank = np.empty(V, np.int64)
    rank[order] = np.arange(V)
    reached = np.unique(got)
    m = rank[reached].max() + 1
    assert set(rank[reached].tolist()) <= set(range(m))
    x = row.astype(np.float64) / 65536.0
    p = np.exp(x - x.max())
    p /= p.sum()
    mass = p[order[:m]].sum()
    # the kept prefix reaches 0.9 of the (integer) mass; DI-Exp's weights are
    # within 7% of the real ones, so the real mass of that prefix is near 0.9
    assert 0.8 < mass < 0.97
    assert p[order[m - 1]] > 0  # the last kept id carries weight
