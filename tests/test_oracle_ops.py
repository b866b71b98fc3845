"""Pins of the oracle's ops: brute force on tiny inputs, a library matmul,
exact rationals, and the real-valued definitions within closed-form bounds."""
import math
from fractions import Fraction

import numpy as np
import pytest

import detint_synth as S
import oracle as O


def half_up(x: Fraction) -> int:
    return math.floor(x + Fraction(1, 2))


# ---------------------------------------------------------------- GEMM

@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (17, 13, 16), (2, 17, 33)])
def test_gemm_bruteforce_python_ints(M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    A = rng.integers(-128, 128, (M, K)).astype(np.int8)
    W = rng.integers(-128, 128, (N, K)).astype(np.int8)
    A[0, 0] = -128
    W[0, 0] = -128
    acc = O.gemm(A, W)
    for i in range(M):
        for j in range(N):
            assert acc[i, j] == sum(int(A[i, k]) * int(W[j, k]) for k in range(K))


def test_gemm_extremes_and_library_matmul():
    K = 3072
    A = np.full((2, K), -128, np.int8)
    W = np.full((3, K), -128, np.int8)
    W[1] = 127
    acc = O.gemm(A, W)
    assert acc[0, 0] == K * 128 * 128 and acc[0, 1] == -K * 128 * 127
    g = S.make_gemm_operands(64, 96, 1024, seed=11)
    acc = O.gemm(g["A"], g["W"])
    np.testing.assert_array_equal(acc, g["A"].astype(np.int64) @ g["W"].astype(np.int64).T)


def test_gemm_wide_weights_match_direct_product():
    rng = np.random.default_rng(12)
    A = rng.integers(-128, 128, (9, 200)).astype(np.int8)
    W16 = rng.integers(-32767, 32768, (31, 200)).astype(np.int16)
    acc = O.gemm(A, W16)
    np.testing.assert_array_equal(acc, A.astype(np.int64) @ W16.astype(np.int64).T)
    # the hi/lo limb identity the GPU path relies on: W16 = 256 * hi + lo
    w = np.arange(-32767, 32768, dtype=np.int64)
    hi, lo = w >> 8, w & 255
    assert hi.min() >= -128 and hi.max() <= 127 and lo.min() >= 0 and lo.max() <= 255
    np.testing.assert_array_equal(256 * hi + lo, w)


def test_gemm_summation_order_free():
    """Exact integer accumulation: any blocking / permutation of K agrees."""
    g = S.make_gemm_operands(8, 40, 1024, seed=13)
    A, W = g["A"], g["W"]
    full = O.gemm(A, W)
    perm = np.random.default_rng(14).permutation(1024)
    np.testing.assert_array_equal(full, O.gemm(A[:, perm], W[:, perm]))
    split = sum(O.gemm(A[:, i:i + 256], W[:, i:i + 256]) for i in range(0, 1024, 256))
    np.testing.assert_array_equal(full, split)


# ------------------------------------------------------------ epilogue

def test_epilogue_modes_against_rationals():
    g = S.make_gemm_operands(5, 7, 1024, seed=15)
    acc = O.gemm(g["A"], g["W"])
    rm, rk, cm, ck = g["row_m"], g["row_k"], g["col_m"], g["col_k"]
    q = O.epilogue(acc, rm, rk, cm, ck, 0, O.REQ_I8)
    fx = O.epilogue(acc, rm, rk, cm, ck, 8, O.FIX)
    base = np.arange(35, dtype=np.int32).reshape(5, 7) * 1000 - 17000
    ra = O.epilogue(acc, rm, rk, cm, ck, 8, O.RES_ADD, out=base)
    raw = O.epilogue(acc, rm, rk, cm, ck, 0, O.RAW)
    clamped = 0
    for i in range(5):
        for j in range(7):
            a = int(acc[i, j])
            r = half_up(Fraction(a * int(rm[i]) * int(cm[j]), 2 ** (int(rk[i]) + ck)))
            clamped += abs(r) > 127
            assert q[i, j] == max(-127, min(127, r))
            y = half_up(Fraction(a * int(rm[i]) * int(cm[j]), 2 ** (int(rk[i]) + ck - 8)))
            assert fx[i, j] == y
            assert ra[i, j] == base[i, j] + y
            assert raw[i, j] == a


def test_epilogue_requant_real_value():
    """out8 approximates acc * (m_r/2^k_r) * (m_c/2^k_c) within half a unit."""
    g = S.make_gemm_operands(64, 512, 3072, seed=16)
    acc = O.gemm(g["A"], g["W"])
    q = O.epilogue(acc, g["row_m"], g["row_k"], g["col_m"], g["col_k"], 0, O.REQ_I8)
    real = (acc * (g["row_m"][:, None] * 2.0 ** -20) * (g["col_m"][None, :] * 2.0 ** -22))
    inside = np.abs(real) < 126.5
    assert np.all(np.abs(q[inside] - real[inside]) <= 0.5 + 1e-9)
    assert np.all(q[~inside] == np.sign(real[~inside]) * 127)
    assert 0 < (~inside).sum() and (~inside).mean() < 0.01   # clamping is exercised


# ------------------------------------------------------------- RMSNorm

def test_rmsnorm_real_value():
    rng = np.random.default_rng(17)
    for n in (64, 256, 1024, 2048):
        h = rng.integers(-(1 << 24), 1 << 24, (12, n)).astype(np.int32)
        h[1] //= 1 << 20      # small-magnitude row
        h[2, :] = 7           # constant row
        g = rng.integers(1 << 12, (1 << 13) + 1, n).astype(np.int16)
        x8, m, k = O.rmsnorm(h, g)
        hf = h.astype(np.float64)
        want = hf / np.sqrt((hf * hf).mean(1, keepdims=True)) * g / 4096.0
        step = m * 2.0 ** -k.astype(np.float64)
        got = x8 * step[:, None]
        err = np.abs(got - want)
        # half an int8 step (one step where the row max rounded to 128 and
        # was clamped) plus the 2^-14.5 relative irms error
        assert np.all(err <= step[:, None] * 1.0 + np.abs(want) * 2 ** -14.4)
        assert np.mean(err <= step[:, None] * 0.5 + np.abs(want) * 2 ** -14.4) > 0.99
        assert np.abs(x8).max(1).min() >= 64


def test_rmsnorm_zero_row_and_bound():
    h = np.zeros((2, 64), np.int32)
    h[1, 3] = 5
    g = np.full(64, 4096, np.int16)
    x8, m, k = O.rmsnorm(h, g)
    assert not x8[0].any() and m[0] == 1 << 14 and k[0] == 26
    # one nonzero entry of 5 among 64: h / rms = 8; DQ keeps it in [64, 128)
    assert 64 <= x8[1, 3] <= 127 and abs(int(x8[1, 3]) * m[1] * 2.0 ** -k[1] - 8.0) < 8.0 / 64
    bad = np.full((1, 64), 1 << 25, np.int32)
    with pytest.raises(O.OracleError):
        O.rmsnorm(bad, g)


def test_rmsnorm_sum_of_squares_domain():
    """The stated domain is a sum of squares below 2^62: the largest rows it
    admits (n = 16384 at |h| = 2^24 - 1, n = 4096 at the 2^25 residual
    bound) normalise to within the real-value bound; one step past it
    (n = 16384 at |h| = 2^24, S = 2^62) is reported as an error."""
    g = np.full(16384, 4096, np.int16)           # gain 1.0
    for n, lim in ((16384, (1 << 24) - 1), (4096, (1 << 25) - 1)):
        h = np.full((2, n), lim, np.int32)
        h[1, ::2] = -lim
        x8, m, k = O.rmsnorm(h, g[:n])
        # every |h| equals the RMS, so each value normalises to +-1
        got = x8 * (m * 2.0 ** -k.astype(np.float64))[:, None]
        assert np.all(np.abs(np.abs(got) - 1.0) <= 2.0 ** -6)
        assert np.array_equal(np.sign(x8), np.sign(h))
    with pytest.raises(O.OracleError):
        O.rmsnorm(np.full((1, 16384), 1 << 24, np.int32), g)


def test_requant_fixed_is_the_rounded_real_product():
    """clamp8 of y * m / 2^k rounded half up, by exact rationals, over values
    that hit both clamps, exact halves and negative halves."""
    from fractions import Fraction
    rng = np.random.default_rng(21)
    y = np.concatenate([rng.integers(-(1 << 24), 1 << 24, 500), [0, 1, -1, 3, -3, 5, -5]]).astype(np.int32)
    for m, k in ((3 << 13, 15), (20000, 30), (1, 0), (16384, 14)):
        q = O.requant_fixed(y, m, k)
        for v, got in zip(y, q):
            want = (Fraction(int(v) * m, 2 ** k) + Fraction(1, 2)).__floor__()
            assert got == max(-127, min(127, want)), (int(v), m, k)


def test_requant_rows():
    rng = np.random.default_rng(18)
    y = rng.integers(-(1 << 22), 1 << 22, (20, 2048)).astype(np.int32)
    q, e = O.requant_rows(y)
    for r in range(20):
        q1, e1 = O.dq(y[r].astype(np.int64))
        assert e1 == e[r]
        np.testing.assert_array_equal(q1, q[r])
        inside = np.abs(y[r] / 2.0 ** e[r]) <= 127
        assert np.all(np.abs(y[r][inside] - q[r][inside] * 2.0 ** e[r]) <= 2.0 ** e[r] / 2)


# ---------------------------------------------------------------- RoPE

def test_rope_identity_at_zero_and_rotation_bound():
    d, P = 128, 600
    cos_t, sin_t = O.rope_tables(P, d, 1_000_000)
    rng = np.random.default_rng(19)
    x = rng.integers(-(1 << 20), 1 << 20, (P, 3, d)).astype(np.int32)
    pos = np.arange(P, dtype=np.int32)
    y = O.rope(x, pos, cos_t, sin_t)
    np.testing.assert_array_equal(y[0], x[0])
    half = d // 2
    theta = 1_000_000.0 ** (-np.arange(half) * 2 / d)
    ang = pos[:, None] * theta[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    a, b = x[..., :half].astype(np.float64), x[..., half:].astype(np.float64)
    ya, yb = a * c - b * s, b * c + a * s
    bound = (np.abs(a) + np.abs(b)) * 2.0 ** -15 + 0.5 + 1e-6
    assert np.all(np.abs(y[..., :half] - ya) <= bound)
    assert np.all(np.abs(y[..., half:] - yb) <= bound)


def test_rope_out_of_table_raises():
    cos_t, sin_t = O.rope_tables(8, 64, 10000)
    with pytest.raises(O.OracleError):
        O.rope(np.zeros((1, 1, 64), np.int32), np.array([8], np.int32), cos_t, sin_t)


# ------------------------------------------------------------- softmax

def _float_softmax(s, valid, M, K, shift):
    x = (s[:valid].astype(np.float64) - s[:valid].max()) * M * 2.0 ** -(K - shift) / 2.0 ** 15
    p = 2.0 ** x
    return p / p.sum()


def test_softmax_properties():
    M, K = O.softmax_mult(28857, 23, 128, 12)
    rng = np.random.default_rng(20)
    R_, Cc = 64, 600
    s = rng.integers(-60000, 60000, (R_, Cc)).astype(np.int32)
    valid = rng.integers(1, Cc + 1, R_).astype(np.int32)
    valid[0] = 1
    valid[1] = Cc
    shift = rng.integers(0, 12, R_).astype(np.int32)
    P = O.softmax(s, valid, shift, M, K)
    assert P[0, 0] == 32767 and not P[0, 1:].any()     # single key -> cap 2^15 - 1
    cmax = 1.0615
    for r in range(R_):
        v = int(valid[r])
        p = P[r, :v].astype(np.int64)
        assert not P[r, v:].any()                        # masked -> 0
        assert abs(int(p.sum()) - (1 << 15)) <= v / 2 + 1 + (p.max() == 32767)
        order = np.argsort(s[r, :v], kind="stable")
        assert np.all(np.diff(p[order]) >= 0)             # monotone in the score
        ref = _float_softmax(s[r], v, M, K, int(shift[r]))
        big = ref * 2 ** 15 > 64
        ratio = p[big] / (ref[big] * 2 ** 15)
        assert np.all(ratio > 1 / cmax - 0.02) and np.all(ratio < cmax + 0.02)


def test_softmax_equal_scores():
    M, K = O.softmax_mult(28857, 23, 128, 12)
    s = np.full((3, 10), 1234, np.int32)
    P = O.softmax(s, np.array([10, 7, 4], np.int32), np.zeros(3, np.int32), M, K)
    for r, v in enumerate((10, 7, 4)):
        assert len(set(P[r, :v].tolist())) == 1
        assert abs(int(P[r, :v].sum()) - 32768) <= v


# -------------------------------------------------------------- SwiGLU

def test_swiglu_real_value():
    rng = np.random.default_rng(21)
    R_, n = 16, 768
    g = rng.normal(0, 6 * 4096, (R_, n)).astype(np.int64)
    u = rng.normal(0, 6 * 4096, (R_, n)).astype(np.int64)
    gu = np.concatenate([g, u], 1).astype(np.int32)
    a8, m, k = O.swiglu(gu, 12)
    gf, uf = g / 4096.0, u / 4096.0
    want = gf / (1 + np.exp(-gf)) * uf
    got = a8 * (m * 2.0 ** -k.astype(np.float64))[:, None]
    step = (m * 2.0 ** -k.astype(np.float64))[:, None]
    # sigmoid error <= 0.0151 absolute -> silu error <= 0.0151 |g|; plus DQ step
    assert np.all(np.abs(got - want) <= 0.0152 * np.abs(gf * uf) + step + 2 ** -11 * np.abs(uf) + 1e-9)


def test_swiglu_zero_gate_and_bound():
    gu = np.zeros((1, 8), np.int32)
    gu[0, 4:] = 4096
    a8, m, k = O.swiglu(gu, 12)
    assert not a8.any()
    bad = np.zeros((1, 8), np.int32)
    bad[0, 0] = 1 << 24
    with pytest.raises(O.OracleError):
        O.swiglu(bad, 12)


# ----------------------------------------------------- argmax and hash

def test_argmax_lowest_id_on_ties():
    rng = np.random.default_rng(22)
    L = rng.integers(-1000, 1000, (50, 300)).astype(np.int32)
    L[3, 10] = L[3, 200] = 5000
    L[4, :] = 7
    L[5, 299] = L[5, 298] = 4000
    got = O.argmax(L)
    np.testing.assert_array_equal(got, np.argmax(L, axis=1))   # numpy picks the first maximum
    assert got[3] == 10 and got[4] == 0 and got[5] == 298


def test_hash_chain_sensitivity():
    import hashlib
    row = np.arange(-5, 100, dtype=np.int32)
    h1 = O.chain_step(O.chain_init(), row)
    assert h1 == hashlib.sha256(hashlib.sha256(b"detint-v0").digest()
                                + b"".join(int(v).to_bytes(4, "little", signed=True) for v in row)).digest()
    row2 = row.copy()
    row2[7] ^= 1
    assert O.chain_step(O.chain_init(), row2) != h1
