"""GPU parity of every libdetint op against the CPU oracle, bit for bit
(tolerance 0: every result is an integer). Inputs are seeded synthetic data;
sizes span several tiles plus ragged tails; the full-size GEMM sweep is
checked on every output element."""
import numpy as np
import pytest

import detint_synth as S
import oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def D():
    import torch
    import integer_only_deterministic_amd as D
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    D.library()
    return D


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


# ------------------------------------------------------------------ GEMM

@pytest.mark.parametrize("K,N", S.GEMM_SWEEP_KN)
def test_gemm_sweep(D, K, N):
    import torch
    """The standalone sweep: M in {1, 8, 64, 512, 2048} x the five projection
    shapes, RAW int32 and per-row x per-column requant to int8, every output
    element against the oracle's int64 brute force."""
    for M in S.GEMM_SWEEP_M:
        g = S.make_gemm_operands(M, N, K, seed=7)
        A, W = dev(g["A"]), dev(g["W"])
        rm, rk, cm = dev(g["row_m"]), dev(g["row_k"]), dev(g["col_m"])
        acc = O.gemm(g["A"], g["W"])                 # every row, int64 brute force
        want = O.epilogue(acc, g["row_m"], g["row_k"], g["col_m"], g["col_k"], 0, O.REQ_I8)
        need = D.detint_gemm_workspace(M, N, K)
        for ws in (None, torch.empty(max(need, 16), dtype=torch.uint8, device="cuda") if need else None):
            raw = host(D.detint_gemm_i8(A, W, ws=ws))
            q = host(D.detint_gemm_i8(A, W, rm, rk, cm, g["col_k"], 0, D.REQ_I8, ws=ws))
            tag = f"M={M} N={N} K={K} ws={ws is not None}"
            np.testing.assert_array_equal(raw, acc, err_msg=f"RAW {tag}")
            np.testing.assert_array_equal(q, want, err_msg=f"REQ_I8 {tag}")
            if need == 0:
                break
        del A, W, acc, want, raw, q


# K % 128 == 0 shapes take the pipelined kernel; (200, 300, 256),
# (1000, 1590, 256), (1000, 3000, 256), (1000, 6100, 256) and (2000, 6000,
# 128) are sized so that its 64x64, 128x64, 128x128, 128x256 and 256x256
# tilings are each chosen, with ragged M and N edges.
# 16 < M <= 64 with K % 512 == 0 takes the skinny kernel (one or two 32-row
# tiles; (40, 16400, 512) two 32-column tiles per workgroup, the last one
# ragged).
@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (3, 5, 48), (16, 77, 32), (17, 130, 64),
                                   (37, 300, 112), (129, 257, 80), (200, 64, 1024), (300, 1000, 3072),
                                   (200, 300, 256), (1000, 1590, 256), (1000, 3000, 256), (1000, 6100, 256),
                                   (2000, 6000, 128),
                                   (32, 1000, 2048), (20, 100, 512), (50, 77, 1024),
                                   (5, 300, 1040), (8, 333, 2064),
                                   (300, 1000, 8192), (40, 700, 4096), (512, 1024, 16384),
                                   (40, 16400, 512)])
def test_gemm_ragged_all_modes(D, M, N, K):
    import torch
    rng = np.random.default_rng(M * 7 + N + K)
    A = rng.integers(-128, 128, (M, K)).astype(np.int8)
    W = rng.integers(-128, 128, (N, K)).astype(np.int8)
    A[0, :] = -128
    W[0, :] = -128
    rm = rng.integers(1 << 14, 1 << 15, M).astype(np.int32)
    rk = rng.integers(14, 22, M).astype(np.int32)
    cm = rng.integers(1 << 14, 1 << 15, N).astype(np.int32)
    acc = O.gemm(A, W)
    base = rng.integers(-(1 << 20), 1 << 20, (M, N)).astype(np.int32)
    dA, dW, drm, drk, dcm = dev(A), dev(W), dev(rm), dev(rk), dev(cm)
    need = D.detint_gemm_workspace(M, N, K)
    # with a workspace, few-tile shapes split K (skinny last-arriver sums or
    # pipelined partials plus a summing epilogue); same bits
    for ws in (None, torch.empty(max(need, 16), dtype=torch.uint8, device="cuda") if need else None):
        np.testing.assert_array_equal(host(D.detint_gemm_i8(dA, dW, ws=ws)), acc)
        np.testing.assert_array_equal(host(D.detint_gemm_i8(dA, dW, drm, drk, dcm, 22, 0, D.REQ_I8, ws=ws)),
                                      O.epilogue(acc, rm, rk, cm, 22, 0, O.REQ_I8))
        np.testing.assert_array_equal(host(D.detint_gemm_i8(dA, dW, drm, drk, dcm, 22, 8, D.FIX, ws=ws)),
                                      O.epilogue(acc, rm, rk, cm, 22, 8, O.FIX))
        out = dev(base)
        D.detint_gemm_i8(dA, dW, drm, drk, dcm, 22, 8, D.RES_ADD, out=out, ws=ws)
        np.testing.assert_array_equal(host(out), O.epilogue(acc, rm, rk, cm, 22, 8, O.RES_ADD, out=base))
        if need == 0:
            break


@pytest.mark.parametrize("mode", ["REQ_I8", "FIX", "RES_ADD"])
@pytest.mark.parametrize("M", [512, 6])
def test_gemm_general_scales(D, mode, M):
    """Mantissas >= 2^15 and (for REQ_I8) shifts from -3 to 70: at M = 512 an
    all-interior 64x64 tiling takes the pipelined kernel's general
    epilogue, not its in-range fast path; at M = 6 the GEMV's epilogue."""
    N, K = 512, 256
    rng = np.random.default_rng(99)
    A = rng.integers(-128, 128, (M, K)).astype(np.int8)
    W = rng.integers(-128, 128, (N, K)).astype(np.int8)
    rm = rng.integers(1 << 14, 1 << 15, M).astype(np.int32)
    rm[::7] = rng.integers(1 << 15, 1 << 20, len(rm[::7]))
    cm = rng.integers(1 << 14, 1 << 15, N).astype(np.int32)
    if mode == "REQ_I8":
        rk = rng.integers(-25, 49, M).astype(np.int32)          # shift = rk + 22
    else:
        rk = rng.integers(40, 49, M).astype(np.int32)           # FIX/RES results stay in int32
    acc = O.gemm(A, W)
    dA, dW, drm, drk, dcm = dev(A), dev(W), dev(rm), dev(rk), dev(cm)
    md = getattr(D, mode)
    if mode == "RES_ADD":
        base = rng.integers(-(1 << 20), 1 << 20, (M, N)).astype(np.int32)
        out = dev(base)
        D.detint_gemm_i8(dA, dW, drm, drk, dcm, 22, 8, md, out=out)
        want = O.epilogue(acc, rm, rk, cm, 22, 8, O.RES_ADD, out=base)
        np.testing.assert_array_equal(host(out), want)
    else:
        got = host(D.detint_gemm_i8(dA, dW, drm, drk, dcm, 22, 8, md))
        np.testing.assert_array_equal(got, O.epilogue(acc, rm, rk, cm, 22, 8, getattr(O, mode)))


def test_gemm_empty(D):
    import torch
    A = torch.zeros((0, 32), dtype=torch.int8, device="cuda")
    W = torch.zeros((5, 32), dtype=torch.int8, device="cuda")
    assert D.detint_gemm_i8(A, W).shape == (0, 5)


# (33, 130, 512) and (300, 200, 1024) take the pipelined kernel's 128x128
# limb tiling, (1000, 6100, 128) its 256x128 one; (32, 130, 2048) and
# (17, 300, 512) the skinny kernel, (29, 16400, 512) its two-tile
# workgroups with a ragged last tile.
@pytest.mark.parametrize("M,N,K", [(1, 100, 2048), (7, 300, 256), (16, 64, 8192), (33, 130, 512),
                                   (300, 200, 1024), (1000, 6100, 128), (32, 130, 2048), (17, 300, 512),
                                   (29, 16400, 512)])
def test_gemm_w16_limbs(D, M, N, K):
    rng = np.random.default_rng(M + N + K)
    A = rng.integers(-128, 128, (M, K)).astype(np.int8)
    W16 = rng.integers(-32767, 32768, (N, K)).astype(np.int16)
    W16[0, :] = -32767
    W16[1, :] = 32767
    rm = rng.integers(1 << 14, 1 << 15, M).astype(np.int32)
    rk = rng.integers(14, 22, M).astype(np.int32)
    cm = rng.integers(1 << 14, 1 << 15, N).astype(np.int32)
    hi, lo = D.detint_split_w16(dev(W16))
    w = W16.astype(np.int64)
    np.testing.assert_array_equal(host(hi), (w >> 8).astype(np.int8))
    np.testing.assert_array_equal(host(lo), ((w & 255) - 128).astype(np.int8))
    acc = O.gemm(A, W16)
    dA, drm, drk, dcm = dev(A), dev(rm), dev(rk), dev(cm)
    need = D.detint_gemm_workspace(M, N, K, limbs=True)
    if need:                  # skinny limb shapes: split K with a workspace, same bits
        import torch
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        np.testing.assert_array_equal(host(D.detint_gemm_w16(dA, hi, lo, ws=ws)), acc)
        np.testing.assert_array_equal(host(D.detint_gemm_w16(dA, hi, lo, drm, drk, dcm, 30, 12, D.FIX, ws=ws)),
                                      O.epilogue(acc, rm, rk, cm, 30, 12, O.FIX))
    np.testing.assert_array_equal(host(D.detint_gemm_w16(dA, hi, lo)), acc)
    np.testing.assert_array_equal(host(D.detint_gemm_w16(dA, hi, lo, drm, drk, dcm, 30, 12, D.FIX)),
                                  O.epilogue(acc, rm, rk, cm, 30, 12, O.FIX))
    np.testing.assert_array_equal(host(D.detint_gemm_w16(dA, hi, lo, drm, drk, dcm, 30, 0, D.REQ_I8)),
                                  O.epilogue(acc, rm, rk, cm, 30, 0, O.REQ_I8))
    base = rng.integers(-(1 << 20), 1 << 20, (M, N)).astype(np.int32)
    out = dev(base)
    D.detint_gemm_w16(dA, hi, lo, drm, drk, dcm, 30, 12, D.RES_ADD, out=out)
    np.testing.assert_array_equal(host(out), O.epilogue(acc, rm, rk, cm, 30, 12, O.RES_ADD, out=base))


# -------------------------------------------------------------- row ops

@pytest.mark.parametrize("R,n", [(1, 1024), (5, 256), (64, 768), (33, 2048), (3, 4096),
                                 (6, 8192), (7, 1022)])
def test_rmsnorm(D, R, n):
    rng = np.random.default_rng(R * n)
    h = rng.integers(-(1 << 24), 1 << 24, (R, n)).astype(np.int32)
    h[0, :] = 0
    if R > 2:
        h[1] //= 1 << 18
        h[2, :] = -77
    g = rng.integers(1 << 12, (1 << 13) + 1, n).astype(np.int16)
    x8, m, k = D.detint_rmsnorm(dev(h), dev(g))
    ox, om, ok = O.rmsnorm(h, g)
    np.testing.assert_array_equal(host(x8), ox)
    np.testing.assert_array_equal(host(m), om)
    np.testing.assert_array_equal(host(k), ok)


def test_rmsnorm_largest_rows(D):
    """The largest rows the stated domain admits: n = 16384 at |h| = 2^24 - 1
    (sum of squares just under 2^62), and n = 4096 at the +-(2^25 - 1)
    residual bound, with mixed signs and one all-maximum row."""
    rng = np.random.default_rng(16384)
    for n, lim in ((16384, (1 << 24) - 1), (4096, (1 << 25) - 1)):
        h = rng.choice([-lim, lim], (3, n)).astype(np.int32)
        h[1] = lim
        h[2, ::2] = rng.integers(-lim, lim + 1, n // 2)
        g = rng.integers(1 << 12, (1 << 13) + 1, n).astype(np.int16)
        x8, m, k = D.detint_rmsnorm(dev(h), dev(g))
        ox, om, ok = O.rmsnorm(h, g)
        np.testing.assert_array_equal(host(m), om, err_msg=f"n={n}")
        np.testing.assert_array_equal(host(k), ok, err_msg=f"n={n}")
        np.testing.assert_array_equal(host(x8), ox, err_msg=f"n={n}")


@pytest.mark.parametrize("n", [64, 128, 768, 1024, 2048, 4096])
def test_rmsnorm_magnitudes(D, n):
    """The integer square root and divisions of irms over the whole range of
    row magnitudes: row i is scaled to about 2^(i % 26), some rows hold a
    single nonzero element, some sit at the +-2^25 residual bound."""
    R = 416
    rng = np.random.default_rng(n + 7)
    h = rng.integers(-(1 << 25) + 1, 1 << 25, (R, n)).astype(np.int64)
    for i in range(R):
        h[i] >>= 25 - (i % 26)
    h[::7, 1:] = 0                                   # one nonzero element
    h[3::11] = rng.choice([-(1 << 25) + 1, (1 << 25) - 1], (len(h[3::11]), n))
    h = h.astype(np.int32)
    g = rng.integers(1 << 12, (1 << 13) + 1, n).astype(np.int16)
    x8, m, k = D.detint_rmsnorm(dev(h), dev(g))
    ox, om, ok = O.rmsnorm(h, g)
    np.testing.assert_array_equal(host(m), om)
    np.testing.assert_array_equal(host(k), ok)
    np.testing.assert_array_equal(host(x8), ox)


@pytest.mark.parametrize("R,n", [(1, 2048), (9, 512), (70, 4096), (5, 8192), (4, 1030)])
def test_requant(D, R, n):
    rng = np.random.default_rng(R + n)
    y = rng.integers(-(1 << 22), 1 << 22, (R, n)).astype(np.int32)
    y[0, :] = 0
    y[-1, :] = rng.integers(-100, 100, n)
    q, e = D.detint_requant(dev(y))
    oq, oe = O.requant_rows(y)
    np.testing.assert_array_equal(host(q), oq)
    np.testing.assert_array_equal(host(e), oe)


@pytest.mark.parametrize("n", [1, 7, 4096, 100003])
def test_requant_fixed(D, n):
    rng = np.random.default_rng(n)
    y = rng.integers(-(1 << 24), 1 << 24, n).astype(np.int32)
    for m, k in ((3 << 13, 15), (20000, 30), (1, 0)):
        np.testing.assert_array_equal(host(D.detint_requant_fixed(dev(y), m, k)), O.requant_fixed(y, m, k))


@pytest.mark.parametrize("d,base", [(64, 1_000_000), (128, 1_000_000), (64, 500_000)])
def test_rope(D, d, base):
    P = 600
    cos_t, sin_t = D.detint_rope_tables(P, d, base)
    rng = np.random.default_rng(d)
    x = rng.integers(-(1 << 22), 1 << 22, (50, 3, d)).astype(np.int32)
    pos = rng.integers(0, P, 50).astype(np.int32)
    pos[0] = 0
    pos[1] = P - 1
    y = D.detint_rope(dev(x), dev(pos), dev(cos_t), dev(sin_t))
    np.testing.assert_array_equal(host(y), O.rope(x, pos, cos_t, sin_t))


def test_softmax(D):
    rng = np.random.default_rng(3)
    R, Cc = 40, 700
    s = rng.integers(-200000, 200000, (R, Cc)).astype(np.int32)
    s[5, :] = 1234
    valid = rng.integers(1, Cc + 1, R).astype(np.int32)
    valid[0], valid[1] = 1, Cc
    shift = rng.integers(0, 12, R).astype(np.int32)
    M, K = O.softmax_mult(28857, 23, 128, 12)
    P = D.detint_softmax(dev(s), dev(valid), dev(shift), M, K)
    np.testing.assert_array_equal(host(P), O.softmax(s, valid, shift, M, K))


# More than 64 rows take the persistent kernel with the sigmoid quotients in
# LDS (ragged against its 512-workgroup grid at 700 rows).
@pytest.mark.parametrize("R,n", [(1, 3072), (13, 768), (4, 8192), (3, 998), (2, 4100), (65, 3072),
                                 (700, 8192), (130, 4100)])
def test_swiglu(D, R, n):
    rng = np.random.default_rng(R * 3 + n)
    gu = rng.normal(0, 8 * 4096, (R, 2 * n)).astype(np.int32)
    gu[0, :n] = 0
    gu[-1, 5] = (1 << 24) - 1
    gu[-1, 6] = -(1 << 24) + 1
    a8, m, k = D.detint_swiglu(dev(gu), 12)
    oa, om, ok = O.swiglu(gu, 12)
    np.testing.assert_array_equal(host(a8), oa)
    np.testing.assert_array_equal(host(m), om)
    np.testing.assert_array_equal(host(k), ok)


@pytest.mark.parametrize("f_a", [14, 15])
def test_swiglu_64_bit_form(D, f_a):
    """The table kernel's 64-bit form: f_a = 14, 15 give the sigmoid shift
    K = f_a - 1 > 12, where the 32-bit form's product bound does not hold
    (f_a = 12, every other test, takes the 32-bit form)."""
    rng = np.random.default_rng(f_a)
    R, n = 130, 4100
    gu = rng.normal(0, 8 * 4096, (R, 2 * n)).astype(np.int32)
    gu[1, 7] = (1 << 24) - 1
    gu[1, 8] = -(1 << 24) + 1
    a8, m, k = D.detint_swiglu(dev(gu), f_a)
    oa, om, ok = O.swiglu(gu, f_a)
    np.testing.assert_array_equal(host(a8), oa)
    np.testing.assert_array_equal(host(m), om)
    np.testing.assert_array_equal(host(k), ok)


def test_swiglu_every_gate(D):
    """Every gate value in [-2^17, 2^17) exactly once (256 shuffled rows of
    1024, so the table-driven kernel runs): with f_a = 12 larger gates all give
    DI-Exp output 0, so this reaches every sigmoid quotient a gate can select."""
    rng = np.random.default_rng(17)
    g = rng.permutation(np.arange(-(1 << 17), 1 << 17, dtype=np.int64)).astype(np.int32)
    u = rng.integers(-(1 << 16), 1 << 16, g.size).astype(np.int32)
    gu = np.concatenate([g.reshape(256, 1024), u.reshape(256, 1024)], axis=1)
    a8, m, k = D.detint_swiglu(dev(gu), 12)
    oa, om, ok = O.swiglu(gu, 12)
    np.testing.assert_array_equal(host(a8), oa)
    np.testing.assert_array_equal(host(m), om)
    np.testing.assert_array_equal(host(k), ok)


# ------------------------------------------------------------- attention

def _cache(rng, slots, nkv, max_pos, d):
    k = rng.integers(-127, 128, (slots, nkv, max_pos, d)).astype(np.int8)
    v = rng.integers(-127, 128, (slots, nkv, max_pos, d)).astype(np.int8)
    return k, v


@pytest.mark.parametrize("nq,nkv,d,max_pos", [(4, 2, 64, 256), (16, 8, 128, 1024), (32, 8, 64, 4096),
                                              (8, 8, 128, 300)])
def test_attention_prefill_and_decode(D, nq, nkv, d, max_pos):
    rng = np.random.default_rng(nq * d + max_pos)
    slots = 3
    kc, vc = _cache(rng, slots, nkv, max_pos, d)
    M, K = O.softmax_mult(20000, 22, d, 12)
    # prefill: three packed sequences (chunked: positions start mid-way)
    lens, starts, sl = [5, 40, 1], [0, 17, max_pos - 1], [2, 0, 1]
    R = sum(lens)
    q8 = rng.integers(-127, 128, (R, nq, d)).astype(np.int8)
    eq = rng.integers(0, 12, (R, nq)).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    pos = np.concatenate([np.arange(s, s + n) for s, n in zip(starts, lens)]).astype(np.int32)
    slot_r = np.repeat(sl, lens).astype(np.int32)
    want = O.attention(q8, eq, kc, vc, pos, slot_r, M, K)
    got = D.detint_attn_prefill(dev(q8), dev(eq), dev(kc), dev(vc), dev(cu), dev(np.int32(starts)),
                                dev(np.int32(sl)), M, K)
    np.testing.assert_array_equal(host(got), want)
    # decode: one row per slot at various context lengths
    ctx = np.array([1, max_pos // 2 + 3, max_pos], np.int32)
    dsl = np.array([1, 2, 0], np.int32)
    q8d, eqd = q8[:3], eq[:3]
    want = O.attention(q8d, eqd, kc, vc, ctx - 1, dsl, M, K)
    got = D.detint_attn_decode(dev(q8d), dev(eqd), dev(kc), dev(vc), dev(ctx), dev(dsl), M, K)
    np.testing.assert_array_equal(host(got), want)


@pytest.mark.parametrize("nq,nkv,d", [(32, 8, 64), (16, 8, 128), (8, 8, 128), (8, 4, 64)])
def test_attention_prefill_long(D, nq, nkv, d):
    """Sequences of several query blocks and key chunks (the MFMA prefill
    path), one starting mid-cache, max_pos not a multiple of 32, and a slot
    id out of range (its rows come back zero)."""
    rng = np.random.default_rng(nq + d)
    max_pos, slots = 500, 2
    kc, vc = _cache(rng, slots, nkv, max_pos, d)
    M, K = O.softmax_mult(20000, 22, d, 12)
    lens, starts, sl = [300, 77, 20], [0, 400, 3], [1, 0, 5]
    R = sum(lens)
    q8 = rng.integers(-127, 128, (R, nq, d)).astype(np.int8)
    eq = rng.integers(0, 12, (R, nq)).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    got = host(D.detint_attn_prefill(dev(q8), dev(eq), dev(kc), dev(vc), dev(cu),
                                     dev(np.int32(starts)), dev(np.int32(sl)), M, K))
    pos = np.concatenate([np.arange(s, s + n) for s, n in zip(starts[:2], lens[:2])]).astype(np.int32)
    slot_r = np.repeat(sl[:2], lens[:2]).astype(np.int32)
    want = O.attention(q8[:377], eq[:377], kc, vc, pos, slot_r, M, K)
    np.testing.assert_array_equal(got[:377], want)
    assert not got[377:].any()


# ---------------------------------------------------------------- layer

@pytest.fixture(scope="module")
def layer_case():
    m = S.make_model("layer256", seed=1)
    h0 = S.make_residual(64, 256, seed=2)
    om = O.OracleModel(m, slots=1)
    h1, _ = om.layer(0, h0, [64], [0], [0])
    return m, h0, h1, om


def test_layer256_prefill(D, layer_case):
    """One Qwen3-style layer (hidden 256, 4/2 heads, d 64, FFN 768), 64
    tokens, residual input uniform in [-2^15, 2^15): int32 residual out and
    the KV cache equal the oracle's."""
    m, h0, h1, om = layer_case
    dm = D.DetintModel(m, n_slots=1)
    got = dm.layer(0, h0, [64], [0], [0])
    np.testing.assert_array_equal(got, h1)
    np.testing.assert_array_equal(host(dm.kc), om.kc)
    np.testing.assert_array_equal(host(dm.vc), om.vc)


def test_layer256_split_and_token_by_token(D, layer_case):
    m, h0, h1, om = layer_case
    dm = D.DetintModel(m, n_slots=2)
    a = dm.layer(0, h0[:20], [20], [0], [1])
    b = dm.layer(0, h0[20:50], [30], [20], [1])
    rows = [a, b] + [dm.layer(0, h0[t:t + 1], [1], [t], [1]) for t in range(50, 64)]
    np.testing.assert_array_equal(np.concatenate(rows), h1)
    np.testing.assert_array_equal(host(dm.kc)[:, 1], om.kc[:, 0])


# -------------------------------------------------------------- lm_head

# S <= 8 int8 rows take the fused decode kernel (four columns per wave for
# one row: V = 4099 leaves a ragged last group); wide tables and S > 8 take
# RMSNorm + lm_head (GEMV up to 16 rows, MFMA GEMM beyond) + argmax.
@pytest.mark.parametrize("S_,V,H,wide", [(1, 151936, 1024, False), (1, 4099, 1024, False), (8, 5000, 256, False),
                                         (5, 4099, 2048, False), (12, 3000, 512, False),
                                         (40, 2000, 256, False), (3, 4099, 512, True)])
def test_final_head(D, S_, V, H, wide):
    """Final RMSNorm + tied lm_head + greedy token from the residual rows,
    with duplicated embedding rows forcing exact ties at the maximum."""
    rng = np.random.default_rng(S_ + V + H)
    h = rng.integers(-(1 << 20), 1 << 20, (S_, H)).astype(np.int32)
    g = rng.integers(1 << 12, (1 << 13) + 1, H).astype(np.int16)
    if wide:
        E = rng.integers(-32767, 32768, (V, H)).astype(np.int16)
    else:
        E = rng.integers(-127, 128, (V, H)).astype(np.int8)
    E[V - 1] = E[V // 2] = E[7]
    em = rng.integers(1 << 14, 1 << 15, V).astype(np.int32)
    em[V - 1] = em[V // 2] = em[7]
    wk, fl = (30, 16) if wide else (22, 16)
    x8, xm, xk = O.rmsnorm(h, g)
    want = O.epilogue(O.gemm(x8, E), xm, xk, em, wk, fl, O.FIX)
    if wide:
        hi, lo = D.detint_split_w16(dev(E))
    else:
        hi, lo = dev(E), None
    logits, tok = D.detint_final_head(dev(h), dev(g), hi, lo, dev(em), wk, fl)
    np.testing.assert_array_equal(host(logits), want)
    np.testing.assert_array_equal(host(tok), O.argmax(want))
    lg2, none = D.detint_final_head(dev(h), dev(g), hi, lo, dev(em), wk, fl, with_token=False)
    assert none is None
    np.testing.assert_array_equal(host(lg2), want)



@pytest.mark.parametrize("S_,V,H,wide", [(1, 151936, 1024, False), (8, 5000, 256, False),
                                         (3, 4099, 512, True), (16, 1000, 256, False)])
def test_lm_head_and_greedy_token(D, S_, V, H, wide):
    rng = np.random.default_rng(S_ * V)
    x8 = rng.integers(-127, 128, (S_, H)).astype(np.int8)
    if wide:
        E = rng.integers(-32767, 32768, (V, H)).astype(np.int16)
    else:
        E = rng.integers(-127, 128, (V, H)).astype(np.int8)
    # duplicated rows make exact ties among the maxima: the lowest id must win
    E[V - 1] = E[V // 2] = E[7]
    rm = rng.integers(1 << 14, 1 << 15, S_).astype(np.int32)
    rk = rng.integers(14, 20, S_).astype(np.int32)
    em = rng.integers(1 << 14, 1 << 15, V).astype(np.int32)
    em[V - 1] = em[V // 2] = em[7] = 1 << 15 - 1
    wk, fl = (30, 16) if wide else (22, 16)
    want = O.epilogue(O.gemm(x8, E), rm, rk, em, wk, fl, O.FIX)
    if wide:
        hi, lo = D.detint_split_w16(dev(E))
    else:
        hi, lo = dev(E), None
    logits, part = D.detint_lm_head(dev(x8), hi, lo, dev(rm), dev(rk), dev(em), wk, fl)
    np.testing.assert_array_equal(host(logits), want)
    tok = host(D.detint_argmax_parts(part))
    np.testing.assert_array_equal(tok, O.argmax(want))
    # a row whose maximum is the tied triple picks id 7
    x8b = np.zeros((1, H), np.int8)
    x8b[0] = np.sign(E[7].astype(np.int64)).astype(np.int8) * 127
    lg, pt = D.detint_lm_head(dev(x8b), hi, lo, dev(rm[:1]), dev(rk[:1]), dev(em), wk, fl)
    lgh = host(lg)
    assert lgh[0, 7] == lgh[0].max() == lgh[0, V // 2] == lgh[0, V - 1]
    assert host(D.detint_argmax_parts(pt))[0] == 7
