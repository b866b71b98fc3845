"""Exact mode on the GPU (BitExact LLM blog, "Three execution paths": bf16
weights kept in the linear layers, products with fixed-point activations):
the prepared integer planes and row exponents, and the product in every
output mode, against the oracle, bit for bit, over GEMV-, skinny- and
MFMA-sized row counts with ragged edges; weights exact mode cannot hold are
flagged."""
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
    D.detint_check()
    return D


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _planes_to_int(planes):
    p = planes.astype(np.int64)
    return (p[0] << 24) + (p[1] << 16) + (p[2] << 8) + p[3] + 128 * (65536 + 256 + 1)


@pytest.mark.parametrize("N,K", [(64, 256), (300, 1024), (7, 2064)])
def test_prepare_matches_oracle(D, N, K):
    Wb = S.make_bf16_weights(N, K, seed=N + K)
    Wb[0, :5] = [0x0001, 0x8000, 0x0000, 0x807F, 0x0080]    # subnormals, signed zeros, smallest normal
    Wb[0, 5:] &= 0x80FF                                      # row 0 stays within a 23-order span
    Wb[1] = 0                                                # an all-zero row
    W_int, row_exp = O.exact_weights(Wb)
    planes, rexp = D.detint_exact_prepare(dev(Wb.view(np.int16)))
    assert D.detint_check() == 0
    np.testing.assert_array_equal(_planes_to_int(planes.cpu().numpy()), W_int)
    np.testing.assert_array_equal(rexp.cpu().numpy(), row_exp)


def test_prepare_flags_weights_it_cannot_hold(D):
    Wb = S.make_bf16_weights(4, 64, seed=9)
    Wb[1, 3] = 0x7F80            # infinity
    D.detint_exact_prepare(dev(Wb.view(np.int16)))
    assert D.detint_check() == D.BOUND_WEIGHT
    Wb = np.full((2, 64), 0x3F80, np.uint16)
    Wb[0, 7] = 0x3300            # 25 binary orders below the rest of its row
    D.detint_exact_prepare(dev(Wb.view(np.int16)))
    assert D.detint_check() == D.BOUND_WEIGHT


@pytest.mark.parametrize("M,N,K", [(1, 300, 1024), (7, 129, 2048), (40, 256, 512), (300, 200, 1024),
                                   (2048, 512, 2048), (5, 77, 48)])
def test_gemm_exact_matches_oracle(D, M, N, K):
    rng = np.random.default_rng(M * N + K)
    Wb = S.make_bf16_weights(N, K, seed=M + 3 * N + K)
    W_int, row_exp = O.exact_weights(Wb)
    A = rng.integers(-128, 128, (M, K)).astype(np.int8)
    A[0] = -128
    rm = rng.integers(1 << 14, 1 << 15, M).astype(np.int32)
    rk = rng.integers(12, 17, M).astype(np.int32)          # activation scale m_r 2^-k_r near 1
    planes, rexp = D.detint_exact_prepare(dev(Wb.view(np.int16)))
    dA, drm, drk = dev(A), dev(rm), dev(rk)
    acc = O.gemm_exact(A, W_int)
    np.testing.assert_array_equal(D.detint_gemm_exact(dA, planes, rexp).cpu().numpy(), acc)
    for mode, frac in ((D.REQ_I8, 0), (D.FIX, 8)):
        got = D.detint_gemm_exact(dA, planes, rexp, drm, drk, frac, mode).cpu().numpy()
        want = O.exact_epilogue(acc, rm, rk, row_exp, frac, mode)
        np.testing.assert_array_equal(got, want, err_msg=f"mode {mode}")
    assert D.detint_check() == 0
