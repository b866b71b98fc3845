"""Device bound checks (BitExact LLM blog, "Reproducibility has a cost":
range checks before residual additions, on the final logits and on the
linear epilogues) and a float-leak guard on the Python side.

Every over-range case below is built from the host: inputs or scales that
push one intermediate past its written bound. The kernels finish normally
(nothing faults or waits); detint_check then reports the expected flag and
clears it. Runs that stay in range report nothing."""
import numpy as np
import pytest

import detint_synth as S

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def D():
    import torch
    import integer_only_deterministic_amd as D
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    D.library()
    D.detint_check()            # start from clear flags
    return D


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("name", ["tiny", "tiny_wide"])
def test_in_range_generation_raises_no_flag(D, name):
    m = S.make_model(name, seed=51)
    prompts = [S.make_prompt(1000, 40, 1), S.make_prompt(1000, 9, 2), S.make_prompt(1000, 70, 3)]
    D.DetintModel(m, n_slots=3).generate(prompts, 6)
    D.DetintModel(m, n_slots=1).generate(prompts[:1], 6)
    assert D.detint_check() == 0


def test_rmsnorm_sum_of_squares_flag(D):
    n = 16384
    g = dev(np.full(n, 4096, np.int16))
    D.detint_rmsnorm(dev(np.full((2, n), (1 << 24) - 1, np.int32)), g)
    assert D.detint_check() == 0                       # S just below 2^62
    D.detint_rmsnorm(dev(np.full((2, n), 1 << 24, np.int32)), g)
    assert D.detint_check() == D.BOUND_NORM            # S = 2^62
    assert D.detint_check() == 0                       # cleared


@pytest.mark.parametrize("M", [1, 6, 40, 512])
@pytest.mark.parametrize("row_k", [0, 1])
def test_gemm_fix_outside_int32_flag(D, M, row_k):
    """FIX results of 2^53-ish: every GEMM path (decode GEMV, GEMV,
    skinny, pipelined with the general and the in-range epilogue)."""
    N, K = 256, 1024
    A = np.full((M, K), 127, np.int8)
    W = np.full((N, K), 127, np.int8)
    rm = dev(np.full(M, 1 << 14, np.int32))
    rk = dev(np.full(M, row_k, np.int32))
    cm = dev(np.full(N, 1 << 14, np.int32))
    dA, dW = dev(A), dev(W)
    D.detint_gemm_i8(dA, dW, rm, rk, cm, 30, 0, D.FIX)          # shift 30 + row_k: in range
    assert D.detint_check() == 0
    D.detint_gemm_i8(dA, dW, rm, rk, cm, 0, 0, D.FIX)           # shift row_k: 2^52 and up
    assert D.detint_check() == D.BOUND_INT32


@pytest.mark.parametrize("M", [1, 40, 512])
def test_gemm_res_add_outside_int32_flag(D, M):
    N, K = 256, 1024
    rng = np.random.default_rng(M)
    A = dev(rng.integers(-128, 128, (M, K)).astype(np.int8))
    W = dev(rng.integers(-128, 128, (N, K)).astype(np.int8))
    rm = dev(np.full(M, 1 << 14, np.int32))
    rk = dev(np.full(M, 20, np.int32))
    cm = dev(np.full(N, 1 << 14, np.int32))
    out = dev(np.full((M, N), (1 << 31) - 1, np.int32))
    D.detint_gemm_i8(A, W, rm, rk, cm, 22, 0, D.RES_ADD, out=out)
    assert D.detint_check() == D.BOUND_INT32
    out = dev(np.zeros((M, N), np.int32))
    D.detint_gemm_i8(A, W, rm, rk, cm, 22, 0, D.RES_ADD, out=out)
    assert D.detint_check() == 0


def test_swiglu_input_flag(D):
    gu = np.zeros((3, 2 * 768), np.int32)
    gu[1, 5] = 1 << 24
    D.detint_swiglu(dev(gu), 12)
    assert D.detint_check() == D.BOUND_SWIGLU


@pytest.mark.parametrize("R", [3, 40, 100])
def test_layer_residual_flag(D, R):
    """A residual stream at the edge of 2^25: the O-proj or down-projection
    residual add pushes it over (GEMV, skinny and pipelined GEMM paths)."""
    m = S.make_model("layer256", seed=52)
    dm = D.DetintModel(m, n_slots=1)
    h = np.full((R, 256), (1 << 25) - 1, np.int32)
    h[:, ::2] = -(1 << 25) + 1
    dm.layer(0, h, [R], [0], [0])
    assert D.detint_check() & D.BOUND_RESIDUAL
    dm.layer(0, S.make_residual(R, 256, seed=3), [R], [0], [0])
    assert D.detint_check() == 0


def test_decode_residual_and_token_id_flags(D):
    """The fused decode step: O-proj column mantissas far above 2^15 push its
    residual add past 2^25; a token id past the vocabulary is flagged and
    embedded as zeros."""
    import torch
    m = S.make_model("tiny", seed=53)
    p = S.make_prompt(1000, 12, 4)
    dm = D.DetintModel(m, n_slots=1)
    hist = torch.zeros((2, 1, 1000), dtype=torch.int32, device="cuda")
    tok = dm.prefill([p], [0], [0], hist, 0)
    dm.decode(tok, [12], [0], 1, hist, 1, use_graph=False)
    assert D.detint_check() == 0
    bad_id = torch.tensor([1000], dtype=torch.int32, device="cuda")
    dm.decode(bad_id, [13], [0], 1, hist, 1, use_graph=False)
    assert D.detint_check() & D.BOUND_ID
    # ~2^15.5 x the drawn mantissas: the O-proj delta of every row passes 2^25 by
    # a wide margin, while |acc * m_r * m_c| stays below 2^63
    m.layers[1].wo_m = np.full_like(m.layers[1].wo_m, 1 << 30)
    dm2 = D.DetintModel(m, n_slots=1)
    tok = dm2.prefill([p], [0], [0], hist, 0)
    D.detint_check()                                   # the prefill's own adds
    dm2.decode(tok, [12], [0], 1, hist, 1, use_graph=False)
    assert D.detint_check() & D.BOUND_RESIDUAL


def test_binding_issues_no_float_tensor_op(D):
    """DetLLM README, "Layout": a guard turns any float in the forward pass
    into an error. Here every torch operation the Python binding issues
    while a model prefills and decodes is intercepted, and any float tensor
    among its inputs or outputs fails the test (the arithmetic itself runs
    in the library's kernels, whose code the device-code scan checks)."""
    import torch
    from torch.utils._python_dispatch import TorchDispatchMode
    from torch.utils._pytree import tree_flatten

    seen = []

    class NoFloat(TorchDispatchMode):
        def __torch_dispatch__(self, func, types, args=(), kwargs=None):
            out = func(*args, **(kwargs or {}))
            for t in tree_flatten((args, kwargs, out))[0]:
                if isinstance(t, torch.Tensor) and t.is_floating_point():
                    raise AssertionError(f"float tensor in {func}: {t.dtype}")
            seen.append(str(func))
            return out

    m = S.make_model("tiny", seed=54)
    dm = D.DetintModel(m, n_slots=2)
    with NoFloat():
        hist = dm.generate([S.make_prompt(1000, 20, 5), S.make_prompt(1000, 7, 6)], 5, use_graph=False)
        hist.cpu()
    assert seen, "the guard saw no torch operation"
