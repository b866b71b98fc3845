"""GPU parity of detint_sample (integer temperature / top-k / top-p sampling)
with the oracle, token for token, with and without a workspace."""
import numpy as np
import pytest

import oracle as O

pytestmark = pytest.mark.gpu

T1 = (23637, 15)          # temperature 1 for logits with 16 fractional bits
HOT = (23637, 17)         # temperature 4
COLD = (1 << 23, 0)       # any gap of one unit already has weight 0


@pytest.fixture(scope="module")
def D():
    import torch
    import integer_only_deterministic_amd as D
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    D.library()
    return D


def _run(D, logits, k, tm, draws, top_p=65536, ws=False):
    import torch
    lg = torch.from_numpy(logits).cuda()
    dr = torch.from_numpy(draws.view(np.int32)).cuda()
    w = None
    if ws:
        w = torch.empty(D.detint_sample_workspace(*logits.shape), dtype=torch.uint8, device="cuda")
    return D.detint_sample(lg, k, tm[0], tm[1], dr, top_p=top_p, ws=w).cpu().numpy()


def _logits(kind, R, V, rng):
    if kind == "spread":   # gaps of a few units at 16 fractional bits
        return rng.normal(0, 3 * 65536, (R, V)).astype(np.int32)
    if kind == "ties":     # few distinct values: ties at the top-k boundary
        return (rng.integers(-4, 4, (R, V)) * 65536).astype(np.int32)
    x = rng.integers(-(1 << 31), 1 << 31, (R, V), dtype=np.int64).astype(np.int32)
    x[:, 0] = np.iinfo(np.int32).min
    x[:, -1] = np.iinfo(np.int32).max
    return x               # "extreme": the whole int32 range


@pytest.mark.parametrize("V", [1, 7, 1000, 4099, 151936])
@pytest.mark.parametrize("kind", ["spread", "ties", "extreme"])
def test_sample_matches_oracle(D, V, kind):
    rng = np.random.default_rng(V + len(kind))
    R = 6
    logits = _logits(kind, R, V, rng)
    draws = rng.integers(0, 1 << 32, R, dtype=np.uint64).astype(np.uint32)
    draws[:2] = [0, (1 << 32) - 1]
    for k in sorted({0, 1, 5, 50, 100, max(V - 1, 1), V}):
        for tm in (T1, HOT, COLD):
            want = O.sample(logits, k, tm[0], tm[1], draws)
            got = _run(D, logits, k, tm, draws)
            np.testing.assert_array_equal(got, want, err_msg=f"k={k} t={tm}")
            # with a workspace: the sliced paths (every id kept, or top-k
            # with at most 8192 slice candidates)
            got = _run(D, logits, k, tm, draws, ws=True)
            np.testing.assert_array_equal(got, want, err_msg=f"k={k} t={tm} (workspace)")


@pytest.mark.parametrize("V", [7, 1000, 151936])
@pytest.mark.parametrize("kind", ["spread", "ties", "extreme"])
def test_sample_top_p_matches_oracle(D, V, kind):
    rng = np.random.default_rng(3 * V + len(kind))
    R = 6
    logits = _logits(kind, R, V, rng)
    draws = rng.integers(0, 1 << 32, R, dtype=np.uint64).astype(np.uint32)
    draws[:2] = [0, (1 << 32) - 1]
    for k in sorted({0, 1, 50, V}):
        for p in (1, 6553, 32768, 58982, 65535):
            for tm in (T1, HOT):
                want = O.sample(logits, k, tm[0], tm[1], draws, top_p=p)
                got = _run(D, logits, k, tm, draws, top_p=p)
                np.testing.assert_array_equal(got, want, err_msg=f"k={k} p={p} t={tm}")
                got = _run(D, logits, k, tm, draws, top_p=p, ws=True)
                np.testing.assert_array_equal(got, want, err_msg=f"k={k} p={p} t={tm} (ws)")


def test_sample_many_draws_one_row(D):
    """One row, 4096 draws across [0, 2^32): every boundary of the inverse
    CDF the draws land on matches the oracle."""
    rng = np.random.default_rng(11)
    row = rng.normal(0, 2 * 65536, 3000).astype(np.int32)
    draws = np.sort(rng.integers(0, 1 << 32, 4096, dtype=np.uint64).astype(np.uint32))
    logits = np.tile(row, (4096, 1))
    for k, p in ((0, 65536), (40, 65536), (0, 58982), (40, 32768)):
        want = O.sample(logits, k, T1[0], T1[1], draws, top_p=p)
        np.testing.assert_array_equal(_run(D, logits, k, T1, draws, top_p=p), want)
        np.testing.assert_array_equal(_run(D, logits, k, T1, draws, top_p=p, ws=True), want)


@pytest.mark.parametrize("V", [2048, 2049, 262144])
def test_sample_slice_edges_and_largest_vocabulary(D, V):
    """Exactly one 2048-id slice, one id past it, and the largest accepted
    vocabulary (128 slices of 2048, 256 of 1024): every path, with and
    without a workspace, token for token."""
    rng = np.random.default_rng(V)
    R = 4
    logits = _logits("spread", R, V, rng)
    draws = rng.integers(0, 1 << 32, R, dtype=np.uint64).astype(np.uint32)
    draws[:2] = [0, (1 << 32) - 1]
    for k, p in ((0, 65536), (1, 65536), (64, 65536), (0, 58982), (64, 58982)):
        want = O.sample(logits, k, T1[0], T1[1], draws, top_p=p)
        for ws in (False, True):
            got = _run(D, logits, k, T1, draws, top_p=p, ws=ws)
            np.testing.assert_array_equal(got, want, err_msg=f"V={V} k={k} p={p} ws={ws}")


def test_sample_graph_replays_match_oracle(D):
    """detint_sample with a workspace captured once into a HIP graph per
    path (all ids, top-50, top-50 then top-p, top-p alone), then replayed
    with new logits and draws copied in eagerly between replays: every
    replay's tokens equal the oracle's."""
    import torch
    V, R = 151936, 4
    lg = torch.zeros((R, V), dtype=torch.int32, device="cuda")
    dr = torch.zeros(R, dtype=torch.int32, device="cuda")
    out = torch.zeros(R, dtype=torch.int32, device="cuda")
    ws = torch.empty(D.detint_sample_workspace(R, V), dtype=torch.uint8, device="cuda")
    for k, p in ((0, 65536), (50, 65536), (50, 58982), (0, 58982)):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            D.detint_sample(lg, k, T1[0], T1[1], dr, out, top_p=p, ws=ws)
        torch.cuda.current_stream().wait_stream(s)
        for rep in range(3):
            rng = np.random.default_rng(1000 * k + p + rep)
            logits = rng.normal(0, 3 * 65536, (R, V)).astype(np.int32)
            draws = rng.integers(0, 1 << 32, R, dtype=np.uint64).astype(np.uint32)
            lg.copy_(torch.from_numpy(logits))
            dr.copy_(torch.from_numpy(draws.view(np.int32)))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            np.testing.assert_array_equal(out.cpu().numpy(),
                                          O.sample(logits, k, T1[0], T1[1], draws, top_p=p),
                                          err_msg=f"k={k} p={p} replay {rep}")
