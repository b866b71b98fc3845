"""detint_final_head_noalloc, the allocation-free variant of
detint_final_head: same logits and greedy tokens as the workspace call, on
two calls in a row (the second smaller, so it runs over what the first left
in the shared per-device scratch), for the fused decode path (int8 table,
up to 8 rows), the limb-table path and the 16-row path; and a request past
the scratch size is rejected before any device work."""
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
    return D


def _case(V, H, wide, seed):
    import torch
    rng = np.random.default_rng(seed)
    if wide:
        w16 = rng.integers(-32767, 32768, (V, H)).astype(np.int16)
        emb = torch.from_numpy(w16).cuda()
        import integer_only_deterministic_amd as D
        hi, lo = D.detint_split_w16(emb)
        emb, emb_lo, w_k = hi, lo, 30
    else:
        emb = torch.from_numpy(rng.integers(-127, 128, (V, H)).astype(np.int8)).cuda()
        emb_lo, w_k = None, 22
    emb_m = torch.from_numpy(rng.integers(1 << 14, 1 << 15, V).astype(np.int32)).cuda()
    gain = torch.from_numpy(rng.integers(1 << 12, (1 << 13) + 1, H).astype(np.int16)).cuda()
    return emb, emb_lo, emb_m, gain, w_k


@pytest.mark.parametrize("V,H,wide,rows", [(151936, 1024, False, (8, 1)), (5000, 256, True, (5, 2)),
                                           (40000, 512, False, (16, 3))])
def test_noalloc_matches_workspace_call_twice(D, V, H, wide, rows):
    import torch
    emb, emb_lo, emb_m, gain, w_k = _case(V, H, wide, V + H)
    rng = np.random.default_rng(V)
    for S_ in rows:                               # second call smaller than the first
        h = torch.from_numpy(rng.integers(-(1 << 22), 1 << 22, (S_, H)).astype(np.int32)).cuda()
        want_l, want_t = D.detint_final_head(h, gain, emb, emb_lo, emb_m, w_k, 16)
        got_l, got_t = D.detint_final_head_noalloc(h, gain, emb, emb_lo, emb_m, w_k, 16)
        torch.cuda.synchronize()
        assert torch.equal(got_l, want_l), f"logits differ, S={S_}"
        assert torch.equal(got_t, want_t), f"tokens differ, S={S_}"


def test_noalloc_rejects_requests_past_its_scratch(D):
    import torch
    V, H = 262144, 1024
    need = D.library().detint_final_head_workspace(64, V, H)
    assert need > 4 << 20
    h = torch.zeros((64, H), dtype=torch.int32, device="cuda")
    emb = torch.zeros((V, H), dtype=torch.int8, device="cuda")
    emb_m = torch.full((V,), 1 << 14, dtype=torch.int32, device="cuda")
    gain = torch.full((H,), 4096, dtype=torch.int16, device="cuda")
    with pytest.raises(D.DetintError) as ei:
        D.detint_final_head_noalloc(h, gain, emb, None, emb_m, 22, 16)
    assert ei.value.code == D.DETINT_EINVAL and "scratch" in str(ei.value)
