"""Paged KV cache (BitExact LLM blog, "What the checks actually compare":
KV-cache reuse, shared prefixes, preemption and chunked prefill must not
change a bit). The cache is a pool of fixed-size pages per layer and each
sequence's positions are mapped through a block table; the oracle keeps its
own contiguous cache, so every comparison below maps the pages back through
the table. Covered: every kernel that reads or writes the cache (QKV
post-processing with and without q/k-norm, the MFMA prefill attention, the
per-row attention, the fused decode attention including its streamed rows
past the first 512), pages scattered at random across sequences, prefix pages
shared by two sequences through their tables (written once, read by both),
preemption by recompute into other pages, and block-table entries outside
the pool, which are flagged."""
import dataclasses

import numpy as np
import pytest

import detint_synth as S
import oracle as O

pytestmark = pytest.mark.gpu

TINY_1K = dataclasses.replace(S.SHAPES["tiny"], name="tiny_1k", max_pos=1024)
WIDE_1K = dataclasses.replace(S.SHAPES["tiny_wide"], name="tiny_wide_1k", max_pos=1024)
LLAMA_HEADS = S.ModelShape("llama_heads_1k", 1, 256, 32, 8, 64, 512, 1000, False, True, 500_000, 1024, 30)


@pytest.fixture(scope="module")
def D():
    import torch
    import integer_only_deterministic_amd as D
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    D.library()
    D.detint_check()
    return D


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def scatter_tables(rng, n_slots, max_blocks, n_pages):
    """A block table whose entries are a random permutation of the pool."""
    perm = rng.permutation(n_pages)[: n_slots * max_blocks]
    return perm.reshape(n_slots, max_blocks).astype(np.int32)


@pytest.mark.parametrize("shape", [TINY_1K, WIDE_1K, LLAMA_HEADS], ids=lambda s: s.name)
@pytest.mark.parametrize("page", [16, 64])
def test_paged_generation_matches_oracle(D, shape, page):
    import torch
    m = S.make_model(shape, seed=81)
    V = shape.vocab
    # lengths: per-row attention (< 16 rows), MFMA prefill, and a context past
    # the 512 rows the decode attention loads up front
    prompts = [S.make_prompt(V, 9, 1), S.make_prompt(V, 300, 2), S.make_prompt(V, 700, 3)]
    n_new = 12
    rows = []
    om = O.OracleModel(m, slots=3)
    om.generate(prompts, n_new, on_step=lambda s, lg: rows.append(lg.copy()))
    rng = np.random.default_rng(page)
    mb = shape.max_pos // page
    n_pages = 3 * mb + 5
    dm = D.DetintModel(m, n_slots=3, page_size=page, n_pages=n_pages)
    dm.block_table.copy_(torch.from_numpy(scatter_tables(rng, 3, mb, n_pages)))
    hist = host(dm.generate(prompts, n_new))
    np.testing.assert_array_equal(hist, np.stack(rows))
    kc, vc = dm.contiguous_cache()
    for b, p in enumerate(prompts):
        n = len(p) + n_new - 1                      # positions written
        np.testing.assert_array_equal(kc[:, b, :, :n], om.kc[:, b, :, :n], err_msg=f"K row {b}")
        np.testing.assert_array_equal(vc[:, b, :, :n], om.vc[:, b, :, :n], err_msg=f"V row {b}")
    assert D.detint_check() == 0


@pytest.mark.parametrize("shape", [TINY_1K, LLAMA_HEADS], ids=lambda s: s.name)
def test_shared_prefix_pages_are_aliased(D, shape):
    """Sequence A holds a 128-token prefix plus its own suffix; sequence B's
    table names A's two prefix pages (page size 64) and B prefills only its
    suffix from position 128. B's logits, then 6 decode steps of both, equal
    the oracle's for each sequence run alone; the shared pages still hold
    A's rows."""
    import torch
    m = S.make_model(shape, seed=82)
    V = shape.vocab
    prefix = S.make_prompt(V, 128, 5)
    a = np.concatenate([prefix, S.make_prompt(V, 50, 6)]).astype(np.int32)
    b = np.concatenate([prefix, S.make_prompt(V, 37, 7)]).astype(np.int32)
    want = []
    for seq in (a, b):
        rows = []
        O.OracleModel(m, slots=1).generate([seq], 7, on_step=lambda s, lg: rows.append(lg[0].copy()))
        want.append(np.stack(rows))
    page, mb = 64, shape.max_pos // 64
    dm = D.DetintModel(m, n_slots=2, page_size=page, n_pages=2 * mb)
    bt = np.arange(2 * mb, dtype=np.int32).reshape(2, mb)
    bt[1, :2] = bt[0, :2]                           # B's prefix pages are A's
    dm.block_table.copy_(torch.from_numpy(bt))
    hist = torch.zeros((8, 2, V), dtype=torch.int32, device="cuda")
    ta = dm.prefill([a], [0], [0], hist, 0)
    k_shared = host(dm.kc[:, bt[0, :2]]).copy()
    tb = dm.prefill([b[128:]], [128], [1], hist, 1)
    np.testing.assert_array_equal(host(dm.kc[:, bt[0, :2]]), k_shared)   # written once, by A
    tok = torch.cat([ta, tb])
    dm.decode(tok, [len(a), len(b)], [0, 1], 6, hist, 2)
    got = host(hist)
    np.testing.assert_array_equal(got[:7, 0], want[0])
    np.testing.assert_array_equal(got[:7, 1], want[1])


def test_preempted_sequence_rebuilt_in_other_pages(D):
    """A sequence decodes 5 steps, loses its pages, and is rebuilt by one
    prefill of its prompt plus the tokens it produced into different pages;
    its next steps equal the uninterrupted oracle run."""
    import torch
    m = S.make_model(TINY_1K, seed=83)
    V = 1000
    p = S.make_prompt(V, 90, 9)
    rows = []
    toks = O.OracleModel(m, slots=1).generate([p], 12, on_step=lambda s, lg: rows.append(lg[0].copy()))
    page, mb = 16, 1024 // 16
    dm = D.DetintModel(m, n_slots=1, page_size=page, n_pages=2 * mb)
    dm.block_table.copy_(torch.arange(mb, dtype=torch.int32, device="cuda").view(1, mb))
    hist = torch.zeros((12, 1, V), dtype=torch.int32, device="cuda")
    tok = dm.prefill([p], [0], [0], hist, 0)
    dm.decode(tok, [90], [0], 5, hist, 1)
    # preempted: new pages (the upper half of the pool), rebuilt by recompute
    dm.block_table.copy_(torch.arange(mb, 2 * mb, dtype=torch.int32, device="cuda").view(1, mb))
    seq = np.concatenate([p, toks[0, :5]]).astype(np.int32)
    tok = dm.prefill([seq], [0], [0], hist, 5)
    dm.decode(tok, [len(seq)], [0], 6, hist, 6)
    np.testing.assert_array_equal(host(hist)[:, 0], np.stack(rows))


def test_block_table_entries_outside_the_pool_are_flagged(D):
    import torch
    m = S.make_model(TINY_1K, seed=84)
    page, mb = 64, 1024 // 64
    dm = D.DetintModel(m, n_slots=1, page_size=page, n_pages=mb)
    bt = np.arange(mb, dtype=np.int32).reshape(1, mb)
    bt[0, 1] = mb + 5                               # positions 64..127
    dm.block_table.copy_(torch.from_numpy(bt))
    hist = torch.zeros((2, 1, 1000), dtype=torch.int32, device="cuda")
    dm.prefill([S.make_prompt(1000, 100, 3)], [0], [0], hist, 0)
    assert D.detint_check() & D.BOUND_PAGE
    dm.prefill([S.make_prompt(1000, 40, 3)], [0], [0], hist, 0)   # stays in page 0
    assert D.detint_check() == 0
