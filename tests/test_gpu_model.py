"""Whole-model GPU parity: logits of every generation step bit-identical to
the CPU oracle, and the invariances the pages claim (batch composition,
split prefill, token-by-token prompt feeding, graph vs eager, repeats).
The Qwen3-0.6B-shaped runs compare against chained per-step logits hashes
that tests/golden/make_golden.py wrote with the oracle alone."""
import json
from pathlib import Path

import numpy as np
import pytest

import detint_synth as S
import oracle as O

pytestmark = pytest.mark.gpu
GOLDEN = Path(__file__).resolve().parent / "golden"


@pytest.fixture(scope="module")
def D():
    import torch
    import integer_only_deterministic_amd as D
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    D.library()
    return D


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


@pytest.mark.parametrize("name", ["tiny", "tiny_wide"])
@pytest.mark.parametrize("use_graph", [True, False])
def test_tiny_generation_matches_oracle(D, name, use_graph):
    m = S.make_model(name, seed=21)
    V = m.shape.vocab
    prompts = [S.make_prompt(V, 7, 1), S.make_prompt(V, 30, 2), S.make_prompt(V, 19, 3)]
    n_new = 24
    rows = []
    toks = O.OracleModel(m, slots=3).generate(prompts, n_new, on_step=lambda s, lg: rows.append(lg.copy()))
    dm = D.DetintModel(m, n_slots=3)
    hist = host(dm.generate(prompts, n_new, use_graph=use_graph))
    want = np.stack(rows)                       # [n_new, B, V]
    for s in range(n_new):
        np.testing.assert_array_equal(hist[s], want[s], err_msg=f"{name} step {s}")
    np.testing.assert_array_equal(hist.argmax(-1).T, toks)


def test_tiny_kv_cache_matches_oracle(D):
    m = S.make_model("tiny", seed=22)
    prompts = [S.make_prompt(1000, 40, 4), S.make_prompt(1000, 9, 5)]
    om = O.OracleModel(m, slots=2)
    om.generate(prompts, 6)
    dm = D.DetintModel(m, n_slots=2)
    dm.generate(prompts, 6)
    np.testing.assert_array_equal(host(dm.kc), om.kc)
    np.testing.assert_array_equal(host(dm.vc), om.vc)


# ------------------------------- per-channel key gains (DetLLM blog footnote 8)

@pytest.mark.parametrize("name", ["tiny", "tiny_wide"])
@pytest.mark.parametrize("use_graph", [True, False])
def test_tiny_key_gains_match_oracle(D, name, use_graph):
    """Seeded key gains on every layer: prefill (QKV post-processing kernel)
    and decode (fused attention, one query head per workgroup) logits, and
    the cached keys, equal the oracle's."""
    m = S.with_key_gains(S.make_model(name, seed=23), seed=24, gmax=2)
    V = m.shape.vocab
    prompts = [S.make_prompt(V, 7, 1), S.make_prompt(V, 30, 2), S.make_prompt(V, 19, 3)]
    rows = []
    om = O.OracleModel(m, slots=3)
    om.generate(prompts, 12, on_step=lambda s, lg: rows.append(lg.copy()))
    dm = D.DetintModel(m, n_slots=3)
    hist = host(dm.generate(prompts, 12, use_graph=use_graph))
    np.testing.assert_array_equal(hist, np.stack(rows))
    np.testing.assert_array_equal(host(dm.kc), om.kc)


def test_tiny_key_gains_batch64_match_oracle(D):
    """64 decode rows: the fused attention takes every query head of a KV
    head per workgroup."""
    m = S.with_key_gains(S.make_model("tiny", seed=25), seed=26, gmax=2)
    prompts = [S.make_prompt(1000, 3 + (i * 7) % 20, 30 + i) for i in range(64)]
    rows = []
    O.OracleModel(m, slots=64).generate(prompts, 4, on_step=lambda s, lg: rows.append(lg.copy()))
    dm = D.DetintModel(m, n_slots=64)
    np.testing.assert_array_equal(host(dm.generate(prompts, 4, use_graph=True)), np.stack(rows))


@pytest.mark.parametrize("nq,nkv,d,qkn,B", [(8, 2, 64, False, 64), (4, 2, 128, True, 3)])
def test_key_gains_512_thread_decode_match_oracle(D, nq, nkv, d, qkn, B):
    """Key gains through the 512-thread decode workgroups: four 64-wide
    query heads per KV head (64 rows), and one 128-wide query head (3 rows)."""
    shape = S.ModelShape("gains_%d_%d" % (d, B), 1, 256, nq, nkv, d, 512, 1000, qkn, False,
                         1_000_000, 256, 22)
    m = S.with_key_gains(S.make_model(shape, seed=27), seed=28, gmax=2)
    prompts = [S.make_prompt(1000, 5 + (i * 11) % 40, 60 + i) for i in range(B)]
    rows = []
    om = O.OracleModel(m, slots=B)
    om.generate(prompts, 4, on_step=lambda s, lg: rows.append(lg.copy()))
    dm = D.DetintModel(m, n_slots=B)
    np.testing.assert_array_equal(host(dm.generate(prompts, 4, use_graph=True)), np.stack(rows))
    np.testing.assert_array_equal(host(dm.kc), om.kc)


def test_tiny_preemption_recompute_matches_uninterrupted(D):
    """Row 1 loses its cache after k decode steps and is rebuilt by one
    prefill of its prompt plus the tokens it produced, in another slot; both
    rows then decode on (graph replays). Every logits row equals the
    uninterrupted run's and the oracle's."""
    import torch
    m = S.make_model("tiny", seed=31)
    V = m.shape.vocab
    p = [S.make_prompt(V, 20, 41), S.make_prompt(V, 13, 42)]
    n, k = 9, 4
    rows = []
    O.OracleModel(m, slots=3).generate(p, n, on_step=lambda s, lg: rows.append(lg.copy()))
    want = np.stack(rows)
    ref = host(D.DetintModel(m, n_slots=3).generate(p, n))
    np.testing.assert_array_equal(ref, want)
    dm = D.DetintModel(m, n_slots=3)
    h1 = torch.zeros((k, 2, V), dtype=torch.int32, device="cuda")
    tok = dm.prefill(p, [0, 0], [0, 1], h1, 0)
    dm.decode(tok, [20, 13], [0, 1], k - 1, h1, 2, use_graph=True)
    a = host(h1)
    gen1 = a[:k - 1, 1].argmax(-1).astype(np.int32)
    re = torch.zeros((1, V), dtype=torch.int32, device="cuda")
    t1 = dm.prefill([np.concatenate([p[1], gen1])], [0], [2], re, 0)
    np.testing.assert_array_equal(host(re)[0], a[k - 1, 1])
    tok2 = torch.stack([tok[0], t1[0]]).contiguous()
    h2 = torch.zeros((n - k, 2, V), dtype=torch.int32, device="cuda")
    dm.decode(tok2, [20 + k - 1, 13 + k - 1], [0, 2], n - k, h2, 0, use_graph=True)
    np.testing.assert_array_equal(np.concatenate([a, host(h2)]), want)


def test_tiny_shared_prefix_copied_cache_matches_full_prefill(D):
    """The second of two sequences that share a 24-token prefix takes the
    first's cached prefix rows (device copy into its slot) and prefills only
    its suffix from position 24; its logits and both rows' decode steps
    (graph replays) equal the oracle's run that prefilled both in full."""
    import torch
    m = S.make_model("tiny", seed=32)
    V = m.shape.vocab
    pre = S.make_prompt(V, 24, 43)
    a = np.concatenate([pre, S.make_prompt(V, 9, 44)])
    b = np.concatenate([pre, S.make_prompt(V, 6, 45)])
    n = 6
    rows = []
    O.OracleModel(m, slots=2).generate([a, b], n, on_step=lambda s, lg: rows.append(lg.copy()))
    dm = D.DetintModel(m, n_slots=2)
    h = torch.zeros((n, 2, V), dtype=torch.int32, device="cuda")
    ta = dm.prefill([a], [0], [0], h, 0)
    dm.kc[:, 1, :, :24] = dm.kc[:, 0, :, :24]
    dm.vc[:, 1, :, :24] = dm.vc[:, 0, :, :24]
    tb = dm.prefill([b[24:]], [24], [1], h, 1)
    tok = torch.stack([ta[0], tb[0]]).contiguous()
    dm.decode(tok, [len(a), len(b)], [0, 1], n - 1, h, 2, use_graph=True)
    np.testing.assert_array_equal(host(h), np.stack(rows))


# ----------------------------------------------------- Qwen3-0.6B shape

@pytest.fixture(scope="module")
def qwen(D):
    g = json.loads((GOLDEN / "qwen3_b1.json").read_text())
    m = S.make_model("qwen3_0.6b", seed=g["model_seed"])
    assert S.model_digest(m) == g["model_digest"], "synthetic model drifted from the golden file"
    return m, g


def test_qwen3_b1_512_steps(D, qwen):
    """64-token prompt + 512 greedy tokens at batch 1: every step's chained
    logits hash and every token equal the oracle's."""
    m, g = qwen
    p0 = S.make_prompt(m.shape.vocab, 64, g["prompt_seed"])
    dm = D.DetintModel(m, n_slots=1)
    hist = host(dm.generate([p0], g["n_new"]))[:, 0]
    chain = D.logits_chain(hist)
    bad = [s for s in range(len(chain)) if chain[s] != g["logits_chain"][0][s]]
    assert not bad, f"first mismatching step {bad[0]}"
    np.testing.assert_array_equal(hist.argmax(-1), g["tokens"][0])


def test_qwen3_b8_row0_hash(D, qwen):
    """The same prompt sharing a batch of 8 with 7 random prompts of 16-256
    tokens: row 0's 512-step hash equals batch 1's."""
    m, g = qwen
    V = m.shape.vocab
    prompts = [S.make_prompt(V, 64, g["prompt_seed"])] + S.make_prompts(V, 7, 16, 256, 2)
    dm = D.DetintModel(m, n_slots=8)
    hist = host(dm.generate(prompts, g["n_new"]))
    assert D.logits_chain(hist[:, 0])[-1] == g["logits_chain"][0][-1]
    g8 = GOLDEN / "qwen3_b8.json"
    if g8.exists():
        gb = json.loads(g8.read_text())
        for b in range(8):
            assert D.logits_chain(hist[:, b])[-1] == gb["logits_chain"][b][-1], f"row {b}"


@pytest.mark.parametrize("variant", ["two_halves", "half_then_tokens"])
def test_qwen3_split_prefill(D, qwen, variant):
    """Prefill in two halves (32 + 32), or 32 tokens then 32 one-by-one; then
    greedy decode. The 512-step hash equals the single-prefill run."""
    import torch
    m, g = qwen
    p0 = S.make_prompt(m.shape.vocab, 64, g["prompt_seed"])
    n_new = g["n_new"]
    dm = D.DetintModel(m, n_slots=1)
    hist = torch.empty((n_new, 1, m.shape.vocab), dtype=torch.int32, device="cuda")
    scratch = torch.empty((1, 1, m.shape.vocab), dtype=torch.int32, device="cuda")
    if variant == "two_halves":
        dm.prefill([p0[:32]], [0], [0], scratch, 0)
        tok = dm.prefill([p0[32:]], [32], [0], hist, 0)
    else:
        dm.prefill([p0[:32]], [0], [0], scratch, 0)
        for t in range(32, 64):
            tok = dm.prefill([p0[t:t + 1]], [t], [0], hist if t == 63 else scratch, 0)
    dm.decode(tok, [64], [0], n_new - 1, hist, 1)
    chain = D.logits_chain(host(hist)[:, 0])
    assert chain == g["logits_chain"][0]


def test_qwen3_repeat_runs_identical(D, qwen):
    m, g = qwen
    p0 = S.make_prompt(m.shape.vocab, 64, g["prompt_seed"])
    dm = D.DetintModel(m, n_slots=1)
    a = host(dm.generate([p0], 64))
    for _ in range(2):
        dm.reset_cache()
        np.testing.assert_array_equal(host(dm.generate([p0], 64)), a)
    assert D.logits_chain(a[:, 0])[-1] == g["logits_chain"][0][63]


# ------------------------------------------- Llama-3.2-1B shape, 16-bit limbs

@pytest.fixture(scope="module")
def llama():
    return S.make_model("llama3.2_1b", seed=0)


def test_llama_limbs_short_generation_matches_oracle(D, llama):
    """Full Llama-3.2-1B shape (16 layers, hidden 2048, 32/8 heads, d 64,
    FFN 8192, vocab 128256, 16-bit limbed weights): two prompts of 130 and 77
    tokens in one prefill call (MFMA prefill attention, several query
    blocks), then 4 batch-2 decode steps; every logits row equals the
    oracle's."""
    m = llama
    V = m.shape.vocab
    prompts = [S.make_prompt(V, 130, 11), S.make_prompt(V, 77, 12)]
    n_new = 5
    rows = []
    toks = O.OracleModel(m, slots=2).generate(prompts, n_new, on_step=lambda s, lg: rows.append(lg.copy()))
    dm = D.DetintModel(m, n_slots=2)
    hist = host(dm.generate(prompts, n_new))
    for s in range(n_new):
        np.testing.assert_array_equal(hist[s], rows[s], err_msg=f"step {s}")
    np.testing.assert_array_equal(hist.argmax(-1).T, toks)


def test_llama_limbs_invariances(D, llama):
    """At the same shape with a 512-token prompt: its last-position logits,
    and the logits of the decode step after it, are the same whether the
    prompt is prefilled in one call, in two halves, or in one call together
    with another prompt."""
    import torch
    m = llama
    V = m.shape.vocab
    p = S.make_prompt(V, 512, 21)
    other = S.make_prompt(V, 300, 22)
    got = {}
    for mode in ("one", "halves", "batched"):
        dm = D.DetintModel(m, n_slots=2)
        rows = torch.zeros((4, V), dtype=torch.int32, device="cuda")   # prefill logits rows
        step = torch.zeros((1, V), dtype=torch.int32, device="cuda")   # the decode step's row
        if mode == "one":
            tok = dm.prefill([p], [0], [0], rows, 0)
            last = 0
        elif mode == "halves":
            dm.prefill([p[:256]], [0], [0], rows, 3)
            tok = dm.prefill([p[256:]], [256], [0], rows, 0)
            last = 0
        else:
            tok = dm.prefill([other, p], [0, 0], [1, 0], rows, 2)[1:]
            last = 3
        dm.decode(tok, [512], [0], 1, step, 0)
        got[mode] = (host(rows[last]), host(step[0]))
        del dm
    for mode in ("halves", "batched"):
        np.testing.assert_array_equal(got[mode][0], got["one"][0], err_msg=f"prefill logits, {mode}")
        np.testing.assert_array_equal(got[mode][1], got["one"][1], err_msg=f"decode logits, {mode}")


def test_qwen3_batch40_split_k_rows_match(D, qwen):
    """40 decode rows take the skinny split-K GEMMs (17-64 rows); row 0 is the
    golden prompt, whose first decode logits must continue the oracle-written
    hash chain, and row 39 must equal the same prompt decoded alone."""
    import torch
    m, g = qwen
    V = m.shape.vocab
    p0 = S.make_prompt(V, 64, g["prompt_seed"])
    prompts = [p0] + S.make_prompts(V, 39, 16, 64, 7)
    dm = D.DetintModel(m, n_slots=40)
    hist = host(dm.generate(prompts, 3))            # [3, 40, V]
    chain = D.logits_chain(hist[:, 0])
    assert chain == g["logits_chain"][0][:3]
    dm1 = D.DetintModel(m, n_slots=1)
    alone = host(dm1.generate([prompts[39]], 3))
    np.testing.assert_array_equal(hist[:, 39], alone[:, 0])


def test_llama_limbs_batch24_split_k_rows_match(D, llama):
    """24 decode rows of the 16-bit-limb model (skinny split-K limb GEMMs):
    rows 0 and 23 equal the same prompts decoded alone."""
    m = llama
    V = m.shape.vocab
    prompts = S.make_prompts(V, 24, 16, 40, 9)
    dm = D.DetintModel(m, n_slots=24)
    hist = host(dm.generate(prompts, 3))
    for r in (0, 23):
        dm1 = D.DetintModel(m, n_slots=1)
        alone = host(dm1.generate([prompts[r]], 3))
        np.testing.assert_array_equal(hist[:, r], alone[:, 0], err_msg=f"row {r}")
        del dm1


@pytest.mark.parametrize("nq,nkv,d,qkn", [(8, 2, 64, False), (4, 2, 128, True)])
def test_decode_attention_long_context_matches_prefill(D, nq, nkv, d, qkn):
    """Decode rows whose context runs past the cached rows the fused decode
    attention loads up front (512-768), so its double-buffered streaming
    loops run, in its launch shapes: 64 rows (a workgroup per KV head; 512
    threads for four 64-wide heads) and one row (a workgroup per query head).
    Each decode step's logits must equal the last-position logits of
    prefilling the prompt plus the decoded token in one call (the MFMA
    prefill attention, itself checked against the oracle)."""
    import torch
    shape = S.ModelShape("long_ctx", 1, 256, nq, nkv, d, 512, 1000, qkn, False,
                         1_000_000, 2048, 22)
    m = S.make_model(shape, seed=5)
    V, B = shape.vocab, 64
    prompts = S.make_prompts(V, B, 900, 1700, 31)
    dm = D.DetintModel(m, n_slots=B)
    first = torch.zeros((B, V), dtype=torch.int32, device="cuda")
    tok = dm.prefill(prompts, [0] * B, list(range(B)), first, 0)
    toks = host(tok).copy()
    step = torch.zeros((B, V), dtype=torch.int32, device="cuda")
    dm.decode(tok, [len(p) for p in prompts], list(range(B)), 1, step, 0, use_graph=False)
    got = host(step)
    del dm

    def reference(r):
        dm1 = D.DetintModel(m, n_slots=1)
        ref = torch.zeros((1, V), dtype=torch.int32, device="cuda")
        dm1.prefill([np.append(prompts[r], toks[r]).astype(np.int32)], [0], [0], ref, 0)
        return host(ref)[0]

    for r in (0, 13, 63):
        np.testing.assert_array_equal(got[r], reference(r), err_msg=f"batch-64 row {r}")
    # one row alone
    r = 7
    dm1 = D.DetintModel(m, n_slots=1)
    one = torch.zeros((1, V), dtype=torch.int32, device="cuda")
    t1 = dm1.prefill([prompts[r]], [0], [0], one, 0)
    assert int(host(t1)[0]) == int(toks[r])
    dm1.decode(t1, [len(prompts[r])], [0], 1, one, 0, use_graph=False)
    np.testing.assert_array_equal(host(one)[0], reference(r), err_msg="batch-1 row")


@pytest.mark.parametrize("name", ["tiny", "tiny_wide"])
def test_mixed_prefill_and_decode_rows_in_one_call(D, name):
    """BitExact LLM blog, "What the checks actually compare": mixed requests.
    One detint_forward call carries a decode row of sequence A (one token at
    its next position), the first prefill chunk of a new sequence B and the
    second chunk of sequence C, each in its own cache slot. Every row's
    logits equal the oracle's for that sequence run alone, and the caches
    equal the oracle's."""
    import torch
    m = S.make_model(name, seed=61)
    V = m.shape.vocab
    a, b, c = S.make_prompt(V, 30, 71), S.make_prompt(V, 23, 72), S.make_prompt(V, 41, 73)
    # oracle: each sequence alone in its slot
    om = O.OracleModel(m, slots=3)
    _, ta = om.forward(a, [30], [0], [0])
    want_a, _ = om.forward(ta, [1], [30], [0])
    want_b, _ = om.forward(b, [23], [0], [1])
    om.forward(c[:20], [20], [0], [2])
    want_c, _ = om.forward(c[20:], [21], [20], [2])
    # GPU: A prefilled and C's first chunk beforehand, then one mixed call
    dm = D.DetintModel(m, n_slots=3)
    scratch = torch.zeros((2, V), dtype=torch.int32, device="cuda")
    tok_a = host(dm.prefill([a, c[:20]], [0, 0], [0, 2], scratch, 0))[0]
    assert tok_a == int(ta[0])
    logits, _ = dm.forward(np.concatenate([[tok_a], b, c[20:]]).astype(np.int32), [1, 23, 21],
                           [30, 0, 20], [0, 1, 2])
    np.testing.assert_array_equal(logits[0], want_a[0], err_msg="decode row")
    np.testing.assert_array_equal(logits[1], want_b[0], err_msg="new prefill")
    np.testing.assert_array_equal(logits[2], want_c[0], err_msg="second chunk")
    np.testing.assert_array_equal(host(dm.kc), om.kc)
    np.testing.assert_array_equal(host(dm.vc), om.vc)
