"""Decode attention at the Llama-3.2-1B shape's long contexts, compared with
the CPU oracle (DetLLM blog, footnote 9: the zero-tolerance checks include a
4k-token context; DetLLM README, "Usage": long-context checks).

The model is one decoder layer with the Llama-3.2-1B head layout (32 query /
8 KV heads of width 64, no q/k-norm, 16-bit limbed weights, RoPE base 5e5,
a 4096-position cache) on a hidden size of 256, so the oracle can recompute
every position in seconds. Prompts of about 2048 tokens are prefilled the
way the benchmark does (four per call), then decoded greedily until row 0
reaches a 4096-token context, in the two launch shapes the fused decode
attention takes for this head layout: one row (a workgroup per query head)
and 32 rows (a workgroup per KV head, four heads, 512 threads). The oracle
then recomputes the checked rows teacher-forced over their whole sequence
(prefill/decode invariance), and every decode step's logits, the greedy
tokens and the cached K/V bytes must be identical."""
import numpy as np
import pytest

import detint_synth as S
import oracle as O

pytestmark = pytest.mark.gpu

SHAPE = S.ModelShape("llama_heads_4k", 1, 256, 32, 8, 64, 512, 1000, False, True,
                     500_000, 4096, 30)


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


@pytest.mark.parametrize("B,check", [(1, (0,)), (32, (0, 17, 31))])
def test_long_context_decode_matches_oracle(D, B, check):
    import torch
    m = S.make_model(SHAPE, seed=41)
    V, P, T = SHAPE.vocab, 2048, SHAPE.max_pos
    # row b has 2048 - b prompt tokens: ragged contexts, row 0 ends at 4096
    prompts = [S.make_prompt(V, P - b, 700 + b) for b in range(B)]
    n_steps = T - P                                  # positions 2048 .. 4095 for row 0
    dm = D.DetintModel(m, n_slots=B)
    hist = torch.zeros((n_steps + 1, B, V), dtype=torch.int32, device="cuda")
    toks = []
    for c in range(0, B, 4):
        sl = list(range(c, min(B, c + 4)))
        toks.append(dm.prefill([prompts[i] for i in sl], [0] * len(sl), sl, hist, c))
    tok = torch.cat(toks)
    dm.decode(tok, [len(p) for p in prompts], list(range(B)), n_steps, hist, B, use_graph=True)
    got = host(hist)                                 # [n_steps + 1, B, V]
    kc, vc = host(dm.kc), host(dm.vc)
    del dm
    for r in check:
        L = len(prompts[r])
        steps = min(n_steps, T - L)                  # decode steps that stay inside the cache
        gen = got[: steps + 1, r].argmax(-1).astype(np.int32)
        seq = np.concatenate([prompts[r], gen[:steps]]).astype(np.int32)
        om = O.OracleModel(m, slots=1)
        want, nxt = om.forward(seq, [len(seq)], [0], [0], all_rows=True)
        # step s of row r is position L - 1 + s
        np.testing.assert_array_equal(got[: steps + 1, r], want[L - 1:], err_msg=f"B={B} row {r}")
        np.testing.assert_array_equal(gen, nxt[L - 1:])
        n = len(seq)
        np.testing.assert_array_equal(kc[0, r, :, :n], om.kc[0, 0, :, :n], err_msg=f"K row {r}")
        np.testing.assert_array_equal(vc[0, r, :, :n], om.vc[0, 0, :, :n], err_msg=f"V row {r}")
    assert len(prompts[0]) + n_steps == T
