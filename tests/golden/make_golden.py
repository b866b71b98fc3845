"""Writes the stored expected values under tests/golden/ by running ONLY the
CPU oracle on seeded synthetic inputs (no GPU code is imported).

    python tests/golden/make_golden.py qwen3_b1     # 64-token prompt + 512 greedy tokens
    python tests/golden/make_golden.py qwen3_b8     # same prompt inside a batch of 8
    python tests/golden/make_golden.py llama_c4     # Llama-shaped rows 0 and 31, context 4096

Each file records the model digest, prompt seeds, per-step chained logits
hashes (SHA-256 over int32 little-endian logits, chained from SHA-256 of the
tag "detint-v0") and the greedy tokens.
"""
import hashlib
import json
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parents[2]
sys.path.insert(0, str(ROOT))

import numpy as np  # noqa: E402

import detint_synth as S  # noqa: E402
import oracle as O  # noqa: E402

HERE = Path(__file__).resolve().parent

QWEN_MODEL_SEED = 0
QWEN_PROMPT_SEED = 1
QWEN_COPROMPT_SEED = 2
N_NEW = 512


def qwen_prompts(m, batch: int):
    p0 = S.make_prompt(m.shape.vocab, 64, QWEN_PROMPT_SEED)
    if batch == 1:
        return [p0]
    return [p0] + S.make_prompts(m.shape.vocab, batch - 1, 16, 256, QWEN_COPROMPT_SEED)


def run(tag: str, batch: int):
    t0 = time.time()
    m = S.make_model("qwen3_0.6b", seed=QWEN_MODEL_SEED)
    prompts = qwen_prompts(m, batch)
    om = O.OracleModel(m, slots=batch)
    chains = [O.chain_init() for _ in range(batch)]
    hashes = [[] for _ in range(batch)]

    def on_step(s, lg):
        for b in range(batch):
            chains[b] = O.chain_step(chains[b], lg[b])
            hashes[b].append(chains[b].hex())
        if s % 64 == 0:
            print(f"step {s} {time.time() - t0:.1f}s", flush=True)

    toks = om.generate(prompts, N_NEW, on_step=on_step)
    tchain = []
    for b in range(batch):
        h = O.chain_init()
        for t in toks[b]:
            h = O.chain_step(h, np.array([t], np.int32))
        tchain.append(h.hex())
    out = dict(
        what="CPU-oracle greedy run of the seeded Qwen3-0.6B-shaped integer model",
        model="qwen3_0.6b", model_seed=QWEN_MODEL_SEED, model_digest=S.model_digest(m),
        prompt_seed=QWEN_PROMPT_SEED, coprompt_seed=QWEN_COPROMPT_SEED,
        prompt_lens=[len(p) for p in prompts], n_new=N_NEW,
        tokens=[t.tolist() for t in toks], logits_chain=hashes, token_chain=tchain,
        oracle_seconds=round(time.time() - t0, 1))
    (HERE / f"{tag}.json").write_text(json.dumps(out))
    print(tag, "logits hash", hashes[0][-1][:12], "tokens", toks[0][:8], flush=True)


# Llama-3.2-1B-shaped 16-bit-limb model: 32 seeded prompts of 2048 tokens
# (prompt set seed 5), decoded greedily to a 4096-token context. The oracle
# runs the checked rows one at a time (batch invariance: a row's bits do not
# depend on its batch), prefilling each prompt in 256-token chunks so that
# the chunk ends give logits at 8 prompt positions (chunked prefill is
# invariant too), then decoding one token per step.
C4_MODEL_SEED = 0
C4_PROMPT_SEED = 5
C4_PROMPTS, C4_PROMPT_LEN, C4_CONTEXT, C4_CHUNK = 32, 2048, 4096, 256
C4_ROWS = (0, 31)
C4_CHAIN_EVERY = 16


def c4_run(shape="llama3.2_1b", rows=C4_ROWS, prompt_len=C4_PROMPT_LEN, context=C4_CONTEXT,
           chunk=C4_CHUNK, out_path=None):
    """Oracle-only expected values of the batch-32 Llama-shaped run: for each
    checked row, the logits hash at every chunk end of the prompt, the
    chained logits hash of the decode (step 0 = the prompt's last position,
    step s = position prompt_len - 1 + s, up to position context - 1), kept
    every C4_CHAIN_EVERY steps and at the last step, and the greedy tokens."""
    t_all = time.time()
    m = S.make_model(shape, seed=C4_MODEL_SEED)
    V = m.shape.vocab
    prompts = S.make_prompts(V, C4_PROMPTS, prompt_len, prompt_len, C4_PROMPT_SEED)
    res = []
    for r in rows:
        t0 = time.time()
        p = prompts[r]
        om = O.OracleModel(m, slots=1)
        pos_hash = {}
        for c0 in range(0, prompt_len, chunk):
            c1 = min(prompt_len, c0 + chunk)
            lg, nxt = om.forward(p[c0:c1], [c1 - c0], [c0], [0])
            pos_hash[c1 - 1] = hashlib.sha256(np.ascontiguousarray(lg[0], "<i4").tobytes()).hexdigest()
        t_pre = time.time() - t0
        h = O.chain_step(O.chain_init(), lg[0])
        chain = {0: h.hex()}
        toks = [int(nxt[0])]
        n_steps = context - prompt_len
        for s in range(1, n_steps + 1):
            lg, nxt = om.forward(np.array([toks[-1]], np.int32), [1], [prompt_len - 1 + s], [0])
            h = O.chain_step(h, lg[0])
            toks.append(int(nxt[0]))
            if s % C4_CHAIN_EVERY == 0 or s == n_steps:
                chain[s] = h.hex()
            if s % 256 == 0:
                print(f"row {r} step {s} {time.time() - t0:.0f}s", flush=True)
        res.append(dict(row=r, prompt_sha256=hashlib.sha256(p.tobytes()).hexdigest(),
                        prompt_logits_sha256={str(k): v for k, v in sorted(pos_hash.items())},
                        logits_chain={str(k): v for k, v in sorted(chain.items())},
                        tokens=toks, oracle_prefill_seconds=round(t_pre, 1),
                        oracle_seconds=round(time.time() - t0, 1)))
        print(f"row {r}: chain {h.hex()[:12]} in {time.time() - t0:.0f}s", flush=True)
    out = dict(
        what="CPU-oracle greedy rows of the batch-32 Llama-3.2-1B-shaped 16-bit-limb run",
        model=shape, model_seed=C4_MODEL_SEED, model_digest=S.model_digest(m),
        prompt_seed=C4_PROMPT_SEED, n_prompts=C4_PROMPTS, prompt_len=prompt_len, context=context,
        chunk=chunk, chain_every=C4_CHAIN_EVERY, rows=res,
        oracle_seconds=round(time.time() - t_all, 1))
    (out_path or HERE / "llama_c4.json").write_text(json.dumps(out))


if __name__ == "__main__":
    which = sys.argv[1:] or ["qwen3_b1"]
    for w in which:
        if w == "llama_c4":
            c4_run()
        else:
            run(w, {"qwen3_b1": 1, "qwen3_b8": 8}[w])
