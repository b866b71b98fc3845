"""Writes the stored expected values under tests/golden/ by running ONLY the
CPU oracle on seeded synthetic inputs (no GPU code is imported).

    python tests/golden/make_golden.py qwen3_b1     # 64-token prompt + 512 greedy tokens
    python tests/golden/make_golden.py qwen3_b8     # same prompt inside a batch of 8

Each file records the model digest, prompt seeds, per-step chained logits
hashes (SHA-256 over int32 little-endian logits, chained from SHA-256 of the
tag "detint-v0") and the greedy tokens.
"""
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


if __name__ == "__main__":
    which = sys.argv[1:] or ["qwen3_b1"]
    for w in which:
        run(w, {"qwen3_b1": 1, "qwen3_b8": 8}[w])
