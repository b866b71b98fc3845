#!/usr/bin/env python3
"""Benchmark of the integer-only forward pass on one MI355X.

A step is one greedy decode step of the Qwen3-0.6B-shaped integer model
(random init, seeded): embedding -> 28 layers (RMSNorm, QKV, q/k-norm,
RoPE, int8 KV cache, DI-Softmax attention, O-proj, SwiGLU FFN) -> final
RMSNorm -> tied lm_head -> int32 logits -> greedy token, captured once
into a HIP graph and replayed. The headline value is decode tokens/s at
batch 1 after a 64-token prompt. The same line reports batch-8 decode and
prefill on that model, the Llama-3.2-1B-shaped 16-bit-limb model (prefill
of 4 x 2048 tokens per call, batch-32 decode to a 4096-token context), the
25-shape int8 GEMM sweep, integer temperature / top-k sampling over the
vocabulary, the roofline of the decode step's fused final RMSNorm + lm_head
kernel, and the CPU oracle on this host. The Qwen runs'
logits are hashed and compared with the oracle-written golden chains
(tests/golden), so the timed runs are also verified runs.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-llama]
    python bench.py --roofline-only     # final-head kernel + copy calibration (counter runs)
    python bench.py --llama-only --llama-steps 64   # the Llama-shaped runs alone (profiling)
"""
from __future__ import annotations

import argparse
import copy
import hashlib
import json
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
I8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, TOP/s
PAGES_DECODE_B1 = 106.3      # the pages' A100 int8 decode tok/s at batch 1 (context only)
PROMPT_LEN = 64


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def timed(fn, n, torch):
    """Average seconds per call of fn over n calls, HIP events on the current stream."""
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(n):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / 1e3 / n


def timed_cold(fn, n, torch):
    """Average seconds of one fn launch with the caches flushed before it:
    reading a 1 GiB buffer evicts the 256 MB Infinity Cache and the L2s with
    clean lines (a write flush would leave dirty lines whose write-back
    during the timed launch halves the read bandwidth it sees; a decode
    step's caches hold clean weight lines), and each launch is bracketed by
    its own HIP events, so the figure is HBM streaming, not cache hits on
    the previous launch's data."""
    a = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
    tot = 0.0
    for _ in range(n):
        a.sum()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        torch.cuda.synchronize()
        tot += s.elapsed_time(e) / 1e3
    del a
    return tot / n


def head_case(D, m, torch):
    """detint_final_head for one row, logits only: the decode step's fused
    final RMSNorm + tied lm_head streaming kernel, launched on its own."""
    import numpy as np
    sh = m.shape
    rng = np.random.default_rng(5)
    h = torch.from_numpy(rng.integers(-(1 << 20), 1 << 20, (1, sh.hidden)).astype(np.int32)).cuda()
    g = torch.from_numpy(m.final_norm).cuda()
    emb = torch.from_numpy(m.emb).cuda()
    emb_m = torch.from_numpy(m.emb_m).cuda()
    ws = torch.empty(D.library().detint_final_head_workspace(1, sh.vocab, sh.hidden),
                     dtype=torch.uint8, device="cuda")
    logits, _ = D.detint_final_head(h, g, emb, None, emb_m, sh.w_k, sh.f_l, ws=ws, with_token=False)
    fn = lambda: D.detint_final_head(h, g, emb, None, emb_m, sh.w_k, sh.f_l, logits, None, ws,
                                     with_token=False)
    # int8 table, its int32 mantissas, int32 logits out; the row and its gains
    nbytes = sh.vocab * sh.hidden + 8 * sh.vocab + 6 * sh.hidden
    return fn, nbytes


def kernel_source_sha() -> str:
    """sha256 over the sources the fused final-head kernel is compiled from."""
    h = hashlib.sha256()
    for f in ("decode.hip", "dev_int.h", "internal.h"):
        h.update((ROOT / "integer_only_deterministic_amd" / "csrc" / f).read_bytes())
    return h.hexdigest()


def traffic_from_profiles():
    """HBM bytes per final-head launch from the committed counter summary, or
    None when the kernel source changed since the counters were taken."""
    f = ROOT / "profiles" / "final_head_hbm_traffic.txt"
    if not f.exists():
        return None
    vals = {}
    for line in f.read_text().splitlines():
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != kernel_source_sha():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def roofline_only(D, S, torch):
    import dataclasses
    # the embedding / lm_head tensor is drawn independently of the layers
    m = S.make_model(dataclasses.replace(S.SHAPES["qwen3_0.6b"], n_layers=0), seed=0)
    fn, nbytes = head_case(D, m, torch)
    for _ in range(3):
        fn()
    t = timed_cold(fn, 20, torch)
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"final_head_us": t * 1e6, "final_head_algorithmic_bytes": nbytes,
                      "copy_bytes": src.numel(), "copy_launches": 5,
                      "kernel_source_sha256": kernel_source_sha()}))


def decode_run(D, dm, prompts, warmup, steps, torch):
    B = len(prompts)
    V = dm.shape.vocab
    hist = torch.empty((1 + warmup + steps, B, V), dtype=torch.int32, device="cuda")
    dm.reset_cache()
    tok = dm.prefill(prompts, [0] * B, list(range(B)), hist, 0)
    step = dm.decode_step_fn(tok, [len(p) for p in prompts], list(range(B)), hist, B)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return hist, (t1 - t0), ev0.elapsed_time(ev1) / 1e3


def gemm_sweep(D, S, torch):
    """The 25-shape int8 GEMM sweep, per-row x per-column requant to int8.
    M >= 512: TOP/s against the i8 MFMA peak (back-to-back launches);
    M <= 64: GB/s against HBM, each launch cache-cold."""
    res = {}
    for Kd, Nd in S.GEMM_SWEEP_KN:
        g = S.make_gemm_operands(max(S.GEMM_SWEEP_M), Nd, Kd, seed=7)
        A, Wt = torch.from_numpy(g["A"]).cuda(), torch.from_numpy(g["W"]).cuda()
        rm, rk = torch.from_numpy(g["row_m"]).cuda(), torch.from_numpy(g["row_k"]).cuda()
        cm = torch.from_numpy(g["col_m"]).cuda()
        for M in S.GEMM_SWEEP_M:
            out = torch.empty((M, Nd), dtype=torch.int8, device="cuda")
            Am, rmm, rkm = A[:M], rm[:M], rk[:M]
            f = lambda: D.detint_gemm_i8(Am, Wt, rmm, rkm, cm, g["col_k"], 0, D.REQ_I8, out)
            for _ in range(3):
                f()
            key = f"M{M}_K{Kd}_N{Nd}"
            if M >= 512:
                t = timed(f, 20, torch)
                tops = 2 * M * Nd * Kd / t / 1e12
                res[key] = {"tops": round(tops, 1), "frac_i8_mfma": round(tops / I8_PEAK_TOPS, 4)}
            else:
                t = timed_cold(f, 10, torch)
                gbs = (M * Kd + Nd * Kd + M * Nd + 8 * (M + Nd)) / t / 1e9
                res[key] = {"gbs": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                            "us": round(t * 1e6, 2)}
            del out
        del A, Wt
    return res


def llama_case(D, S, torch, dec_steps: int):
    """Llama-3.2-1B-shaped model with 16-bit limbed weights: 32 seeded
    2048-token prompts prefilled 4 per call, then batch-32 greedy decode
    from position 2048 (HIP-graph segments of 256 steps)."""
    import numpy as np
    m = S.make_model("llama3.2_1b", seed=0)
    sh = m.shape
    B, P, SEG = 32, 2048, 256
    prompts = S.make_prompts(sh.vocab, B, P, P, 5)
    dm = D.DetintModel(m, n_slots=B)
    scratch = torch.empty((B, sh.vocab), dtype=torch.int32, device="cuda")
    toks, times = [], []
    for c in range(B // 4):
        sl = list(range(4 * c, 4 * c + 4))
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        toks.append(dm.prefill([prompts[i] for i in sl], [0] * 4, sl, scratch, 4 * c))
        torch.cuda.synchronize()
        times.append(time.perf_counter() - t0)
    t_pref = float(np.median(times[1:]))
    L, H, F, nq, nkv, d = sh.n_layers, sh.hidden, sh.ffn, sh.n_q, sh.n_kv, sh.head_dim
    lin_mac = L * H * ((nq + 2 * nkv) * d + nq * d + 2 * F) + L * F * H   # per token
    att_mac = L * nq * d * 3 * 4 * (P * (P + 1) // 2)                     # QK^T + 2 P.V limbs, causal
    ops = 2 * (2 * lin_mac * 4 * P + att_mac)                              # x2 limbs on the linears
    tok = torch.cat(toks)
    hist = torch.empty((SEG, B, sh.vocab), dtype=torch.int32, device="cuda")
    done, t_dec, n_timed, pos = 0, 0.0, 0, P
    first = None
    while done < dec_steps:
        n = min(SEG, dec_steps - done)
        step = dm.decode_step_fn(tok, [pos] * B, list(range(B)), hist, 0)
        step()                      # first replay of a fresh graph: untimed
        torch.cuda.synchronize()
        if first is None:
            first = hist[0, 0].clone()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n - 1):
            step()
        e1.record()
        torch.cuda.synchronize()
        t_dec += e0.elapsed_time(e1) / 1e3
        n_timed += n - 1
        done += n
        pos += n
    # batch invariance: prompt 0 alone, first decode step's logits equal row 0's
    dm1 = dm
    dm1.reset_cache()
    t1 = dm1.prefill([prompts[0]], [0], [0], scratch, 0)
    h1 = torch.empty((1, 1, sh.vocab), dtype=torch.int32, device="cuda")
    dm1.decode_step_fn(t1, [P], [0], h1, 0, use_graph=False)()
    torch.cuda.synchronize()
    inv = bool(torch.equal(h1[0, 0], first))
    w_bytes = 2 * (L * H * ((nq + 2 * nkv) * d + nq * d + 2 * F + F) + sh.vocab * H)
    ctx_avg = P + 1 + (dec_steps - 1) / 2
    step_bytes = w_bytes + 2 * L * nkv * d * B * ctx_avg
    tps = B * n_timed / t_dec
    return {
        "workload": "Llama-3.2-1B-shaped integer model, 16-bit limbed weights (random init, seed 0)",
        "prefill_4x2048_tok_s": round(4 * P / t_pref, 1),
        "prefill_ms_per_call": round(1e3 * t_pref, 2),
        "prefill_tops": round(ops / t_pref / 1e12, 1),
        "prefill_frac_i8_mfma": round(ops / t_pref / 1e12 / I8_PEAK_TOPS, 4),
        "decode_b32_tok_s": round(tps, 1),
        "decode_b32_ms_per_step": round(1e3 * t_dec / n_timed, 3),
        "decode_b32_hbm_frac": round(step_bytes * tps / B / 1e9 / HBM_PEAK_GBS, 4),
        "decode_ctx_range": [P + 1, P + dec_steps],
        "batch_invariant_row0": inv,
    }


def sampling_case(D, torch, with_cpu: bool):
    """detint_sample (integer temperature / top-k sampling) on rows of the
    Qwen3-shaped vocabulary (151936 seeded int32 logits, gaps of a few units
    at 16 fractional bits), temperature 1, batch 1 and 8: all tokens, top-50,
    top-p 0.9 and both. Algorithmic bytes per call: one read of the logits plus the draw
    and the token per row. The oracle's tokens for the same rows and draws
    are compared, and its time per row is reported beside it."""
    import numpy as np
    V, tm, tk = 151936, 23637, 15
    rng = np.random.default_rng(2026)
    lg_h = rng.normal(0, 3 * 65536, (8, V)).astype(np.int32)
    dr_h = rng.integers(0, 1 << 32, 8, dtype=np.uint64).astype(np.uint32)
    lg, dr = torch.from_numpy(lg_h).cuda(), torch.from_numpy(dr_h.view(np.int32)).cuda()
    ws = torch.empty(D.detint_sample_workspace(8, V), dtype=torch.uint8, device="cuda")
    res = {"workload": "detint_sample over %d int32 logits per row, temperature 1" % V}
    for R in (1, 8):
        for k, p in ((0, 65536), (50, 65536), (0, 58982), (50, 58982)):
            out = torch.empty(R, dtype=torch.int32, device="cuda")
            f = lambda: D.detint_sample(lg[:R], k, tm, tk, dr[:R], out, top_p=p, ws=ws)
            for _ in range(3):
                f()
            t = timed(f, 50, torch)
            nbytes = R * (4 * V + 8)
            key = "b%d_%s%s" % (R, "top%d" % k if k else ("" if p < 65536 else "all"),
                                ("_" if k else "") + "top_p0.9" if p < 65536 else "")
            res[key] = {"us": round(t * 1e6, 2), "gbs": round(nbytes / t / 1e9, 1),
                        "frac_hbm": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4)}
            if with_cpu and R == 8:
                import oracle as O
                t0 = time.perf_counter()
                want = O.sample(lg_h, k, tm, tk, dr_h, top_p=p)
                res[key]["oracle_ms_per_row"] = round((time.perf_counter() - t0) * 1e3 / R, 2)
                res[key]["tokens_equal_oracle"] = bool(np.array_equal(out.cpu().numpy(), want))
    return res


def cpu_baseline(m, p0, seconds: float, gpu_tokens):
    import numpy as np
    import oracle as O
    threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    om = O.OracleModel(m, slots=1)
    t0 = time.perf_counter()
    _, tok = om.forward(p0, [len(p0)], [0], [0])
    t1 = time.perf_counter()
    toks = [int(tok[0])]
    pos = len(p0)
    while time.perf_counter() - t1 < seconds and len(toks) < len(gpu_tokens):
        _, tok = om.forward(np.array([toks[-1]], np.int32), [1], [pos], [0])
        pos += 1
        toks.append(int(tok[0]))
    t2 = time.perf_counter()
    n = len(toks) - 1
    agree = toks == [int(t) for t in gpu_tokens[: len(toks)]]
    return dict(value=round(n / (t2 - t1), 3) if n else None, unit="tok/s", cores=threads,
                kind="oracle",
                sample=f"batch-1 greedy decode of the same model: {len(p0)}-token prefill "
                       f"({t1 - t0:.1f} s, untimed) then {n} decode steps in {t2 - t1:.1f} s; "
                       f"tokens {'equal' if agree else 'DIFFER from'} the GPU run's")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=448)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--roofline-only", action="store_true")
    ap.add_argument("--no-llama", action="store_true")
    ap.add_argument("--llama-only", action="store_true")
    ap.add_argument("--llama-steps", type=int, default=2047)
    args = ap.parse_args()
    if args.gpus != 1:
        log("bench.py: runs on one GPU only (the integer forward pass is data-parallel by "
            "sequence: more GPUs would each hold the weights and their own KV-cache slots, "
            "with no collective in the step). Use --gpus 1.")
        sys.exit(2)
    if args.warmup + args.steps > 511:
        log("bench.py: warmup + steps must be <= 511 (64-token prompt + 512 steps fit the cache)")
        sys.exit(2)

    import numpy as np
    import torch

    import detint_synth as S
    import integer_only_deterministic_amd as D

    D.library()
    torch.cuda.set_device(0)
    if args.roofline_only:
        roofline_only(D, S, torch)
        return
    if args.llama_only:
        print(json.dumps(llama_case(D, S, torch, args.llama_steps)), flush=True)
        return

    gold = json.loads((ROOT / "tests" / "golden" / "qwen3_b1.json").read_text())
    gold8 = json.loads((ROOT / "tests" / "golden" / "qwen3_b8.json").read_text())
    log("building the seeded Qwen3-0.6B-shaped model ...")
    m = S.make_model("qwen3_0.6b", seed=gold["model_seed"])
    sh = m.shape
    assert S.model_digest(m) == gold["model_digest"]
    dm = D.DetintModel(m, n_slots=8)
    p0 = S.make_prompt(sh.vocab, PROMPT_LEN, gold["prompt_seed"])
    co = S.make_prompts(sh.vocab, 7, 16, 256, gold["coprompt_seed"])
    W, K = args.warmup, args.steps

    # ---- decode, batch 1 (headline) ----
    log(f"decode b1: prefill {PROMPT_LEN}, {W} warmup + {K} timed graph replays")
    hist, wall1, ev1 = decode_run(D, dm, [p0], W, K, torch)
    h1 = hist.cpu().numpy()
    chain1 = D.logits_chain(h1[:, 0])
    exact_b1 = chain1 == gold["logits_chain"][0][: len(chain1)]
    gpu_tokens = h1[:, 0].argmax(-1)
    tps1 = K / wall1

    # ---- decode, batch 8: the prompt among 7 random co-prompts ----
    log("decode b8")
    hist8, wall8, _ = decode_run(D, dm, [p0] + co, W, K, torch)
    h8 = hist8.cpu().numpy()
    exact_b8 = all(D.logits_chain(h8[:, b]) == gold8["logits_chain"][b][: h8.shape[0]] for b in range(8))
    tps8 = 8 * K / wall8
    del hist8, h8

    # ---- decode, batch 1, with per-channel key gains on every layer (the
    # same weights, seeded gains in [0, 2]): the cost of the rescale path ----
    log("decode b1 with key gains")
    mg = copy.copy(m)
    mg.layers = [copy.copy(L) for L in m.layers]
    S.with_key_gains(mg, seed=gold["model_seed"] + 1, gmax=2)
    dmg = D.DetintModel(mg, n_slots=1)
    _, wallg, _ = decode_run(D, dmg, [p0], W, K, torch)
    tps_gain = K / wallg
    del dmg, mg
    torch.cuda.empty_cache()

    # ---- prefill: the batch-8 ragged prompts in one call, and the 64-token prompt ----
    log("prefill")
    scratch = torch.empty((8, sh.vocab), dtype=torch.int32, device="cuda")
    rag = [p0] + co
    ntok = sum(len(p) for p in rag)
    t_rag = timed(lambda: dm.prefill(rag, [0] * 8, list(range(8)), scratch, 0), 5, torch)
    t_64 = timed(lambda: dm.prefill([p0], [0], [0], scratch, 0), 10, torch)

    # ---- the 25-shape int8 GEMM sweep ----
    log("GEMM sweep")
    gemm = gemm_sweep(D, S, torch)

    # ---- roofline of the largest-traffic kernel of the step: the fused
    # final RMSNorm + lm_head GEMV (one launch streams the 155.6 MB table) ----
    log("final-head kernel")
    fn, nbytes = head_case(D, m, torch)
    for _ in range(3):
        fn()
    t_head = timed_cold(fn, 30, torch)
    achieved = nbytes / t_head / 1e9
    traffic = traffic_from_profiles()

    llama = None
    if not args.no_llama:
        del dm
        torch.cuda.empty_cache()
        log("Llama-3.2-1B-shaped model: prefill 4 x 2048 per call, batch-32 decode to 4096")
        llama = llama_case(D, S, torch, args.llama_steps)

    log("integer sampling")
    sampling = sampling_case(D, torch, not args.no_cpu)
    cpu = None if args.no_cpu else cpu_baseline(m, p0, args.cpu_seconds, gpu_tokens)

    weights = sum(L.wqkv.size + L.wo.size + L.wgu.size + L.wd.size for L in m.layers) + m.emb.size
    ctx_avg = PROMPT_LEN + 1 + W + (K + 1) / 2
    step_bytes = weights + 2 * sh.n_layers * sh.n_kv * sh.head_dim * ctx_avg
    big = [v["frac_i8_mfma"] for v in gemm.values() if "frac_i8_mfma" in v]
    line = {
        "metric": "decode tok/s @bs1/8, prefill tok/s; i8 GEMM % MFMA peak; bit-exact logits",
        "value": round(tps1, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(1e3 * wall1 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(tps1 / PAGES_DECODE_B1, 2),
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "Qwen3-0.6B-shaped integer model (random init, seed 0), greedy "
                               "decode at batch 1 after a 64-token prompt, one HIP-graph replay per token",
                   "batch": 1, "prompt_len": PROMPT_LEN, "decode_steps_timed": K,
                   "ctx_range": [PROMPT_LEN + 1 + W, PROMPT_LEN + W + K]},
        "bit_exact": {"decode_b1_vs_oracle_chain": bool(exact_b1),
                      "decode_b8_vs_oracle_chain": bool(exact_b8),
                      "b1_logits_hash": chain1[-1][:12]},
        "decode_b1_key_gains_tok_s": round(tps_gain, 2),
        "decode_b8_tok_s": round(tps8, 1),
        "prefill_tok_s": {"ragged_8_prompts_%d_tokens" % ntok: round(ntok / t_rag, 1),
                          "prompt_64": round(PROMPT_LEN / t_64, 1)},
        "decode_b1_hbm_frac": round(step_bytes * tps1 / 1e9 / HBM_PEAK_GBS, 4),
        "llama3.2_1b_limbs": llama,
        "sampling": sampling,
        "gemm_sweep_req_i8": gemm,
        "gemm_best_frac_i8_mfma": round(max(big), 4),
        "roofline": {"bound": "hbm",
                     "kernel": "fused final RMSNorm + tied lm_head GEMV, 1 row (fgemv<1,2,1,1,4>)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": nbytes,
                     "avg_launch_us": round(t_head * 1e6, 2)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
