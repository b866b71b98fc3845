#!/usr/bin/env python3
"""Benchmark of the integer-only forward pass on one MI355X.

A step is one greedy decode step of the Qwen3-0.6B-shaped integer model
(random init, seeded): embedding -> 28 layers (RMSNorm, QKV, q/k-norm,
RoPE, int8 KV cache, DI-Softmax attention, O-proj, SwiGLU FFN) -> final
RMSNorm -> tied lm_head -> int32 logits -> greedy token, captured once
into a HIP graph and replayed. The headline value is decode tokens/s at
batch 1 after a 64-token prompt, timed over a window of the 512-step decode
centred on the middle of its context range; its roofline is the whole
step's HBM traffic against 8 TB/s. The same line reports the other
configurations: one Qwen-style layer (hidden 256) with its latency, kernel
count and the oracle's single-thread time; the 25-shape int8 GEMM sweep with
the oracle's GOPS; batch-8 decode and prefill on the Qwen3 shape; the
Llama-3.2-1B-shaped 16-bit-limb model (prefill of 4 x 2048 tokens per call,
batch-32 decode to a 4096-token context, rows 0 and 31 checked against the
oracle-written chain); integer sampling; the fused final-head kernel's own
roofline; and the CPU oracle on this host. Every Qwen and Llama run's logits
are hashed and compared with the oracle-written golden chains (tests/golden),
so the timed runs are also verified runs.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-llama]
    python bench.py --roofline-only     # final-head kernel + copy calibration (counter runs)
    python bench.py --decode-only       # batch-1 decode steps + copy calibration (counter runs)
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


def timed_graph(fn, n, torch, reps=5):
    """Average seconds per call of fn with the host's launch cost taken out:
    n back-to-back calls captured once into a HIP graph, replayed reps
    times, HIP events around the replays (a standalone call's argument
    checks and Python marshalling take longer than a small GEMM runs)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(n):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3 / (n * reps)


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


def kernel_source_sha(files=("decode.hip", "dev_int.h", "internal.h")) -> str:
    """sha256 over the sources a measured kernel set is compiled from."""
    h = hashlib.sha256()
    for f in files:
        h.update((ROOT / "integer_only_deterministic_amd" / "csrc" / f).read_bytes())
    return h.hexdigest()


# sources of the batch-1 decode step's kernels
DECODE_SOURCES = ("decode.hip", "attention.hip", "rowops.hip", "qkv_dev.h", "dev_int.h", "internal.h")


def profile_value(name, key, files):
    """A number from a committed counter summary under profiles/, or None
    when the kernels' sources changed since the counters were taken."""
    f = ROOT / "profiles" / name
    if not f.exists():
        return None
    vals = {}
    for line in f.read_text().splitlines():
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != kernel_source_sha(files):
        return None
    try:
        return float(vals[key])
    except (KeyError, ValueError):
        return None


def graph_kernel_count(fn, torch) -> int:
    """Kernel nodes of fn's launches, captured into a HIP graph."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    g = torch.cuda.CUDAGraph(keep_graph=True)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=st):
        fn()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    h = ctypes.c_void_p(g.raw_cuda_graph())
    n = ctypes.c_size_t(0)
    if hip.hipGraphGetNodes(h, None, ctypes.byref(n)) != 0:
        return -1
    nodes = (ctypes.c_void_p * n.value)()
    hip.hipGraphGetNodes(h, nodes, ctypes.byref(n))
    kind, k = ctypes.c_int(0), 0
    for nd in nodes:
        hip.hipGraphNodeGetType(ctypes.c_void_p(nd), ctypes.byref(kind))
        k += kind.value == 0                       # hipGraphNodeTypeKernel
    del g
    return k


def copy_calibration(torch):
    """Five plain 256 MiB device copies, for scaling the HBM byte counters."""
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    return src.numel()


def roofline_only(D, S, torch):
    import dataclasses
    # the embedding / lm_head tensor is drawn independently of the layers
    m = S.make_model(dataclasses.replace(S.SHAPES["qwen3_0.6b"], n_layers=0), seed=0)
    fn, nbytes = head_case(D, m, torch)
    for _ in range(3):
        fn()
    t = timed_cold(fn, 20, torch)
    nb = copy_calibration(torch)
    print(json.dumps({"final_head_us": t * 1e6, "final_head_algorithmic_bytes": nbytes,
                      "copy_bytes": nb, "copy_launches": 5,
                      "kernel_source_sha256": kernel_source_sha()}))


def decode_run(D, dm, prompts, warmup, steps, torch):
    """Prefill, `warmup` untimed decode steps, then `steps` timed graph
    replays; returns the logits history and the wall / event seconds."""
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
    """The 25-shape int8 GEMM sweep, per-row x per-column requant to int8,
    each call with the workspace detint_gemm_workspace asks for (split-K on
    few-tile shapes). M >= 512: TOP/s against the i8 MFMA peak (20
    back-to-back calls replayed from a HIP graph, so the host's per-call
    cost is not timed); M <= 64: GB/s against HBM, each launch cache-cold
    (its flush covers the host's launch cost)."""
    res = {}
    for Kd, Nd in S.GEMM_SWEEP_KN:
        g = S.make_gemm_operands(max(S.GEMM_SWEEP_M), Nd, Kd, seed=7)
        A, Wt = torch.from_numpy(g["A"]).cuda(), torch.from_numpy(g["W"]).cuda()
        rm, rk = torch.from_numpy(g["row_m"]).cuda(), torch.from_numpy(g["row_k"]).cuda()
        cm = torch.from_numpy(g["col_m"]).cuda()
        for M in S.GEMM_SWEEP_M:
            out = torch.empty((M, Nd), dtype=torch.int8, device="cuda")
            Am, rmm, rkm = A[:M], rm[:M], rk[:M]
            need = D.detint_gemm_workspace(M, Nd, Kd)
            ws = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None
            f = lambda: D.detint_gemm_i8(Am, Wt, rmm, rkm, cm, g["col_k"], 0, D.REQ_I8, out, ws=ws)
            for _ in range(3):
                f()
            key = f"M{M}_K{Kd}_N{Nd}"
            if M >= 512:
                t = timed_graph(f, 20, torch)
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


def omp_threads(n: int):
    """Thread count of the oracle's OpenMP regions issued from this thread."""
    import ctypes
    ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(n))


def host_threads() -> int:
    return int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))


def c0_case(D, S, torch, with_cpu: bool):
    """One Qwen-style decoder layer (hidden 256, 4/2 heads, d 64, FFN 768),
    prefill of 64 tokens on a seeded residual in [-2^15, 2^15): the output
    residual against the oracle's, the GPU layer latency (HIP events, 50
    back-to-back calls on fresh copies of the input; also replayed from a
    HIP graph, without the host's launch cost), the kernels one call
    launches, and the oracle's time on one host thread."""
    import numpy as np
    m = S.make_model("layer256", seed=1)
    h0 = S.make_residual(64, 256, seed=2)
    dm = D.DetintModel(m, n_slots=1)
    cu, st, sl = (torch.tensor(a, dtype=torch.int32, device="cuda") for a in ([0, 64], [0], [0]))
    ws = dm.workspace(64, 1)
    n = 50
    hs = torch.from_numpy(np.ascontiguousarray(h0)).cuda().repeat(n + 1, 1, 1)

    def call(i):
        D._call("detint_layer_forward", dm.handle, 0, D._p(hs[i]), D._p(dm.kc), D._p(dm.vc), 1, 64,
                D._p(cu), D._p(st), D._p(sl), 1, 64, D._p(ws), ws.numel(), D._stream())

    call(n)
    got = hs[n].cpu().numpy()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n):
        call(i)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / n
    kernels = graph_kernel_count(lambda: call(0), torch)
    # the same n calls replayed from a HIP graph (the layer's kernels
    # without the host's launch cost), each replay on fresh copies
    fresh = torch.from_numpy(np.ascontiguousarray(h0)).cuda().repeat(n + 1, 1, 1)
    gs = torch.cuda.Stream()
    gs.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=gs):
        for i in range(n):
            call(i)
    torch.cuda.current_stream().wait_stream(gs)
    hs.copy_(fresh)
    g.replay()
    hs.copy_(fresh)
    torch.cuda.synchronize()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    us_graph = e0.elapsed_time(e1) * 1e3 / n
    res = {"workload": "one Qwen-style layer, hidden 256, 4/2 heads, d 64, FFN 768, 64-token prefill",
           "gpu_layer_us": round(us, 2), "gpu_layer_us_graph": round(us_graph, 2), "kernels_per_call": kernels,
           "weight_bytes": int(sum(a.size for a in (m.layers[0].wqkv, m.layers[0].wo, m.layers[0].wgu,
                                                    m.layers[0].wd)))}
    if with_cpu:
        import oracle as O
        omp_threads(1)
        t0 = time.perf_counter()
        want, _ = O.OracleModel(m, slots=1).layer(0, h0, [64], [0], [0])
        res["oracle_1thread_s"] = round(time.perf_counter() - t0, 4)
        omp_threads(host_threads())
        res["bit_exact_vs_oracle"] = bool(np.array_equal(got, want))
    return res


def c1_oracle_gops(S, seconds_per_shape: float = 1.5):
    """The oracle's int64 brute-force GEMM on the sweep's operands: GOPS
    (2 M N K / s) on a bounded row sample of each (K, N) shape, with all
    host threads and with one."""
    import numpy as np
    import oracle as O
    res = {}
    for Kd, Nd in S.GEMM_SWEEP_KN:
        g = S.make_gemm_operands(64, Nd, Kd, seed=7)
        out = {}
        for tag, nt in (("all_threads", host_threads()), ("one_thread", 1)):
            omp_threads(nt)
            rows, t = 1, 0.0
            while True:
                t0 = time.perf_counter()
                O.gemm(g["A"][:rows], g["W"])
                t = time.perf_counter() - t0
                if t > seconds_per_shape / 4 or rows >= 64:
                    break
                rows *= 2
            out[tag] = round(2 * rows * Nd * Kd / t / 1e9, 2)
            out[tag + "_rows"] = rows
        res[f"K{Kd}_N{Nd}"] = out
    omp_threads(host_threads())
    return res


def llama_case(D, S, torch, dec_steps: int, with_cpu: bool = False):
    """Llama-3.2-1B-shaped model with 16-bit limbed weights: 32 seeded
    2048-token prompts prefilled 4 per call, then batch-32 greedy decode
    from position 2048 (HIP-graph segments of 256 steps). Rows 0 and 31 are
    hashed step by step (outside the timed replays) and compared with the
    chain the oracle wrote (tests/golden/llama_c4.json)."""
    import numpy as np
    gold = json.loads((ROOT / "tests" / "golden" / "llama_c4.json").read_text())
    m = S.make_model(gold["model"], seed=gold["model_seed"])
    sh = m.shape
    B, P, SEG = gold["n_prompts"], gold["prompt_len"], 256
    dec_steps = min(dec_steps, gold["context"] - P)
    prompts = S.make_prompts(sh.vocab, B, P, P, gold["prompt_seed"])
    dm = D.DetintModel(m, n_slots=B)
    first = torch.empty((B, sh.vocab), dtype=torch.int32, device="cuda")
    toks, times = [], []
    for c in range(B // 4):
        sl = list(range(4 * c, 4 * c + 4))
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        toks.append(dm.prefill([prompts[i] for i in sl], [0] * 4, sl, first, 4 * c))
        torch.cuda.synchronize()
        times.append(time.perf_counter() - t0)
    t_pref = float(np.median(times[1:]))
    L, H, F, nq, nkv, d = sh.n_layers, sh.hidden, sh.ffn, sh.n_q, sh.n_kv, sh.head_dim
    lin_mac = L * H * ((nq + 2 * nkv) * d + nq * d + 2 * F) + L * F * H   # per token
    att_mac = L * nq * d * 3 * 4 * (P * (P + 1) // 2)                     # QK^T + 2 P.V limbs, causal
    ops = 2 * (2 * lin_mac * 4 * P + att_mac)                              # x2 limbs on the linears
    rows = [r["row"] for r in gold["rows"]]
    chains = {r: hashlib.sha256(b"detint-v0").digest() for r in rows}
    checks = {r: 0 for r in rows}
    bad = []

    def absorb(block, s0):
        rb = block[:, rows].cpu().numpy()
        for k, r in enumerate(rows):
            want = gold["rows"][k]["logits_chain"]
            for i in range(rb.shape[0]):
                chains[r] = hashlib.sha256(chains[r] + np.ascontiguousarray(rb[i, k], "<i4").tobytes()).digest()
                key = str(s0 + i)
                if key in want:
                    checks[r] += 1
                    if want[key] != chains[r].hex():
                        bad.append((r, s0 + i))

    absorb(first.view(1, B, sh.vocab), 0)
    tok = torch.cat(toks)
    hist = torch.empty((SEG, B, sh.vocab), dtype=torch.int32, device="cuda")
    done, t_dec, n_timed, pos = 0, 0.0, 0, P
    while done < dec_steps:
        n = min(SEG, dec_steps - done)
        step = dm.decode_step_fn(tok, [pos] * B, list(range(B)), hist, 0)
        step()                      # first replay of a fresh graph: untimed
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n - 1):
            step()
        e1.record()
        torch.cuda.synchronize()
        t_dec += e0.elapsed_time(e1) / 1e3
        n_timed += n - 1
        absorb(hist[:n], done + 1)
        done += n
        pos += n
    w_bytes = 2 * (L * H * ((nq + 2 * nkv) * d + nq * d + 2 * F + F) + sh.vocab * H)
    ctx_avg = P + 1 + (dec_steps - 1) / 2
    step_bytes = w_bytes + 2 * L * nkv * d * B * ctx_avg
    tps = B * n_timed / t_dec
    res = {
        "workload": "Llama-3.2-1B-shaped integer model, 16-bit limbed weights (random init, seed 0)",
        "prefill_4x2048_tok_s": round(4 * P / t_pref, 1),
        "prefill_ms_per_call": round(1e3 * t_pref, 2),
        "prefill_tops": round(ops / t_pref / 1e12, 1),
        "prefill_frac_i8_mfma": round(ops / t_pref / 1e12 / I8_PEAK_TOPS, 4),
        "decode_b32_tok_s": round(tps, 1),
        "decode_b32_ms_per_step": round(1e3 * t_dec / n_timed, 3),
        "decode_b32_hbm_frac": round(step_bytes * tps / B / 1e9 / HBM_PEAK_GBS, 4),
        "decode_ctx_range": [P + 1, P + dec_steps],
        "rows_vs_oracle_chain": {str(r): {"checkpoints": checks[r],
                                          "equal": not any(b[0] == r for b in bad)} for r in rows},
    }
    del dm, hist, first
    torch.cuda.empty_cache()
    if with_cpu:
        # the oracle on a bounded sample of the same work: the first 256-token
        # chunk of row 0's prompt, then 8 decode steps after it
        import oracle as O
        om = O.OracleModel(m, slots=1)
        t0 = time.perf_counter()
        _, nx = om.forward(prompts[0][:256], [256], [0], [0])
        t1 = time.perf_counter()
        t = [int(nx[0])]
        for k in range(8):
            _, nx = om.forward(np.array([t[-1]], np.int32), [1], [256 + k], [0])
            t.append(int(nx[0]))
        t2 = time.perf_counter()
        pre_tps, dec_tps = 256 / (t1 - t0), 8 / (t2 - t1)
        res["oracle"] = {"cores": host_threads(), "prefill_tok_s": round(pre_tps, 2),
                         "decode_tok_s": round(dec_tps, 3),
                         "seconds_per_4096_token_row_projected": round(P / pre_tps + (gold["context"] - P) / dec_tps, 1),
                         "seconds_per_row_recorded_with_golden": [r["oracle_seconds"] for r in gold["rows"]],
                         "sample": "256-token prefill chunk of row 0 and 8 decode steps after it; the "
                                   "projection ignores attention's growth with context"}
    return res


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


def barrier_probe(D, torch):
    """Cost of one device-wide barrier between 256 resident workgroups (the
    step a persistent decode kernel would take between phases), per mode of
    detint_probe_barrier, against one node of a HIP graph of tiny kernels
    (what each phase costs as its own launch)."""
    names = {0: "flags_release_acquire", 1: "counter_release_acquire",
             2: "two_level_flags_release_acquire", 3: "flags_relaxed_no_fences_lower_bound"}
    out = {}
    for mode, name in names.items():
        fails = D.detint_probe_barrier(mode, 20) | D.detint_probe_barrier(mode, 2020)
        t20 = timed(lambda: D.detint_probe_barrier(mode, 20, wait=False), 5, torch)
        t2020 = timed(lambda: D.detint_probe_barrier(mode, 2020, wait=False), 5, torch)
        out[name] = {"us_per_barrier": round((t2020 - t20) / 2000 * 1e6, 3), "failures": fails}
    x = torch.zeros(1, dtype=torch.int32, device="cuda")
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        x.add_(1)
        with torch.cuda.graph(g, stream=st):
            for _ in range(140):
                x.add_(1)
    torch.cuda.current_stream().wait_stream(st)
    out["graph_node_us"] = round(timed(g.replay, 20, torch) / 140 * 1e6, 3)
    out["workgroups"] = 256
    return out


def decode_only(D, S, torch, steps: int, warmup: int):
    """Batch-1 decode of the Qwen3-0.6B shape for counter runs: prefill, a
    few graph replays, then the copy calibration."""
    gold = json.loads((ROOT / "tests" / "golden" / "qwen3_b1.json").read_text())
    m = S.make_model("qwen3_0.6b", seed=gold["model_seed"])
    dm = D.DetintModel(m, n_slots=1)
    p0 = S.make_prompt(m.shape.vocab, PROMPT_LEN, gold["prompt_seed"])
    hist, _, ev = decode_run(D, dm, [p0], warmup, steps, torch)
    chain = D.logits_chain(hist.cpu().numpy()[:, 0])
    nb = copy_calibration(torch)
    print(json.dumps({"decode_steps": warmup + steps, "ms_per_step": 1e3 * ev / steps,
                      "chain_equal": chain == gold["logits_chain"][0][: len(chain)],
                      "copy_bytes": nb, "copy_launches": 5,
                      "kernel_source_sha256": kernel_source_sha(DECODE_SOURCES)}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=448)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--roofline-only", action="store_true")
    ap.add_argument("--decode-only", action="store_true")
    ap.add_argument("--no-llama", action="store_true")
    ap.add_argument("--llama-only", action="store_true")
    ap.add_argument("--llama-steps", type=int, default=2048)
    ap.add_argument("--barrier-probe", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        log("bench.py: runs on one GPU only (the integer forward pass is data-parallel by "
            "sequence: more GPUs would each hold the weights and their own KV-cache slots, "
            "with no collective in the step). Use --gpus 1.")
        sys.exit(2)
    if args.warmup + args.steps > 511 or args.steps < 1 or args.warmup < 0:
        log("bench.py: 1 <= steps and warmup + steps <= 511 (64-token prompt + 512 steps fit the cache)")
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
    if args.decode_only:
        decode_only(D, S, torch, args.steps, args.warmup)
        return
    if args.llama_only:
        print(json.dumps(llama_case(D, S, torch, args.llama_steps)), flush=True)
        return
    if args.barrier_probe:
        print(json.dumps({"grid_barrier_probe": barrier_probe(D, torch)}), flush=True)
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
    K = args.steps
    # untimed lead-in: at least the requested warmup, and enough steps that
    # the timed window sits in the middle of the 512-step decode's context
    W = max(args.warmup, min(511 - K, 256 - K // 2))

    # ---- decode, batch 1 (headline) ----
    log(f"decode b1: prefill {PROMPT_LEN}, {W} untimed + {K} timed graph replays")
    hist, wall1, ev1 = decode_run(D, dm, [p0], W, K, torch)
    h1 = hist.cpu().numpy()
    chain1 = D.logits_chain(h1[:, 0])
    exact_b1 = chain1 == gold["logits_chain"][0][: len(chain1)]
    gpu_tokens = h1[:, 0].argmax(-1)
    tps1 = K / wall1
    del hist, h1
    # kernels of one decode step (its graph captured again, not replayed)
    one = torch.empty((2, 1, sh.vocab), dtype=torch.int32, device="cuda")
    tok1 = torch.tensor([int(gpu_tokens[-1])], dtype=torch.int32, device="cuda")
    step_kernels = graph_kernel_count(dm.decode_step_fn(tok1, [PROMPT_LEN + W + K], [0], one, 0,
                                                        use_graph=False), torch)
    del one, tok1

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

    # ---- one Qwen-style layer (hidden 256) ----
    log("single layer")
    c0 = c0_case(D, S, torch, not args.no_cpu)

    # ---- the 25-shape int8 GEMM sweep ----
    log("GEMM sweep")
    gemm = gemm_sweep(D, S, torch)

    # ---- the fused final RMSNorm + lm_head GEMV on its own (the largest
    # single launch of the step: one launch streams the 155.6 MB table) ----
    log("final-head kernel")
    fn, nbytes = head_case(D, m, torch)
    for _ in range(3):
        fn()
    t_head = timed_cold(fn, 30, torch)
    head_gbs = nbytes / t_head / 1e9

    llama = None
    if not args.no_llama:
        del dm
        torch.cuda.empty_cache()
        log("Llama-3.2-1B-shaped model: prefill 4 x 2048 per call, batch-32 decode to 4096")
        llama = llama_case(D, S, torch, args.llama_steps, with_cpu=not args.no_cpu)

    log("integer sampling")
    sampling = sampling_case(D, torch, not args.no_cpu)
    log("grid barrier probe")
    barrier = barrier_probe(D, torch)
    cpu = None
    c1_cpu = None
    if not args.no_cpu:
        log("oracle on the host cores")
        cpu = cpu_baseline(m, p0, args.cpu_seconds, gpu_tokens)
        c1_cpu = c1_oracle_gops(S)

    # algorithmic bytes of one batch-1 decode step at the timed window's mean
    # context: every weight byte once (lm_head included), the K and V bytes
    # of every cached position, the per-channel mantissas and the logits
    weights = sum(L.wqkv.size + L.wo.size + L.wgu.size + L.wd.size for L in m.layers) + m.emb.size
    mant = 4 * (sum(L.wqkv_m.size + L.wo_m.size + L.wgu_m.size + L.wd_m.size for L in m.layers)
                + m.emb_m.size)
    ctx_avg = PROMPT_LEN + W + (K + 1) / 2
    step_bytes = weights + mant + 4 * sh.vocab + 2 * sh.n_layers * sh.n_kv * sh.head_dim * ctx_avg
    step_s = ev1 / K
    step_traffic = profile_value("decode_qwen3_step_hbm_traffic.txt", "hbm_bytes_per_step", DECODE_SOURCES)
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
        "vs_baseline_context": "the pages' 106.3 tok/s: trained Qwen3-0.6B, int8 decode at batch 1 on an "
                               "NVIDIA A100; another machine, context only",
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "Qwen3-0.6B-shaped integer model (random init, seed 0), greedy "
                               "decode at batch 1 after a 64-token prompt, one HIP-graph replay per token",
                   "batch": 1, "prompt_len": PROMPT_LEN, "decode_steps_timed": K,
                   "ctx_range": [PROMPT_LEN + 1 + W, PROMPT_LEN + W + K]},
        "bit_exact": {"decode_b1_vs_oracle_chain": bool(exact_b1),
                      "decode_b8_vs_oracle_chain": bool(exact_b8),
                      "b1_logits_hash": chain1[-1][:12]},
        "roofline": {"bound": "hbm",
                     "kernel": "the whole batch-1 decode step: one HIP-graph replay of %d kernels "
                               "(5 per layer, embedding, final head, greedy token)" % step_kernels,
                     "achieved": round(step_bytes / step_s / 1e9, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(step_bytes / step_s / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": step_traffic,
                     "algorithmic_bytes_per_step": int(step_bytes),
                     "avg_step_us": round(step_s * 1e6, 2)},
        "decode_b1_key_gains_tok_s": round(tps_gain, 2),
        "decode_b8_tok_s": round(tps8, 1),
        "prefill_tok_s": {"ragged_8_prompts_%d_tokens" % ntok: round(ntok / t_rag, 1),
                          "prompt_64": round(PROMPT_LEN / t_64, 1)},
        "single_layer_c0": c0,
        "llama3.2_1b_limbs": llama,
        "sampling": sampling,
        "gemm_sweep_req_i8": gemm,
        "gemm_best_frac_i8_mfma": round(max(big), 4),
        "gemm_sweep_oracle_gops": c1_cpu,
        "grid_barrier_probe": barrier,
        "final_head_kernel_roofline": {
            "bound": "hbm",
            "kernel": "fused final RMSNorm + tied lm_head GEMV, 1 row (fgemv<1,4,1,1,4>), cache-cold launches",
            "achieved": round(head_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(head_gbs / HBM_PEAK_GBS, 4),
            "traffic": profile_value("final_head_hbm_traffic.txt", "hbm_bytes_per_launch",
                                     ("decode.hip", "dev_int.h", "internal.h")),
            "algorithmic_bytes_per_launch": nbytes, "avg_launch_us": round(t_head * 1e6, 2)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
