"""Real-valued (float64) shadow of the integer model, for tests only.

It reads the same integer weights as real numbers (w * m * 2^-k, gains
g * 2^-12) and runs the textbook Qwen3/Llama decoder in float64: RMSNorm,
projections, per-head RMSNorm on q/k (Qwen3), rotate-half RoPE with exact
cos/sin, causal softmax(q k^T / sqrt(d)), SwiGLU. It shares nothing with the
oracle; it checks that the integer scales are wired to the real quantities
they claim to represent (not bit-parity).
"""
import math

import numpy as np


def wreal(w, m, k):
    return w.astype(np.float64) * m.astype(np.float64)[:, None] * 2.0 ** -k


def rmsnorm(x, g):
    rms = np.sqrt((x * x).mean(axis=-1, keepdims=True))
    return x / rms * (g.astype(np.float64) / 4096.0)


def rope(x, pos, base):
    """x [..., T, d], pos [T]; pairs (i, i + d/2)."""
    d = x.shape[-1]
    half = d // 2
    theta = base ** (-np.arange(half, dtype=np.float64) * 2 / d)
    ang = pos[:, None].astype(np.float64) * theta[None, :]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def silu(x):
    return x / (1.0 + np.exp(-x))


def layer(shape, L, h, pos):
    """One decoder layer on one sequence: h [T, H] real, pos [T]."""
    H, nq, nkv, d, F = shape.hidden, shape.n_q, shape.n_kv, shape.head_dim, shape.ffn
    wk = shape.w_k
    x = rmsnorm(h, L.attn_norm)
    qkv = x @ wreal(L.wqkv, L.wqkv_m, wk).T
    T = h.shape[0]
    q = qkv[:, : nq * d].reshape(T, nq, d).transpose(1, 0, 2)
    k = qkv[:, nq * d:(nq + nkv) * d].reshape(T, nkv, d).transpose(1, 0, 2)
    v = qkv[:, (nq + nkv) * d:].reshape(T, nkv, d).transpose(1, 0, 2)
    if shape.qk_norm:
        q = rmsnorm(q, L.q_norm)
        k = rmsnorm(k, L.k_norm)
    q = rope(q, pos, shape.rope_base)
    k = rope(k, pos, shape.rope_base)
    out = np.zeros((nq, T, d))
    mask = pos[None, :] <= pos[:, None]
    for hh in range(nq):
        kv = hh * nkv // nq
        s = q[hh] @ k[kv].T / math.sqrt(d)
        s = np.where(mask, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[hh] = p @ v[kv]
    o = out.transpose(1, 0, 2).reshape(T, nq * d)
    h = h + o @ wreal(L.wo, L.wo_m, wk).T
    x2 = rmsnorm(h, L.ffn_norm)
    gu = x2 @ wreal(L.wgu, L.wgu_m, wk).T
    a = silu(gu[:, :F]) * gu[:, F:]
    return h + a @ wreal(L.wd, L.wd_m, wk).T


def forward_logits(model, ids):
    """Float logits for every position of one sequence."""
    sh = model.shape
    E = wreal(model.emb, model.emb_m, sh.w_k)
    h = E[np.asarray(ids)]
    pos = np.arange(len(ids))
    for L in model.layers:
        h = layer(sh, L, h, pos)
    x = rmsnorm(h, model.final_norm)
    return x @ E.T
