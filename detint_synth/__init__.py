"""Seeded synthetic inputs: model artifacts, prompts, GEMM operands.

This module is the one piece of Python shared by the CPU oracle and the HIP
path. It draws random numbers and lays them out; it performs none of the
integer forward pass. Everything it produces stands in for what the pages
call the offline "prepare" stage (float -> int artifact) and for their
prompts/datasets, none of which exist here:

* linear weights: int8 = clip(rint(N(0, 40)), -127, 127); 16-bit variant
  clip(rint(N(0, 40*256)), -32767, 32767);
* every weight tensor carries a per-output-channel dyadic scale m / 2^k with
  m uniform in [2^14, 2^15) and one shift k per tensor;
* RMSNorm / q-norm / k-norm gains: int16 uniform in [2^12, 2^13], read as
  gain * 2^-12;
* static KV-cache scales: the pages calibrate them offline on data; with
  random weights we pick them from the closed-form activation RMS the
  weight statistics imply (a stand-in for that calibration pass);
* prompts: token ids uniform in [0, vocab).

Float appears here only to draw and calibrate the artifact, never in the
forward pass (DetLLM README, "Layout": prepare.py is the offline float stage;
DetLLM blog, "DetLLM": K/V use offline-calibrated fixed scales).
"""
from __future__ import annotations

import hashlib
import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

__all__ = [
    "ModelShape", "SHAPES", "make_model", "make_prompt", "make_prompts",
    "make_residual", "make_gemm_operands", "GEMM_SWEEP_M", "GEMM_SWEEP_KN",
    "make_bf16_weights", "bf16_to_float64",
    "model_digest",
]

# --------------------------------------------------------------------------
# shapes


@dataclass(frozen=True)
class ModelShape:
    name: str
    n_layers: int
    hidden: int
    n_q: int
    n_kv: int
    head_dim: int
    ffn: int
    vocab: int
    qk_norm: bool          # Qwen3-style per-head RMSNorm on q and k
    wide: bool             # 16-bit fixed-point linear weights (hi/lo limbs)
    rope_base: int         # RoPE base (integer-valued)
    max_pos: int           # rows of the RoPE tables / KV-cache capacity
    w_k: int               # per-tensor shift k of every weight scale m/2^k
    f_res: int = 8         # fractional bits of the int32 residual stream
    f_n: int = 12          # fractional bits of normalised q/k and of v
    f_a: int = 12          # fractional bits of SwiGLU gate/up
    f_l: int = 16          # fractional bits of the int32 logits

    @property
    def qkv_out(self) -> int:
        return (self.n_q + 2 * self.n_kv) * self.head_dim


SHAPES = {
    # one Qwen3-style layer: hidden 256, 4 q / 2 kv heads, head_dim 64, FFN 768
    "layer256": ModelShape("layer256", 1, 256, 4, 2, 64, 768, 0, True, False,
                           1_000_000, 256, 22),
    # small whole models for quick end-to-end parity (same arithmetic)
    "tiny": ModelShape("tiny", 2, 256, 4, 2, 64, 768, 1000, True, False,
                       1_000_000, 512, 22),
    "tiny_wide": ModelShape("tiny_wide", 2, 256, 4, 2, 64, 768, 1000, False,
                            True, 500_000, 512, 30),
    # Qwen3-0.6B shape: 28 layers, hidden 1024, 16/8 heads, d 128, FFN 3072
    "qwen3_0.6b": ModelShape("qwen3_0.6b", 28, 1024, 16, 8, 128, 3072,
                             151936, True, False, 1_000_000, 1024, 22),
    # Llama-3.2-1B shape: 16 layers, hidden 2048, 32/8 heads, d 64, FFN 8192
    "llama3.2_1b": ModelShape("llama3.2_1b", 16, 2048, 32, 8, 64, 8192,
                              128256, False, True, 500_000, 4096, 30),
}

# the standalone GEMM sweep: rows M x (K, N) of the five projection shapes
GEMM_SWEEP_M = (1, 8, 64, 512, 2048)
GEMM_SWEEP_KN = ((1024, 4096), (2048, 1024), (1024, 6144), (3072, 1024),
                 (1024, 151936))

# --------------------------------------------------------------------------
# random draws

_CHUNK = 1 << 22


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def _normal_clip(key: tuple, n: int, sigma: float, lim: int, dtype) -> np.ndarray:
    """clip(rint(N(0, sigma)), -lim, lim), drawn in fixed chunks so the result
    does not depend on thread count."""
    def one(i):
        cnt = min(_CHUNK, n - i * _CHUNK)
        x = _rng(*key, i).standard_normal(cnt, dtype=np.float32)
        x *= np.float32(sigma)
        np.rint(x, out=x)
        np.clip(x, -lim, lim, out=x)
        return x.astype(dtype)
    nchunks = (n + _CHUNK - 1) // _CHUNK
    if nchunks <= 1:
        return one(0) if n else np.zeros(0, dtype)
    with ThreadPoolExecutor(8) as ex:
        parts = list(ex.map(one, range(nchunks)))
    return np.concatenate(parts)


def _weight(seed: int, tid: int, rows: int, cols: int, wide: bool) -> np.ndarray:
    if wide:
        w = _normal_clip((seed, tid, 16), rows * cols, 40.0 * 256, 32767, np.int16)
    else:
        w = _normal_clip((seed, tid, 8), rows * cols, 40.0, 127, np.int8)
    return w.reshape(rows, cols)


def _mant(seed: int, tid: int, n: int) -> np.ndarray:
    return _rng(seed, tid, 77).integers(1 << 14, 1 << 15, n, dtype=np.int64).astype(np.int32)


def _gain(seed: int, tid: int, n: int) -> np.ndarray:
    return _rng(seed, tid, 55).integers(1 << 12, (1 << 13) + 1, n, dtype=np.int64).astype(np.int16)


def _dyadic_of(scale: float) -> tuple[int, int]:
    """Offline float scale -> (m, k) with m in [2^14, 2^15) and m/2^k ~ scale."""
    f, ex = math.frexp(scale)
    m = int(math.floor(f * (1 << 15) + 0.5))
    k = 15 - ex
    if m == 1 << 15:
        m, k = 1 << 14, k - 1
    return m, k


def _kv_scales(shape: ModelShape) -> dict:
    """Closed-form stand-in for the offline KV calibration pass.

    Normalised activations entering a projection have RMS ~ RMS(gain) ~ 1.53;
    a weight's real value is w * m * 2^-k with E[m] = 1.5 * 2^14. The
    projected value then has RMS sqrt(H) * 1.53 * sigma_w * 1.5 * 2^14 * 2^-k.
    The cache stores 127 at ~5 RMS.
    """
    g_rms = math.sqrt((4096 ** 2 + 4096 * 8192 + 8192 ** 2) / 3) / 4096
    sig_w = 40.0 * (256 if shape.wide else 1)
    proj_rms = math.sqrt(shape.hidden) * g_rms * sig_w * 1.5 * 2 ** 14 * 2.0 ** -shape.w_k
    k_rms = g_rms if shape.qk_norm else proj_rms
    kq_m, kq_k = _dyadic_of(127.0 / (5.0 * k_rms * 2 ** shape.f_n))
    vq_m, vq_k = _dyadic_of(127.0 / (5.0 * proj_rms * 2 ** shape.f_n))
    return dict(kq_m=kq_m, kq_k=kq_k, vq_m=vq_m, vq_k=vq_k)


@dataclass
class Layer:
    attn_norm: np.ndarray
    wqkv: np.ndarray
    wqkv_m: np.ndarray
    wo: np.ndarray
    wo_m: np.ndarray
    ffn_norm: np.ndarray
    wgu: np.ndarray          # rows [0, F) gate, [F, 2F) up
    wgu_m: np.ndarray
    wd: np.ndarray
    wd_m: np.ndarray
    q_norm: np.ndarray | None
    k_norm: np.ndarray | None
    kq_m: int
    kq_k: int
    vq_m: int
    vq_k: int
    k_gain: np.ndarray | None = None  # [n_kv, d] int8 per-channel key gains, or None


@dataclass
class Model:
    shape: ModelShape
    seed: int
    layers: list
    emb: np.ndarray | None = None       # [V, H] int8 (int16 when wide); tied lm_head
    emb_m: np.ndarray | None = None     # [V] per-row mantissa
    final_norm: np.ndarray | None = None
    meta: dict = field(default_factory=dict)


def make_model(shape: ModelShape | str, seed: int = 0, with_vocab: bool = True) -> Model:
    """Seeded random-init integer model of the given shape."""
    if isinstance(shape, str):
        shape = SHAPES[shape]
    H, d, F = shape.hidden, shape.head_dim, shape.ffn
    layers = []
    kv = _kv_scales(shape)
    for li in range(shape.n_layers):
        t = 100 * (li + 1)
        layers.append(Layer(
            attn_norm=_gain(seed, t + 1, H),
            wqkv=_weight(seed, t + 2, shape.qkv_out, H, shape.wide),
            wqkv_m=_mant(seed, t + 2, shape.qkv_out),
            wo=_weight(seed, t + 3, H, shape.n_q * d, shape.wide),
            wo_m=_mant(seed, t + 3, H),
            ffn_norm=_gain(seed, t + 4, H),
            wgu=_weight(seed, t + 5, 2 * F, H, shape.wide),
            wgu_m=_mant(seed, t + 5, 2 * F),
            wd=_weight(seed, t + 6, H, F, shape.wide),
            wd_m=_mant(seed, t + 6, H),
            q_norm=_gain(seed, t + 7, d) if shape.qk_norm else None,
            k_norm=_gain(seed, t + 8, d) if shape.qk_norm else None,
            **kv,
        ))
    m = Model(shape=shape, seed=seed, layers=layers)
    if with_vocab and shape.vocab:
        m.emb = _weight(seed, 1, shape.vocab, H, shape.wide)
        m.emb_m = _mant(seed, 1, shape.vocab)
        m.final_norm = _gain(seed, 2, H)
    return m


def model_digest(m: Model) -> str:
    """sha256 over every tensor and constant, in a fixed order."""
    h = hashlib.sha256()
    h.update(repr(m.shape).encode())
    for arr in ([m.emb, m.emb_m, m.final_norm] if m.emb is not None else []):
        h.update(np.ascontiguousarray(arr).tobytes())
    for L in m.layers:
        for name in ("attn_norm", "wqkv", "wqkv_m", "wo", "wo_m", "ffn_norm",
                     "wgu", "wgu_m", "wd", "wd_m", "q_norm", "k_norm"):
            a = getattr(L, name)
            if a is not None:
                h.update(np.ascontiguousarray(a).tobytes())
        h.update(np.array([L.kq_m, L.kq_k, L.vq_m, L.vq_k], np.int64).tobytes())
        if L.k_gain is not None:
            h.update(np.ascontiguousarray(L.k_gain).tobytes())
    return h.hexdigest()


def with_key_gains(m: Model, seed: int, gmax: int = 3) -> Model:
    """The same model with seeded per-channel key gains in [0, gmax] on every
    layer (random stand-ins for calibrated ones)."""
    rng = np.random.default_rng(seed)
    sh = m.shape
    for L in m.layers:
        L.k_gain = rng.integers(0, gmax + 1, (sh.n_kv, sh.head_dim)).astype(np.int8)
    return m


# --------------------------------------------------------------------------
# activations / prompts / GEMM operands


def make_prompt(vocab: int, length: int, seed: int) -> np.ndarray:
    return _rng(seed, 9001).integers(0, vocab, length, dtype=np.int64).astype(np.int32)


def make_prompts(vocab: int, n: int, lo: int, hi: int, seed: int) -> list:
    """n prompts with lengths uniform in {lo..hi} (inclusive)."""
    r = _rng(seed, 9002)
    lens = r.integers(lo, hi + 1, n)
    return [make_prompt(vocab, int(L), seed * 1000 + 17 + i) for i, L in enumerate(lens)]


def make_residual(rows: int, hidden: int, seed: int) -> np.ndarray:
    """int32 residual rows uniform in [-2^15, 2^15)."""
    return _rng(seed, 9003).integers(-(1 << 15), 1 << 15, (rows, hidden),
                                     dtype=np.int64).astype(np.int32)


def make_bf16_weights(N: int, K: int, seed: int, sigma: float = 0.02,
                      max_span: int = 23) -> np.ndarray:
    """bf16 bit patterns [N, K] (uint16) of N(0, sigma) draws, rounded to the
    nearest bf16 (ties to even) with integer operations on the float32 bit
    patterns. Entries more than max_span binary orders below their row's
    largest exponent are set to +0: the stand-in for trained bf16 weights
    keeps every row within the exponent span that the exact-mode integers
    hold (the arithmetic itself is exact for whatever bf16 values it gets)."""
    x = _rng(seed, N, K, 16).standard_normal((N, K), dtype=np.float32) * np.float32(sigma)
    b = x.view(np.uint32).astype(np.uint64)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
    E = ((b >> 7) & 255).astype(np.int32)
    emax = E.max(axis=1, keepdims=True)
    b[E < emax - max_span] = 0
    return b


def bf16_to_float64(bits: np.ndarray) -> np.ndarray:
    """Exact real values of bf16 bit patterns (a bf16 is the top half of a
    float32)."""
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def make_gemm_operands(M: int, N: int, K: int, seed: int) -> dict:
    """int8 operands uniform in [-128, 127] with per-row (activation) and
    per-column (weight) dyadic scales: row m ~ U[2^14, 2^15), k = 20;
    column m ~ U[2^14, 2^15), k = 22."""
    r = _rng(seed, M, N, K)
    A = r.integers(-128, 128, (M, K), dtype=np.int64).astype(np.int8)
    W = r.integers(-128, 128, (N, K), dtype=np.int64).astype(np.int8)
    row_m = r.integers(1 << 14, 1 << 15, M, dtype=np.int64).astype(np.int32)
    col_m = r.integers(1 << 14, 1 << 15, N, dtype=np.int64).astype(np.int32)
    return dict(A=A, W=W, row_m=row_m, row_k=np.full(M, 20, np.int32),
                col_m=col_m, col_k=22)
