"""CPU oracle for the integer-only forward pass (TEST INFRASTRUCTURE ONLY).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package; the product library never does. The arithmetic lives in
``detint_oracle.c`` (plain C, int64); this module only marshals numpy arrays
through ctypes and keeps a model's host arrays alive.
"""
from __future__ import annotations

import ctypes as C
import hashlib
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "detint_oracle.c"
# DETINT_ORACLE_LIB selects another build of the same source (the test that
# runs the oracle under UndefinedBehaviorSanitizer)
_LIB = Path(os.environ.get("DETINT_ORACLE_LIB", str(_HERE / "liboracle.so")))

# 16 bits of the cache layout etc. are fixed by the C code; these are the
# epilogue modes it understands.
RAW, REQ_I8, FIX, RES_ADD = 0, 1, 2, 3


def build(force: bool = True) -> Path:
    """Compile the oracle with gcc (plain -O2, OpenMP over rows/columns)."""
    if force or not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = _LIB.with_suffix(".so.tmp")
        subprocess.run(["gcc", "-O2", "-std=gnu11", "-fopenmp", "-fPIC", "-shared",
                        "-Wall", "-Wno-unused-function", "-o", str(tmp), str(_SRC), "-lm"],
                       check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not _LIB.exists():
            build(force=True)
        _lib = C.CDLL(str(_LIB))
        _declare(_lib)
    return _lib


i8p = np.ctypeslib.ndpointer(np.int8, flags="C_CONTIGUOUS")
i16p = np.ctypeslib.ndpointer(np.int16, flags="C_CONTIGUOUS")
i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
u32p = np.ctypeslib.ndpointer(np.uint32, flags="C_CONTIGUOUS")
i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
vp = C.c_void_p
i64 = C.c_int64
i32 = C.c_int32


class OrcLayer(C.Structure):
    _fields_ = [("wqkv", vp), ("wqkv16", vp), ("wqkv_m", vp),
                ("wo", vp), ("wo16", vp), ("wo_m", vp),
                ("wgu", vp), ("wgu16", vp), ("wgu_m", vp),
                ("wd", vp), ("wd16", vp), ("wd_m", vp),
                ("attn_norm", vp), ("ffn_norm", vp), ("q_norm", vp), ("k_norm", vp),
                ("kq_m", i32), ("kq_k", i32), ("vq_m", i32), ("vq_k", i32), ("k_gain", vp)]


class OrcModel(C.Structure):
    _fields_ = [("n_layers", i64), ("hidden", i64), ("n_q", i64), ("n_kv", i64),
                ("head_dim", i64), ("ffn", i64), ("vocab", i64), ("max_pos", i64),
                ("qk_norm", i32), ("wide", i32), ("w_k", i32), ("f_res", i32),
                ("f_n", i32), ("f_a", i32), ("f_l", i32), ("pad_", i32),
                ("emb", vp), ("emb16", vp), ("emb_m", vp), ("final_norm", vp),
                ("rope_cos", vp), ("rope_sin", vp), ("layers", C.POINTER(OrcLayer))]


_DUMP_FIELDS = [("x1", np.int8), ("x1_m", np.int32), ("x1_k", np.int32),
                ("qkv_acc", np.int64), ("q8", np.int8), ("eq", np.int32),
                ("attn", np.int32), ("o8", np.int8), ("o_m", np.int32), ("o_k", np.int32),
                ("h_mid", np.int32), ("x2", np.int8), ("x2_m", np.int32), ("x2_k", np.int32),
                ("gu", np.int32), ("a8", np.int8), ("a_m", np.int32), ("a_k", np.int32)]


class OrcDump(C.Structure):
    _fields_ = [(n, vp) for n, _ in _DUMP_FIELDS]


def _declare(L):
    L.orc_error.restype = C.c_int
    L.orc_error_msg.restype = C.c_char_p
    L.orc_rshift_round.restype = i64
    L.orc_rshift_round.argtypes = [i64, C.c_int]
    L.orc_div_round.restype = i64
    L.orc_div_round.argtypes = [i64, i64]
    L.orc_isqrt.restype = C.c_uint64
    L.orc_isqrt.argtypes = [C.c_uint64]
    L.orc_bitlen.restype = C.c_int
    L.orc_bitlen.argtypes = [C.c_uint64]
    L.orc_diexp.restype = i32
    L.orc_diexp.argtypes = [i64]
    L.orc_irms.argtypes = [i64, i64, C.POINTER(i32), C.POINTER(i32)]
    L.orc_dq.argtypes = [i64p, i64, i8p, C.POINTER(i32)]
    for f in ("orc_softmax_mult",):
        getattr(L, f).argtypes = [i32, i32, i64, i32, C.POINTER(i32), C.POINTER(i32)]
    L.orc_sigmoid_q15.restype = i32
    L.orc_sigmoid_q15.argtypes = [i64, i32, i32]
    L.orc_swiglu_mult.argtypes = [i32, C.POINTER(i32), C.POINTER(i32)]
    L.orc_v_dequant.argtypes = [i32, i32, C.POINTER(i32), C.POINTER(i32)]
    L.orc_rope_tables.argtypes = [i16p, i16p, i64, i64, i64]
    L.orc_gemm.argtypes = [vp, vp, vp, i64, i64, i64, i64p]
    L.orc_epilogue.argtypes = [i64p, i64, i64, i32p, i32p, i32p, i32, i32, i32, vp]
    L.orc_rmsnorm.argtypes = [i32p, i16p, i64, i64, i8p, i32p, i32p]
    L.orc_requant_rows.argtypes = [i32p, i64, i64, i8p, i32p]
    L.orc_requant_fixed.argtypes = [i32p, i64, i32, i32, i8p]
    L.orc_rope.argtypes = [i32p, i32p, i16p, i16p, i64, i64, i64, i64]
    L.orc_softmax.argtypes = [i32p, i32p, i32p, i64, i64, i32, i32, i16p]
    L.orc_swiglu.argtypes = [i32p, i64, i64, i32, i8p, i32p, i32p]
    L.orc_layer_forward.argtypes = [C.POINTER(OrcModel), i64, i32p, i64, i32p, i32p, i32p,
                                    i64, i8p, i8p, i64, C.POINTER(OrcDump)]
    L.orc_embed.argtypes = [C.POINTER(OrcModel), i32p, i64, i32p]
    L.orc_forward.argtypes = [C.POINTER(OrcModel), i32p, i64, i32p, i32p, i32p, i64,
                              i8p, i8p, i64, i32, i32p, vp]
    L.orc_argmax.argtypes = [i32p, i64, i64, i32p]
    L.orc_sample.argtypes = [i32p, i64, i64, i64, i32, i32, i32, u32p, i32p]
    u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
    L.orc_exact_weights.argtypes = [u16p, i64, i64, i32p, i32p]
    L.orc_gemm_exact.argtypes = [i8p, i32p, i64, i64, i64, i64p]
    L.orc_exact_epilogue.argtypes = [i64p, i64, i64, i32p, i32p, i32p, i32, i32, vp]
    L.orc_attention.argtypes = [i8p, i32p, i8p, i8p, i32p, i32p, i64, i64, i64, i64, i64, i64,
                                i32, i32, i32p]


class OracleError(RuntimeError):
    pass


def _check():
    L = lib()
    if L.orc_error():
        msg = L.orc_error_msg().decode()
        L.orc_clear_error()
        raise OracleError(msg)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


# --------------------------------------------------------------------------
# primitives

def rshift_round(x: int, s: int) -> int:
    v = lib().orc_rshift_round(int(x), int(s)); _check(); return v


def div_round(a: int, b: int) -> int:
    v = lib().orc_div_round(int(a), int(b)); _check(); return v


def isqrt(n: int) -> int:
    return lib().orc_isqrt(int(n))


def bitlen(x: int) -> int:
    return lib().orc_bitlen(int(x))


def diexp(u: int) -> int:
    v = lib().orc_diexp(int(u)); _check(); return v


def irms(S: int, n: int) -> tuple[int, int]:
    m, sh = i32(), i32()
    lib().orc_irms(int(S), int(n), C.byref(m), C.byref(sh)); _check()
    return m.value, sh.value


def dq(y) -> tuple[np.ndarray, int]:
    y = _c(y, np.int64)
    q = np.zeros(y.size, np.int8)
    e = i32()
    lib().orc_dq(y, y.size, q, C.byref(e)); _check()
    return q, e.value


def softmax_mult(kq_m: int, kq_k: int, d: int, f_n: int) -> tuple[int, int]:
    M, K = i32(), i32()
    lib().orc_softmax_mult(kq_m, kq_k, d, f_n, C.byref(M), C.byref(K))
    return M.value, K.value


def swiglu_mult(f_a: int) -> tuple[int, int]:
    M, K = i32(), i32()
    lib().orc_swiglu_mult(f_a, C.byref(M), C.byref(K))
    return M.value, K.value


def sigmoid_q15(g: int, Mg: int, Kg: int) -> int:
    v = lib().orc_sigmoid_q15(int(g), int(Mg), int(Kg)); _check(); return v


def v_dequant(vq_m: int, vq_k: int) -> tuple[int, int]:
    M, K = i32(), i32()
    lib().orc_v_dequant(vq_m, vq_k, C.byref(M), C.byref(K)); _check()
    return M.value, K.value


def rope_tables(P: int, d: int, base: int) -> tuple[np.ndarray, np.ndarray]:
    c = np.zeros((P, d // 2), np.int16)
    s = np.zeros((P, d // 2), np.int16)
    lib().orc_rope_tables(c, s, P, d, int(base))
    return c, s


# --------------------------------------------------------------------------
# ops

def gemm(A, W) -> np.ndarray:
    """Exact int64 accumulators of A[M,K] (int8) x W[N,K]^T (int8 or int16)."""
    A = _c(A, np.int8)
    M, K = A.shape
    N = W.shape[0]
    acc = np.zeros((M, N), np.int64)
    if W.dtype == np.int16:
        W = _c(W, np.int16)
        lib().orc_gemm(A.ctypes.data, None, W.ctypes.data, M, N, K, acc)
    else:
        W = _c(W, np.int8)
        lib().orc_gemm(A.ctypes.data, W.ctypes.data, None, M, N, K, acc)
    _check()
    return acc


def epilogue(acc, row_m, row_k, col_m, col_k: int, frac: int, mode: int, out=None):
    acc = _c(acc, np.int64)
    M, N = acc.shape
    if mode == REQ_I8:
        out = np.zeros((M, N), np.int8)
    elif mode in (RAW, FIX):
        out = np.zeros((M, N), np.int32)
    else:
        out = _c(out, np.int32).copy()
    lib().orc_epilogue(acc, M, N, _c(row_m, np.int32), _c(row_k, np.int32), _c(col_m, np.int32),
                       int(col_k), int(frac), int(mode), out.ctypes.data)
    _check()
    return out


def gemm_i8(A, W, row_m=None, row_k=None, col_m=None, col_k=0, frac=0, mode=RAW, out=None):
    acc = gemm(A, W)
    M, N = acc.shape
    if mode == RAW:
        return epilogue(acc, np.zeros(M), np.zeros(M), np.zeros(N), 0, 0, RAW)
    return epilogue(acc, row_m, row_k, col_m, col_k, frac, mode, out)


def exact_weights(Wbits):
    """bf16 bit patterns [N, K] (uint16) -> (W_int int32 [N, K], row_exp int32
    [N]) with w = W_int * 2^row_exp exactly (orc_exact_weights)."""
    Wbits = _c(Wbits, np.uint16)
    N, K = Wbits.shape
    W_int = np.zeros((N, K), np.int32)
    row_exp = np.zeros(N, np.int32)
    lib().orc_exact_weights(Wbits, N, K, W_int, row_exp); _check()
    return W_int, row_exp


def gemm_exact(A, W_int) -> np.ndarray:
    A = _c(A, np.int8)
    W_int = _c(W_int, np.int32)
    M, K = A.shape
    N = W_int.shape[0]
    acc = np.zeros((M, N), np.int64)
    lib().orc_gemm_exact(A, W_int, M, N, K, acc); _check()
    return acc


def exact_epilogue(acc, row_m, row_k, row_exp, frac: int, mode: int):
    acc = _c(acc, np.int64)
    M, N = acc.shape
    out = np.zeros((M, N), {RAW: np.int64, REQ_I8: np.int8, FIX: np.int32}[mode])
    lib().orc_exact_epilogue(acc, M, N, _c(row_m, np.int32), _c(row_k, np.int32),
                             _c(row_exp, np.int32), int(frac), int(mode), out.ctypes.data)
    _check()
    return out


def rmsnorm(h, g):
    h = _c(h, np.int32)
    R_, n = h.shape
    x8 = np.zeros((R_, n), np.int8)
    m = np.zeros(R_, np.int32)
    k = np.zeros(R_, np.int32)
    lib().orc_rmsnorm(h, _c(g, np.int16), R_, n, x8, m, k); _check()
    return x8, m, k


def requant_rows(y):
    y = _c(y, np.int32)
    R_, n = y.shape
    q = np.zeros((R_, n), np.int8)
    e = np.zeros(R_, np.int32)
    lib().orc_requant_rows(y, R_, n, q, e); _check()
    return q, e


def requant_fixed(y, m: int, k: int):
    """clamp8(R(y * m, k)) elementwise (the K/V cache quantisation)."""
    y = _c(y, np.int32)
    q = np.zeros(y.shape, np.int8)
    lib().orc_requant_fixed(y.ravel(), y.size, int(m), int(k), q.ravel()); _check()
    return q


def rope(x, pos, cos_t, sin_t):
    """x: [R, heads, d] int32 (copied), pos: [R]."""
    x = _c(x, np.int32).copy()
    R_, heads, d = x.shape
    lib().orc_rope(x, _c(pos, np.int32), _c(cos_t, np.int16), _c(sin_t, np.int16),
                   R_, heads, d, cos_t.shape[0]); _check()
    return x


def softmax(s, valid, shift, M: int, K: int):
    s = _c(s, np.int32)
    R_, Cc = s.shape
    P = np.zeros((R_, Cc), np.int16)
    lib().orc_softmax(s, _c(valid, np.int32), _c(shift, np.int32), R_, Cc, int(M), int(K), P)
    _check()
    return P


def swiglu(gu, f_a: int):
    """gu: [R, 2n] int32, gate in [:, :n], up in [:, n:]."""
    gu = _c(gu, np.int32)
    R_, n2 = gu.shape
    n = n2 // 2
    a8 = np.zeros((R_, n), np.int8)
    m = np.zeros(R_, np.int32)
    k = np.zeros(R_, np.int32)
    lib().orc_swiglu(gu, R_, n, int(f_a), a8, m, k); _check()
    return a8, m, k


def attention(q8, eq, kc, vc, pos, slot, M: int, K: int):
    """q8 [R, nq, d], eq [R, nq]; kc/vc one layer [slots, nkv, max_pos, d]."""
    q8 = _c(q8, np.int8)
    R_, nq, d = q8.shape
    slots, nkv, max_pos, _ = kc.shape
    out = np.zeros((R_, nq, d), np.int32)
    lib().orc_attention(q8, _c(eq, np.int32), _c(kc, np.int8), _c(vc, np.int8), _c(pos, np.int32),
                        _c(slot, np.int32), R_, nq, nkv, d, slots, max_pos, int(M), int(K), out)
    _check()
    return out


def argmax(logits):
    logits = _c(logits, np.int32)
    R_, V = logits.shape
    out = np.zeros(R_, np.int32)
    lib().orc_argmax(logits, R_, V, out)
    return out


def sample(logits, top_k: int, t_m: int, t_k: int, draws, top_p: int = 65536):
    """Integer temperature / top-k / top-p sampling of each row with the
    caller's uniform 32-bit draws; top_p is p in units of 2^-16 (65536: off).
    orc_sample states the reading."""
    logits = _c(logits, np.int32)
    R_, V = logits.shape
    draws = _c(draws, np.uint32)
    assert draws.shape == (R_,)
    out = np.zeros(R_, np.int32)
    lib().orc_sample(logits, R_, V, int(top_k), int(top_p), int(t_m), int(t_k), draws, out)
    _check()
    return out


# --------------------------------------------------------------------------
# model driver


class OracleModel:
    """Holds a synthetic model's host arrays in the oracle's struct form plus
    the oracle's own KV cache ([layer][slot][kv head][position][d] int8)."""

    def __init__(self, model, slots: int = 1):
        self.model = model
        sh = model.shape
        self.shape = sh
        self.slots = slots
        self._keep = []
        cos_t, sin_t = rope_tables(sh.max_pos, sh.head_dim, sh.rope_base)
        self.rope_cos, self.rope_sin = cos_t, sin_t
        layers = (OrcLayer * sh.n_layers)()
        for i, Lw in enumerate(model.layers):
            st = layers[i]
            for name in ("wqkv", "wo", "wgu", "wd"):
                w = self._ptr(getattr(Lw, name))
                if sh.wide:
                    setattr(st, name + "16", w)
                else:
                    setattr(st, name, w)
                setattr(st, name + "_m", self._ptr(getattr(Lw, name + "_m")))
            st.attn_norm = self._ptr(Lw.attn_norm)
            st.ffn_norm = self._ptr(Lw.ffn_norm)
            st.q_norm = self._ptr(Lw.q_norm) if Lw.q_norm is not None else None
            st.k_norm = self._ptr(Lw.k_norm) if Lw.k_norm is not None else None
            st.kq_m, st.kq_k, st.vq_m, st.vq_k = Lw.kq_m, Lw.kq_k, Lw.vq_m, Lw.vq_k
            kg = getattr(Lw, "k_gain", None)
            st.k_gain = self._ptr(np.ascontiguousarray(kg, np.int8)) if kg is not None else None
        self._layers = layers
        md = OrcModel(n_layers=sh.n_layers, hidden=sh.hidden, n_q=sh.n_q, n_kv=sh.n_kv,
                      head_dim=sh.head_dim, ffn=sh.ffn, vocab=sh.vocab, max_pos=sh.max_pos,
                      qk_norm=int(sh.qk_norm), wide=int(sh.wide), w_k=sh.w_k, f_res=sh.f_res,
                      f_n=sh.f_n, f_a=sh.f_a, f_l=sh.f_l)
        if model.emb is not None:
            if sh.wide:
                md.emb16 = self._ptr(model.emb)
            else:
                md.emb = self._ptr(model.emb)
            md.emb_m = self._ptr(model.emb_m)
            md.final_norm = self._ptr(model.final_norm)
        md.rope_cos = self._ptr(cos_t)
        md.rope_sin = self._ptr(sin_t)
        md.layers = C.cast(layers, C.POINTER(OrcLayer))
        self.md = md
        self.reset_cache()

    def _ptr(self, a):
        a = np.ascontiguousarray(a)
        self._keep.append(a)
        return a.ctypes.data

    def reset_cache(self):
        sh = self.shape
        shp = (sh.n_layers, self.slots, sh.n_kv, sh.max_pos, sh.head_dim)
        self.kc = np.zeros(shp, np.int8)
        self.vc = np.zeros(shp, np.int8)

    @staticmethod
    def _seqs(lens, starts, slots):
        cu = np.zeros(len(lens) + 1, np.int32)
        cu[1:] = np.cumsum(lens)
        return cu, _c(starts, np.int32), _c(slots, np.int32)

    def layer(self, l: int, h, lens, starts, slots, dump: bool = False):
        """Run layer l in place on h [R, H]; returns (h, intermediates)."""
        sh = self.shape
        h = _c(h, np.int32).copy()
        R_ = h.shape[0]
        cu, st, sl = self._seqs(lens, starts, slots)
        d_arrays = {}
        dp = None
        if dump:
            H, F, nq, d = sh.hidden, sh.ffn, sh.n_q, sh.head_dim
            shapes = dict(x1=(R_, H), x1_m=(R_,), x1_k=(R_,), qkv_acc=(R_, sh.qkv_out),
                          q8=(R_, nq, d), eq=(R_, nq), attn=(R_, nq * d), o8=(R_, nq * d),
                          o_m=(R_,), o_k=(R_,), h_mid=(R_, H), x2=(R_, H), x2_m=(R_,),
                          x2_k=(R_,), gu=(R_, 2 * F), a8=(R_, F), a_m=(R_,), a_k=(R_,))
            dp = OrcDump()
            for name, dt in _DUMP_FIELDS:
                arr = np.zeros(shapes[name], dt)
                d_arrays[name] = arr
                setattr(dp, name, arr.ctypes.data)
        lib().orc_layer_forward(C.byref(self.md), l, h, R_, cu, st, sl, len(lens),
                                self.kc, self.vc, self.slots, C.byref(dp) if dp else None)
        _check()
        return h, d_arrays

    def embed(self, ids):
        """Residual rows h0 [R, H] of the token ids (orc_embed)."""
        ids = _c(ids, np.int32)
        h = np.zeros((ids.size, self.shape.hidden), np.int32)
        lib().orc_embed(C.byref(self.md), ids, ids.size, h)
        _check()
        return h

    def forward(self, ids, lens, starts, slots, all_rows: bool = False):
        """ids packed over sequences -> (logits [S or R, V] int32, next tokens)."""
        sh = self.shape
        ids = _c(ids, np.int32)
        cu, st, sl = self._seqs(lens, starts, slots)
        nout = ids.size if all_rows else len(lens)
        logits = np.zeros((nout, sh.vocab), np.int32)
        nxt = np.zeros(nout, np.int32)
        lib().orc_forward(C.byref(self.md), ids, ids.size, cu, st, sl, len(lens),
                          self.kc, self.vc, self.slots, int(all_rows), logits, nxt.ctypes.data)
        _check()
        return logits, nxt

    def generate(self, prompts, n_new: int, on_step=None):
        """Greedy generation for a batch of prompts (slot i = prompt i): one
        prefill call over all prompts, then n_new - 1 one-token steps. Returns
        (tokens [B, n_new], logits chain objects). on_step(step, logits [B,V])
        is called with every step's logits (step 0 = the prefill)."""
        B = len(prompts)
        assert B <= self.slots
        lens = [len(p) for p in prompts]
        ids = np.concatenate([np.asarray(p, np.int32) for p in prompts])
        logits, nxt = self.forward(ids, lens, [0] * B, list(range(B)))
        toks = np.zeros((B, n_new), np.int32)
        toks[:, 0] = nxt
        if on_step:
            on_step(0, logits)
        pos = np.array(lens, np.int32)
        for s in range(1, n_new):
            logits, nxt = self.forward(toks[:, s - 1], [1] * B, pos, list(range(B)))
            pos += 1
            toks[:, s] = nxt
            if on_step:
                on_step(s, logits)
        return toks


def chain_init() -> bytes:
    """Start of the chained per-step logits hash: SHA-256 of a fixed tag."""
    return hashlib.sha256(b"detint-v0").digest()


def chain_step(hprev: bytes, row) -> bytes:
    """H_{s+1} = SHA-256(H_s || int32 little-endian bytes of the row)."""
    return hashlib.sha256(hprev + np.ascontiguousarray(row, dtype="<i4").tobytes()).digest()
