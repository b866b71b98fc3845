"""Python binding of libdetint (integer-only transformer forward pass, gfx950).

Marshalling only: every function forwards torch tensors' device pointers and
the current HIP stream to the C ABI in include/detint.h under the same name.
There is no fallback path: without the built libdetint.so (see build.py)
every call raises.
"""
from __future__ import annotations

import ctypes as C
import hashlib
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
LIB_PATH = _HERE / "libdetint.so"

DETINT_OK, DETINT_EINVAL, DETINT_EUNSUPPORTED, DETINT_EHIP, DETINT_EBOUND = 0, 1, 2, 3, 4
BOUND_RESIDUAL, BOUND_INT32, BOUND_NORM, BOUND_SWIGLU, BOUND_ID, BOUND_WEIGHT, BOUND_PAGE = (
    1, 2, 4, 8, 16, 32, 64)
RAW, REQ_I8, FIX, RES_ADD = 0, 1, 2, 3
FWD_ADVANCE = 1


class DetintError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libdetint error {code}: {msg}")
        self.code = code


_lib = None
vp, i64, i32 = C.c_void_p, C.c_int64, C.c_int32
pi32 = C.POINTER(C.c_int32)


class LayerDesc(C.Structure):
    _fields_ = [("wqkv", vp), ("wqkv_lo", vp), ("wqkv_m", vp),
                ("wo", vp), ("wo_lo", vp), ("wo_m", vp),
                ("wgu", vp), ("wgu_lo", vp), ("wgu_m", vp),
                ("wd", vp), ("wd_lo", vp), ("wd_m", vp),
                ("attn_norm", vp), ("ffn_norm", vp), ("q_norm", vp), ("k_norm", vp),
                ("kq_m", i32), ("kq_k", i32), ("vq_m", i32), ("vq_k", i32), ("k_gain", vp)]


class ModelDesc(C.Structure):
    _fields_ = [("n_layers", i64), ("hidden", i64), ("n_q", i64), ("n_kv", i64),
                ("head_dim", i64), ("ffn", i64), ("vocab", i64), ("max_pos", i64),
                ("qk_norm", i32), ("wide", i32), ("w_k", i32), ("f_res", i32),
                ("f_n", i32), ("f_a", i32), ("f_l", i32), ("reserved", i32),
                ("emb", vp), ("emb_lo", vp), ("emb_m", vp), ("final_norm", vp),
                ("rope_cos", vp), ("rope_sin", vp), ("layers", C.POINTER(LayerDesc))]


class KvDesc(C.Structure):
    _fields_ = [("k", vp), ("v", vp), ("n_slots", i64), ("n_pages", i64), ("page_size", i64),
                ("block_table", vp), ("max_blocks", i64)]


_SIGS = {
    "detint_version": (C.c_char_p, []),
    "detint_last_error": (C.c_char_p, []),
    "detint_check": (i32, [vp, C.POINTER(C.c_uint32)]),
    "detint_probe_barrier": (i32, [i32, i32, C.POINTER(C.c_uint32), vp]),
    "detint_gemm_workspace": (i64, [i64, i64, i64, i32]),
    "detint_gemm_i8": (i32, [vp, vp, i64, i64, i64, vp, vp, vp, i32, i32, i32, vp, vp, i64, vp]),
    "detint_gemm_w16": (i32, [vp, vp, vp, i64, i64, i64, vp, vp, vp, i32, i32, i32, vp, vp, i64, vp]),
    "detint_split_w16": (i32, [vp, i64, vp, vp, vp]),
    "detint_exact_prepare": (i32, [vp, i64, i64, vp, vp, vp]),
    "detint_gemm_exact_workspace": (i64, [i64, i64]),
    "detint_gemm_exact": (i32, [vp, vp, vp, i64, i64, i64, vp, vp, i32, i32, vp, vp, i64, vp]),
    "detint_rmsnorm": (i32, [vp, vp, i64, i64, vp, vp, vp, vp]),
    "detint_requant": (i32, [vp, i64, i64, vp, vp, vp]),
    "detint_requant_fixed": (i32, [vp, i64, i32, i32, vp, vp]),
    "detint_rope": (i32, [vp, vp, vp, vp, i64, i64, i64, i64, vp]),
    "detint_softmax": (i32, [vp, vp, vp, i64, i64, i32, i32, vp, vp]),
    "detint_swiglu": (i32, [vp, i64, i64, i32, vp, vp, vp, vp]),
    "detint_attn_prefill": (i32, [vp, vp, vp, vp, i64, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                  i32, i32, vp, vp]),
    "detint_attn_decode": (i32, [vp, vp, vp, vp, i64, vp, vp, i64, i64, i64, i64, i64, i32, i32,
                                 vp, vp]),
    "detint_rope_tables": (i32, [vp, vp, i64, i64, i64]),
    "detint_softmax_mult": (i32, [i32, i32, i64, i32, pi32, pi32]),
    "detint_swiglu_mult": (i32, [i32, pi32, pi32]),
    "detint_v_dequant": (i32, [i32, i32, pi32, pi32]),
    "detint_model_create": (i32, [C.POINTER(ModelDesc), C.POINTER(vp)]),
    "detint_model_destroy": (None, [vp]),
    "detint_workspace_size": (i64, [vp, i64, i64]),
    "detint_forward": (i32, [vp, vp, vp, i64, vp, i64, vp, vp, vp, i64, i64, vp, vp, vp, i32, vp,
                             i64, vp]),
    "detint_kv_bytes": (i64, [vp, C.POINTER(KvDesc)]),
    "detint_forward_kv": (i32, [vp, C.POINTER(KvDesc), vp, i64, vp, vp, vp, i64, i64, vp, vp, vp, i32,
                                vp, i64, vp]),
    "detint_lm_head_parts": (i64, [i64]),
    "detint_lm_head": (i32, [vp, vp, vp, i64, i64, i64, vp, vp, vp, i32, i32, vp, vp, vp]),
    "detint_argmax_parts": (i32, [vp, i64, i64, vp, vp]),
    "detint_sample": (i32, [vp, i64, i64, i64, i32, i32, i32, vp, vp, vp, i64, vp]),
    "detint_sample_workspace": (i64, [i64, i64]),
    "detint_final_head_workspace": (i64, [i64, i64, i64]),
    "detint_final_head": (i32, [vp, i64, i64, vp, vp, vp, vp, i64, i32, i32, vp, vp, vp, i64, vp]),
    "detint_final_head_noalloc": (i32, [vp, i64, i64, vp, vp, vp, vp, i64, i32, i32, vp, vp, vp]),
    "detint_layer_forward": (i32, [vp, i64, vp, vp, vp, i64, i64, vp, vp, vp, i64, i64, vp, i64,
                                   vp]),
}


def library():
    """The loaded libdetint (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is not built: run integer_only_deterministic_amd/build.py "
                               "(or __graft_entry__.build())")
        lib = C.CDLL(str(LIB_PATH))
        for name, (res, args) in _SIGS.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def _call(name, *args):
    lib = library()
    rc = getattr(lib, name)(*args)
    if rc != DETINT_OK:
        raise DetintError(rc, lib.detint_last_error().decode())


def _torch():
    import torch
    return torch


def _stream():
    return _torch().cuda.current_stream().cuda_stream


def _p(t, dtype=None):
    """Device pointer of a contiguous CUDA tensor (None -> NULL)."""
    if t is None:
        return None
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("expected a CUDA tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {t.dtype}")
    return t.data_ptr()


# ------------------------------------------------------------------ ops

def detint_check() -> int:
    """Wait for the current stream, then read and clear the device's bound
    flags (BOUND_* bits; 0 when every intermediate stayed in its bound)."""
    lib = library()
    f = C.c_uint32(0)
    rc = lib.detint_check(_stream(), C.byref(f))
    if rc not in (DETINT_OK, DETINT_EBOUND):
        raise DetintError(rc, lib.detint_last_error().decode())
    return int(f.value)


def detint_probe_barrier(mode: int, rounds: int, wait: bool = True):
    """Enqueue `rounds` device-wide barriers of the given mode (a measurement,
    see detint.h); with wait, synchronise and return the failure bits."""
    f = C.c_uint32(0)
    _call("detint_probe_barrier", int(mode), int(rounds), C.byref(f) if wait else None, _stream())
    return int(f.value) if wait else None


def detint_gemm_workspace(M: int, N: int, K: int, limbs: bool = False) -> int:
    return library().detint_gemm_workspace(int(M), int(N), int(K), int(bool(limbs)))


def _ws(ws):
    return (_p(ws), ws.numel() * ws.element_size()) if ws is not None else (None, 0)


def detint_gemm_i8(A, W, row_m=None, row_k=None, col_m=None, col_k=0, frac=0, mode=RAW, out=None,
                   ws=None):
    """ws: optional uint8 device workspace of detint_gemm_workspace(M, N, K)
    bytes (split-K for few-tile shapes; the same bits either way)."""
    torch = _torch()
    M, K = A.shape
    N = W.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.int8 if mode == REQ_I8 else torch.int32, device=A.device)
    _call("detint_gemm_i8", _p(A, torch.int8), _p(W, torch.int8), M, N, K, _p(row_m), _p(row_k),
          _p(col_m), int(col_k), int(frac), int(mode), _p(out), *_ws(ws), _stream())
    return out


def detint_gemm_w16(A, W_hi, W_lo, row_m=None, row_k=None, col_m=None, col_k=0, frac=0, mode=RAW,
                    out=None, ws=None):
    torch = _torch()
    M, K = A.shape
    N = W_hi.shape[0]
    if out is None:
        dt = {RAW: torch.int64, REQ_I8: torch.int8}.get(mode, torch.int32)
        out = torch.empty((M, N), dtype=dt, device=A.device)
    _call("detint_gemm_w16", _p(A, torch.int8), _p(W_hi, torch.int8), _p(W_lo, torch.int8), M, N, K,
          _p(row_m), _p(row_k), _p(col_m), int(col_k), int(frac), int(mode), _p(out), *_ws(ws),
          _stream())
    return out


def detint_split_w16(W16):
    torch = _torch()
    hi = torch.empty(W16.shape, dtype=torch.int8, device=W16.device)
    lo = torch.empty(W16.shape, dtype=torch.int8, device=W16.device)
    _call("detint_split_w16", _p(W16, torch.int16), W16.numel(), _p(hi), _p(lo), _stream())
    return hi, lo


def detint_exact_prepare(W_bits):
    """bf16 bit patterns [N, K] (a 16-bit device tensor) -> (planes int8
    [4, N, K], row_exp int32 [N]): exact-mode weights (see detint.h)."""
    torch = _torch()
    N, K = W_bits.shape
    if W_bits.element_size() != 2:
        raise TypeError("expected 16-bit bf16 bit patterns")
    planes = torch.empty((4, N, K), dtype=torch.int8, device=W_bits.device)
    row_exp = torch.empty(N, dtype=torch.int32, device=W_bits.device)
    _call("detint_exact_prepare", _p(W_bits), N, K, _p(planes), _p(row_exp), _stream())
    return planes, row_exp


def detint_gemm_exact(A, planes, row_exp, row_m=None, row_k=None, frac=0, mode=RAW, out=None, ws=None):
    torch = _torch()
    M, K = A.shape
    N = planes.shape[1]
    if out is None:
        dt = {RAW: torch.int64, REQ_I8: torch.int8}.get(mode, torch.int32)
        out = torch.empty((M, N), dtype=dt, device=A.device)
    need = library().detint_gemm_exact_workspace(M, N)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=A.device)
    _call("detint_gemm_exact", _p(A, torch.int8), _p(planes, torch.int8), _p(row_exp, torch.int32), M, N,
          K, _p(row_m), _p(row_k), int(frac), int(mode), _p(out), _p(ws), ws.numel(), _stream())
    return out


def detint_rmsnorm(h, gain):
    torch = _torch()
    R_, n = h.shape
    x8 = torch.empty((R_, n), dtype=torch.int8, device=h.device)
    rm = torch.empty(R_, dtype=torch.int32, device=h.device)
    rk = torch.empty(R_, dtype=torch.int32, device=h.device)
    _call("detint_rmsnorm", _p(h, torch.int32), _p(gain, torch.int16), R_, n, _p(x8), _p(rm), _p(rk),
          _stream())
    return x8, rm, rk


def detint_requant(y):
    torch = _torch()
    R_, n = y.shape
    q = torch.empty((R_, n), dtype=torch.int8, device=y.device)
    e = torch.empty(R_, dtype=torch.int32, device=y.device)
    _call("detint_requant", _p(y, torch.int32), R_, n, _p(q), _p(e), _stream())
    return q, e


def detint_requant_fixed(y, m, k):
    """clamp8(R(y * m, k)) elementwise (int32 device tensor -> int8)."""
    torch = _torch()
    q = torch.empty(y.shape, dtype=torch.int8, device=y.device)
    _call("detint_requant_fixed", _p(y, torch.int32), y.numel(), int(m), int(k), _p(q), _stream())
    return q


def detint_rope(x, pos, cos_t, sin_t):
    """In place on x [R, heads, d] int32."""
    torch = _torch()
    R_, heads, d = x.shape
    _call("detint_rope", _p(x, torch.int32), _p(pos, torch.int32), _p(cos_t, torch.int16),
          _p(sin_t, torch.int16), R_, heads, d, cos_t.shape[0], _stream())
    return x


def detint_softmax(s, valid, shift, mult_m, mult_k):
    torch = _torch()
    R_, Cc = s.shape
    P = torch.empty((R_, Cc), dtype=torch.int16, device=s.device)
    _call("detint_softmax", _p(s, torch.int32), _p(valid, torch.int32), _p(shift, torch.int32), R_, Cc,
          int(mult_m), int(mult_k), _p(P), _stream())
    return P


def detint_swiglu(gu, f_a):
    torch = _torch()
    R_, n2 = gu.shape
    n = n2 // 2
    a8 = torch.empty((R_, n), dtype=torch.int8, device=gu.device)
    rm = torch.empty(R_, dtype=torch.int32, device=gu.device)
    rk = torch.empty(R_, dtype=torch.int32, device=gu.device)
    _call("detint_swiglu", _p(gu, torch.int32), R_, n, int(f_a), _p(a8), _p(rm), _p(rk), _stream())
    return a8, rm, rk


def detint_attn_prefill(q8, e_q, k_cache, v_cache, cu_seqlens, start_pos, slot, mult_m, mult_k):
    """k_cache / v_cache: one layer, [n_slots, n_kv, max_pos, d] int8."""
    torch = _torch()
    R_, nq, d = q8.shape
    n_slots, nkv, max_pos, _ = k_cache.shape
    out = torch.empty((R_, nq, d), dtype=torch.int32, device=q8.device)
    _call("detint_attn_prefill", _p(q8, torch.int8), _p(e_q, torch.int32), _p(k_cache, torch.int8),
          _p(v_cache, torch.int8), n_slots, _p(cu_seqlens, torch.int32), _p(start_pos, torch.int32),
          _p(slot, torch.int32), slot.numel(), R_, nq, nkv, d, max_pos, int(mult_m), int(mult_k),
          _p(out), _stream())
    return out


def detint_attn_decode(q8, e_q, k_cache, v_cache, ctx_len, slot, mult_m, mult_k):
    torch = _torch()
    B, nq, d = q8.shape
    n_slots, nkv, max_pos, _ = k_cache.shape
    out = torch.empty((B, nq, d), dtype=torch.int32, device=q8.device)
    _call("detint_attn_decode", _p(q8, torch.int8), _p(e_q, torch.int32), _p(k_cache, torch.int8),
          _p(v_cache, torch.int8), n_slots, _p(ctx_len, torch.int32), _p(slot, torch.int32), B, nq,
          nkv, d, max_pos, int(mult_m), int(mult_k), _p(out), _stream())
    return out


def detint_lm_head(x8, emb, emb_lo, row_m, row_k, emb_m, w_k, f_l, logits=None, part=None):
    """Logits [S, V] and greedy-argmax partials [S, detint_lm_head_parts(V)]."""
    torch = _torch()
    S_, H = x8.shape
    V = emb.shape[0]
    npart = library().detint_lm_head_parts(V)
    if logits is None:
        logits = torch.empty((S_, V), dtype=torch.int32, device=x8.device)
    if part is None:
        part = torch.empty((S_, npart), dtype=torch.int64, device=x8.device)
    _call("detint_lm_head", _p(x8, torch.int8), _p(emb, torch.int8), _p(emb_lo), S_, V, H, _p(row_m),
          _p(row_k), _p(emb_m), int(w_k), int(f_l), _p(logits), _p(part), _stream())
    return logits, part


def detint_final_head(h, gain, emb, emb_lo, emb_m, w_k, f_l, logits=None, next_tok=None, ws=None,
                      with_token=True):
    """Final RMSNorm + tied lm_head + greedy token for the rows of h [S, H]:
    returns (logits [S, V], next_tok [S] or None when with_token is False)."""
    torch = _torch()
    S_, H = h.shape
    V = emb.shape[0]
    if logits is None:
        logits = torch.empty((S_, V), dtype=torch.int32, device=h.device)
    if next_tok is None and with_token:
        next_tok = torch.empty(S_, dtype=torch.int32, device=h.device)
    nbytes = library().detint_final_head_workspace(S_, V, H)
    if ws is None:
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=h.device)
    _call("detint_final_head", _p(h, torch.int32), S_, H, _p(gain, torch.int16), _p(emb, torch.int8),
          _p(emb_lo, torch.int8) if emb_lo is not None else None, _p(emb_m, torch.int32), V,
          int(w_k), int(f_l), _p(logits, torch.int32), _p(next_tok, torch.int32) if with_token else None,
          _p(ws),
          ws.numel() * ws.element_size(), _stream())
    return logits, next_tok


def detint_final_head_noalloc(h, gain, emb, emb_lo, emb_m, w_k, f_l, logits=None, next_tok=None,
                              with_token=True):
    """detint_final_head without a workspace (the library's per-device
    scratch; see detint.h)."""
    torch = _torch()
    S_, H = h.shape
    V = emb.shape[0]
    if logits is None:
        logits = torch.empty((S_, V), dtype=torch.int32, device=h.device)
    if next_tok is None and with_token:
        next_tok = torch.empty(S_, dtype=torch.int32, device=h.device)
    _call("detint_final_head_noalloc", _p(h, torch.int32), S_, H, _p(gain, torch.int16),
          _p(emb, torch.int8), _p(emb_lo, torch.int8) if emb_lo is not None else None,
          _p(emb_m, torch.int32), V, int(w_k), int(f_l), _p(logits, torch.int32),
          _p(next_tok, torch.int32) if with_token else None, _stream())
    return logits, next_tok


def detint_argmax_parts(part):
    torch = _torch()
    S_, npart = part.shape
    out = torch.empty(S_, dtype=torch.int32, device=part.device)
    _call("detint_argmax_parts", _p(part, torch.int64), S_, npart, _p(out), _stream())
    return out


def detint_sample_workspace(R: int, V: int) -> int:
    return library().detint_sample_workspace(int(R), int(V))


def detint_sample(logits, top_k: int, t_m: int, t_k: int, draws, out=None, top_p: int = 65536,
                  ws=None):
    """Integer temperature / top-k / top-p sampling of each row with the
    caller's uniform uint32 draws; top_p is p in units of 2^-16 (65536: off);
    ws an optional uint8 device workspace of detint_sample_workspace(R, V)
    bytes. See detint.h."""
    torch = _torch()
    R_, V = logits.shape
    if out is None:
        out = torch.empty(R_, dtype=torch.int32, device=logits.device)
    if draws.dtype not in (torch.int32, torch.uint32) or draws.shape != (R_,):
        raise TypeError("draws: one 32-bit integer per row (uint32, or int32 holding the bits)")
    _call("detint_sample", _p(logits, torch.int32), R_, V, int(top_k), int(top_p), int(t_m),
          int(t_k), _p(draws), _p(out), _p(ws), 0 if ws is None else ws.numel() * ws.element_size(),
          _stream())
    return out


# ---------------------------------------------------------- host set-up

def detint_rope_tables(P: int, d: int, base: int):
    c = np.zeros((P, d // 2), np.int16)
    s = np.zeros((P, d // 2), np.int16)
    _call("detint_rope_tables", c.ctypes.data, s.ctypes.data, P, d, int(base))
    return c, s


def _pair(name, *args):
    a, b = i32(), i32()
    _call(name, *args, C.byref(a), C.byref(b))
    return a.value, b.value


def detint_softmax_mult(kq_m, kq_k, d, f_n):
    return _pair("detint_softmax_mult", int(kq_m), int(kq_k), int(d), int(f_n))


def detint_swiglu_mult(f_a):
    return _pair("detint_swiglu_mult", int(f_a))


def detint_v_dequant(vq_m, vq_k):
    return _pair("detint_v_dequant", int(vq_m), int(vq_k))


# -------------------------------------------------------------- model


class DetintModel:
    """A synthetic integer model resident in device memory, driven through
    detint_forward. Weights are uploaded once; 16-bit weights are split into
    limb planes on the device with detint_split_w16."""

    def __init__(self, model, n_slots: int = 1, device: str = "cuda", page_size: int = 0,
                 n_pages: int = 0):
        """page_size > 0: the KV cache is a pool of n_pages pages of page_size
        positions per layer, addressed through self.block_table (device int32
        [n_slots, max_blocks], filled by the caller; detint_forward_kv)."""
        torch = _torch()
        self.torch = torch
        sh = model.shape
        self.shape = sh
        self.n_slots = n_slots
        self.device = device
        self._keep = []

        def up(a, dt=None):
            t = torch.from_numpy(np.ascontiguousarray(a)).to(device)
            self._keep.append(t)
            return t

        def weight(a):
            if sh.wide:
                w16 = up(a)
                hi, lo = detint_split_w16(w16)
                self._keep += [hi, lo]
                return _p(hi), _p(lo)
            return _p(up(a)), None

        layers = (LayerDesc * sh.n_layers)()
        for i, Lw in enumerate(model.layers):
            st = layers[i]
            for name in ("wqkv", "wo", "wgu", "wd"):
                hi, lo = weight(getattr(Lw, name))
                setattr(st, name, hi)
                setattr(st, name + "_lo", lo)
                setattr(st, name + "_m", _p(up(getattr(Lw, name + "_m"))))
            st.attn_norm = _p(up(Lw.attn_norm))
            st.ffn_norm = _p(up(Lw.ffn_norm))
            st.q_norm = _p(up(Lw.q_norm)) if Lw.q_norm is not None else None
            st.k_norm = _p(up(Lw.k_norm)) if Lw.k_norm is not None else None
            st.kq_m, st.kq_k, st.vq_m, st.vq_k = Lw.kq_m, Lw.kq_k, Lw.vq_m, Lw.vq_k
            kg = getattr(Lw, "k_gain", None)
            st.k_gain = _p(up(np.ascontiguousarray(kg, np.int8))) if kg is not None else None
        cos_t, sin_t = detint_rope_tables(sh.max_pos, sh.head_dim, sh.rope_base)
        self.rope_cos, self.rope_sin = up(cos_t), up(sin_t)
        d = ModelDesc(n_layers=sh.n_layers, hidden=sh.hidden, n_q=sh.n_q, n_kv=sh.n_kv,
                      head_dim=sh.head_dim, ffn=sh.ffn, vocab=sh.vocab, max_pos=sh.max_pos,
                      qk_norm=int(sh.qk_norm), wide=int(sh.wide), w_k=sh.w_k, f_res=sh.f_res,
                      f_n=sh.f_n, f_a=sh.f_a, f_l=sh.f_l)
        if model.emb is not None:
            d.emb, d.emb_lo = weight(model.emb)
            d.emb_m = _p(up(model.emb_m))
            d.final_norm = _p(up(model.final_norm))
        else:
            d.vocab = 0
        d.rope_cos, d.rope_sin = _p(self.rope_cos), _p(self.rope_sin)
        d.layers = C.cast(layers, C.POINTER(LayerDesc))
        self._layers, self._desc = layers, d
        h = vp()
        _call("detint_model_create", C.byref(d), C.byref(h))
        self.handle = h
        self.page_size = page_size
        if page_size:
            self.max_blocks = (sh.max_pos + page_size - 1) // page_size
            cache_shape = (sh.n_layers, n_pages, sh.n_kv, page_size, sh.head_dim)
            self.block_table = torch.zeros((n_slots, self.max_blocks), dtype=torch.int32, device=device)
        else:
            cache_shape = (sh.n_layers, n_slots, sh.n_kv, sh.max_pos, sh.head_dim)
            self.block_table = None
        self.kc = torch.zeros(cache_shape, dtype=torch.int8, device=device)
        self.vc = torch.zeros(cache_shape, dtype=torch.int8, device=device)
        self.kv = KvDesc(k=_p(self.kc), v=_p(self.vc), n_slots=n_slots, n_pages=n_pages,
                         page_size=page_size,
                         block_table=_p(self.block_table) if page_size else None,
                         max_blocks=self.max_blocks if page_size else 0)
        self._ws = None
        torch.cuda.synchronize()

    def __del__(self):
        try:
            if getattr(self, "handle", None) and _lib is not None:
                _lib.detint_model_destroy(self.handle)
        except Exception:
            pass

    def reset_cache(self):
        self.kc.zero_()
        self.vc.zero_()

    def contiguous_cache(self):
        """Paged pools gathered into the contiguous layout [layers, slots,
        n_kv, max_pos, d] through the block table (host arrays)."""
        sh = self.shape
        if not self.page_size:
            return self.kc.cpu().numpy(), self.vc.cpu().numpy()
        bt = self.block_table.cpu().numpy()
        out = []
        for pool in (self.kc.cpu().numpy(), self.vc.cpu().numpy()):
            c = np.zeros((sh.n_layers, self.n_slots, sh.n_kv, self.max_blocks * self.page_size,
                          sh.head_dim), np.int8)
            for s_ in range(self.n_slots):
                for b in range(self.max_blocks):
                    c[:, s_, :, b * self.page_size:(b + 1) * self.page_size] = pool[:, bt[s_, b]]
            out.append(c[:, :, :, : sh.max_pos])
        return out[0], out[1]

    def workspace(self, R: int, S: int):
        need = library().detint_workspace_size(self.handle, R, S)
        if self._ws is None or self._ws.numel() < need:
            self._ws = self.torch.empty(need, dtype=self.torch.uint8, device=self.device)
        return self._ws

    def forward_raw(self, ids, R, cu, start, slot, S, max_seqlen, logits, row_base, next_tok, flags=0):
        """Direct detint_forward on device tensors (all int32)."""
        ws = self.workspace(R, S)
        if self.page_size:
            _call("detint_forward_kv", self.handle, C.byref(self.kv), _p(ids), R, _p(cu), _p(start),
                  _p(slot), S, max_seqlen, _p(logits), _p(row_base), _p(next_tok), int(flags), _p(ws),
                  ws.numel(), _stream())
            return
        _call("detint_forward", self.handle, _p(self.kc), _p(self.vc), self.n_slots, _p(ids), R, _p(cu),
              _p(start), _p(slot), S, max_seqlen, _p(logits), _p(row_base), _p(next_tok), int(flags),
              _p(ws), ws.numel(), _stream())

    def layer(self, l: int, h, lens, starts, slots):
        """detint_layer_forward on a host int32 residual [R, H]; returns it updated."""
        torch = self.torch
        dev = self.device
        lens = list(lens)
        cu = np.zeros(len(lens) + 1, np.int32)
        cu[1:] = np.cumsum(lens)
        t = lambda a: torch.tensor(np.asarray(a, np.int32), device=dev)
        ht = torch.from_numpy(np.ascontiguousarray(h, np.int32)).to(dev)
        R_, S = int(cu[-1]), len(lens)
        ws = self.workspace(R_, S)
        # keep the argument tensors referenced until the launch is enqueued
        cu_t, st_t, sl_t = t(cu), t(starts), t(slots)
        _call("detint_layer_forward", self.handle, int(l), _p(ht), _p(self.kc), _p(self.vc),
              self.n_slots, R_, _p(cu_t), _p(st_t), _p(sl_t), S, max(lens), _p(ws),
              ws.numel(), _stream())
        return ht.cpu().numpy()

    def forward(self, ids, lens, starts, slots):
        """Host-array convenience: returns (logits [S, V], next tokens) on the host."""
        torch = self.torch
        dev = self.device
        lens = list(lens)
        cu = np.zeros(len(lens) + 1, np.int32)
        cu[1:] = np.cumsum(lens)
        t = lambda a: torch.tensor(np.asarray(a, np.int32), device=dev)
        ids_t, cu_t, st_t, sl_t = t(ids), t(cu), t(starts), t(slots)
        S = len(lens)
        logits = torch.empty((S, self.shape.vocab), dtype=torch.int32, device=dev)
        nxt = torch.empty(S, dtype=torch.int32, device=dev)
        self.forward_raw(ids_t, int(cu[-1]), cu_t, st_t, sl_t, S, max(lens), logits, None, nxt)
        return logits.cpu().numpy(), nxt.cpu().numpy()

    def _t(self, a):
        return self.torch.tensor(np.asarray(a, np.int32), device=self.device)

    def prefill(self, seqs, starts, slots, hist, base_row: int):
        """One detint_forward over packed token sequences; the logits of each
        sequence's last row go to rows base_row.. of hist (viewed [rows, V]).
        Returns the device tensor of greedy next tokens [S]."""
        torch = self.torch
        lens = [len(q) for q in seqs]
        cu = np.zeros(len(seqs) + 1, np.int32)
        cu[1:] = np.cumsum(lens)
        ids = self._t(np.concatenate([np.asarray(q, np.int32) for q in seqs]))
        tok = torch.empty(len(seqs), dtype=torch.int32, device=self.device)
        self.forward_raw(ids, int(cu[-1]), self._t(cu), self._t(starts), self._t(slots), len(seqs),
                         max(lens), hist, self._t([base_row]), tok)
        return tok

    def decode_step_fn(self, tok, pos, slots, hist, base_row: int, use_graph: bool = True):
        """Return a callable that performs one greedy decode step for B rows
        starting from tokens `tok` (device [B]) at positions `pos`: one
        detint_forward with ADVANCE, so token, positions and the logits
        history row (rows base_row + i*B .. + B for step i) advance on the
        device. With use_graph the step is captured once into a HIP graph and
        the callable replays it."""
        torch = self.torch
        B = len(pos)
        dec = dict(cu=self._t(list(range(B + 1))), start=self._t(pos), slot=self._t(slots),
                   base=self._t([base_row]), tok=tok)
        self._dec = dec
        self.workspace(B, B)

        def step():
            self.forward_raw(dec["tok"], B, dec["cu"], dec["start"], dec["slot"], B, 1, hist, dec["base"],
                             dec["tok"], FWD_ADVANCE)

        if not use_graph:
            return step
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            step()
        torch.cuda.current_stream().wait_stream(s)
        self._graph = g
        return g.replay

    def decode(self, tok, pos, slots, n_steps: int, hist, base_row: int, use_graph: bool = True):
        """n_steps greedy decode steps (see decode_step_fn)."""
        if n_steps <= 0:
            return
        step = self.decode_step_fn(tok, pos, slots, hist, base_row, use_graph)
        for _ in range(n_steps):
            step()

    def generate(self, prompts, n_new: int, use_graph: bool = True, hist=None):
        """Greedy generation (slot i = prompt i): one prefill call over all
        prompts, then n_new - 1 decode steps. Returns the device logits
        history [n_new, B, V] (step 0 = the prefill's last-position logits)."""
        B = len(prompts)
        if hist is None:
            hist = self.torch.empty((n_new, B, self.shape.vocab), dtype=self.torch.int32, device=self.device)
        tok = self.prefill(prompts, [0] * B, list(range(B)), hist, 0)
        self.decode(tok, [len(p) for p in prompts], list(range(B)), n_new - 1, hist, B, use_graph)
        return hist


def logits_chain(hist_rows) -> list:
    """Chained per-step logits hash of one sequence: H_0 = SHA-256("detint-v0"),
    H_{s+1} = SHA-256(H_s || int32 little-endian logits of step s). Returns
    the hex digests after every step."""
    h = hashlib.sha256(b"detint-v0").digest()
    out = []
    for row in hist_rows:
        h = hashlib.sha256(h + np.ascontiguousarray(row, dtype="<i4").tobytes()).digest()
        out.append(h.hex())
    return out
