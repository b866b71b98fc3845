"""CPU-side checks of the HIP library: it loads, exports every symbol the
header declares, its host-side set-up arithmetic (RoPE tables, softmax /
SiLU multipliers, V dequant scale) equals the oracle's, and argument
validation rejects bad calls before any device work. No GPU needed."""
import ctypes as C
import re
from pathlib import Path

import numpy as np
import pytest

import detint_synth as S
import oracle as O

ROOT = Path(__file__).resolve().parent.parent


@pytest.fixture(scope="module")
def D():
    import integer_only_deterministic_amd as D
    if not D.LIB_PATH.exists():
        from integer_only_deterministic_amd import build
        build.build()
    D.library()
    return D


def header_symbols():
    text = (ROOT / "include" / "detint.h").read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(detint_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(D):
    names = header_symbols()
    assert len(names) >= 20
    lib = C.CDLL(str(D.LIB_PATH))
    for n in names:
        assert hasattr(lib, n), n
    # the binding covers the same names
    assert set(names) <= set(D._SIGS), set(names) - set(D._SIGS)
    for n in ("detint_gemm_i8", "detint_rmsnorm", "detint_rope", "detint_attn_prefill",
              "detint_attn_decode", "detint_softmax", "detint_swiglu", "detint_requant",
              "detint_forward"):
        assert n in names


def test_rope_tables_match_oracle(D):
    for P, d, base in ((1024, 128, 1_000_000), (256, 64, 1_000_000), (4096, 64, 500_000)):
        c1, s1 = D.detint_rope_tables(P, d, base)
        c2, s2 = O.rope_tables(P, d, base)
        np.testing.assert_array_equal(c1, c2)
        np.testing.assert_array_equal(s1, s2)


def test_setup_constants_match_oracle(D):
    for name in ("layer256", "qwen3_0.6b", "llama3.2_1b"):
        sh = S.SHAPES[name]
        kv = S._kv_scales(sh)
        assert D.detint_softmax_mult(kv["kq_m"], kv["kq_k"], sh.head_dim, sh.f_n) == \
            O.softmax_mult(kv["kq_m"], kv["kq_k"], sh.head_dim, sh.f_n)
        assert D.detint_v_dequant(kv["vq_m"], kv["vq_k"]) == O.v_dequant(kv["vq_m"], kv["vq_k"])
    rng = np.random.default_rng(0)
    for _ in range(300):
        a, b, d = int(rng.integers(1 << 14, 1 << 15)), int(rng.integers(5, 40)), int(rng.choice([64, 128]))
        assert D.detint_softmax_mult(a, b, d, 12) == O.softmax_mult(a, b, d, 12)
        assert D.detint_v_dequant(a, b) == O.v_dequant(a, b)
    for f in range(0, 20):
        assert D.detint_swiglu_mult(f) == O.swiglu_mult(f)


def test_validation_rejects_before_device_work(D):
    lib = D.library()
    fake = C.c_void_p(4096)
    # K not a multiple of 16
    rc = lib.detint_gemm_i8(fake, fake, 4, 4, 15, None, None, None, 0, 0, D.RAW, fake, None, 0, None)
    assert rc == D.DETINT_EINVAL and b"multiple of 16" in lib.detint_last_error()
    # misaligned operand
    rc = lib.detint_gemm_i8(C.c_void_p(4097), fake, 4, 4, 16, None, None, None, 0, 0, D.RAW, fake, None, 0, None)
    assert rc == D.DETINT_EINVAL
    # K beyond the int32 accumulator bound
    rc = lib.detint_gemm_i8(fake, fake, 4, 4, 1 << 20, None, None, None, 0, 0, D.RAW, fake, None, 0, None)
    assert rc == D.DETINT_EINVAL
    # scaled modes need scales
    rc = lib.detint_gemm_i8(fake, fake, 4, 4, 16, None, None, None, 0, 0, D.REQ_I8, fake, None, 0, None)
    assert rc == D.DETINT_EINVAL
    # empty GEMM is a no-op
    assert lib.detint_gemm_i8(None, None, 0, 4, 16, None, None, None, 0, 0, D.RAW, None, None, 0, None) == 0
    # the int32 accumulator bound: 131072 * (-128)^2 = 2^31 does not fit, 131056 does
    assert lib.detint_gemm_i8(None, None, 0, 4, 131056, None, None, None, 0, 0, D.RAW, None, None, 0, None) == 0
    assert lib.detint_gemm_i8(None, None, 0, 4, 131072, None, None, None, 0, 0, D.RAW, None,
                              None, 0, None) == D.DETINT_EINVAL
    # workspace sizes: split-K only where the shape gives few tiles
    assert lib.detint_gemm_workspace(32, 1024, 8192, 0) > 0          # skinny rows, long K
    assert lib.detint_gemm_workspace(512, 1024, 8192, 0) >= 4 * 8 * 512 * 1024
    assert lib.detint_gemm_workspace(512, 1024, 2048, 0) == 0        # short K: no split
    assert lib.detint_gemm_workspace(2048, 151936, 1024, 0) == 0     # fills the chip
    assert lib.detint_gemm_workspace(-1, 4, 16, 0) == -1
    # unsupported attention head_dim
    rc = lib.detint_attn_decode(fake, fake, fake, fake, 1, fake, fake, 1, 4, 2, 96, 64, 1 << 14, 10,
                                fake, None)
    assert rc == D.DETINT_EUNSUPPORTED
    # model without layers
    desc = D.ModelDesc(n_layers=1, hidden=256, n_q=4, n_kv=2, head_dim=64, ffn=768, vocab=0, max_pos=64)
    h = C.c_void_p()
    assert lib.detint_model_create(C.byref(desc), C.byref(h)) == D.DETINT_EINVAL
    assert lib.detint_workspace_size(None, 1, 1) == -1
    # key gains need kq_k >= 8 (the key shift kq_k - g stays >= 1)
    L = D.LayerDesc(wqkv=fake, wqkv_m=fake, wo=fake, wo_m=fake, wgu=fake, wgu_m=fake, wd=fake,
                    wd_m=fake, attn_norm=fake, ffn_norm=fake, kq_m=1 << 14, kq_k=7,
                    vq_m=1 << 14, vq_k=20, k_gain=fake)
    layers = (D.LayerDesc * 1)(L)
    desc.layers = C.cast(layers, C.POINTER(D.LayerDesc))
    desc.rope_cos = desc.rope_sin = fake
    assert lib.detint_model_create(C.byref(desc), C.byref(h)) == D.DETINT_EINVAL
    assert b"kq_k >= 8" in lib.detint_last_error()
    # sampling: vocabulary, temperature and top-p ranges; empty batch is a no-op
    T = (23637, 15)
    rc = lib.detint_sample(fake, 1, 262145, 0, 65536, *T, fake, fake, None, 0, None)
    assert rc == D.DETINT_EINVAL and b"262144" in lib.detint_last_error()
    assert lib.detint_sample(fake, 1, 100, 0, 0, *T, fake, fake, None, 0, None) == D.DETINT_EINVAL
    assert lib.detint_sample(fake, 1, 100, 0, 65537, *T, fake, fake, None, 0, None) == D.DETINT_EINVAL
    assert lib.detint_sample(fake, 1, 100, 0, 65536, 0, 15, fake, fake, None, 0, None) == D.DETINT_EINVAL
    assert lib.detint_sample(fake, 1, 100, 0, 65536, 1 << 24, 15, fake, fake, None, 0,
                             None) == D.DETINT_EINVAL
    assert lib.detint_sample(fake, 1, 100, 0, 65536, 23637, 63, fake, fake, None, 0,
                             None) == D.DETINT_EINVAL
    assert lib.detint_sample(None, 1, 100, 0, 65536, *T, fake, fake, None, 0, None) == D.DETINT_EINVAL
    assert lib.detint_sample(fake, 1, 100, 0, 65536, *T, fake, fake, C.c_void_p(4097), 64,
                             None) == D.DETINT_EINVAL  # misaligned workspace
    assert lib.detint_sample(None, 0, 100, 0, 65536, *T, None, None, None, 0, None) == D.DETINT_OK
    # candidates (16384 x 8 B), 149 slice maxima and 596 step sums, 75 cut keys
    assert lib.detint_sample_workspace(8, 151936) == 8 * (16384 * 8 + 149 * 20 + 75 * 4)
    assert lib.detint_sample_workspace(1, 262145) == -1
    # barrier probe: mode and round ranges
    assert lib.detint_probe_barrier(4, 10, None, None) == D.DETINT_EINVAL
    assert lib.detint_probe_barrier(0, -1, None, None) == D.DETINT_EINVAL


def test_no_cpu_fallback_without_library(tmp_path, monkeypatch):
    import integer_only_deterministic_amd as D
    monkeypatch.setattr(D, "LIB_PATH", tmp_path / "missing.so")
    monkeypatch.setattr(D, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        D.library()
