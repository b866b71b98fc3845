"""The oracle under UndefinedBehaviorSanitizer: the C source is rebuilt with
-fsanitize=undefined (signed overflow, shifts out of range, misaligned or
out-of-bounds accesses the checks can see) and the process aborts on the
first report. A child process then drives every oracle entry point over
the cases the pins use: rounding edges, GEMMs with extreme operands and both
weight widths, every epilogue mode, RMSNorm at the top of its domain,
softmax, SwiGLU, RoPE, attention, a whole layer with its dump, generation
with both tiny models and with key gains, and integer sampling."""
import os
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent

DRIVER = r'''
import numpy as np
import detint_synth as S
import oracle as O
assert O.lib()._name.endswith("liboracle_ubsan.so")
for x in (0, 1, -1, 2**40 + 3, -(2**40) - 3, 2**61, -(2**61)):
    for s in (-3, 0, 1, 7, 31, 62):
        try:
            O.rshift_round(x, s)
        except O.OracleError:
            pass
for a, b in ((0, 1), (7, 2), (2**60, 3)):
    O.div_round(a, b)
for n in (0, 1, 2**62, 2**64 - 1):
    O.isqrt(n)
for u in (0, -1, -32768, -(2**20), -(2**40)):
    O.diexp(u)
O.irms(2**62 - 1, 16384); O.irms(1, 1)
rng = np.random.default_rng(0)
A = rng.integers(-128, 128, (9, 64)).astype(np.int8); A[0] = -128
W = rng.integers(-128, 128, (7, 64)).astype(np.int8); W[0] = -128
W16 = rng.integers(-32767, 32768, (7, 64)).astype(np.int16)
acc = O.gemm(A, W); O.gemm(A, W16)
rm = rng.integers(1 << 14, 1 << 15, 9).astype(np.int32); rk = np.full(9, 20, np.int32)
cm = rng.integers(1 << 14, 1 << 15, 7).astype(np.int32)
for mode in (O.RAW, O.REQ_I8, O.FIX, O.RES_ADD):
    O.epilogue(acc, rm, rk, cm, 22, 8, mode, out=np.zeros((9, 7), np.int32))
h = rng.integers(-(2**24) + 1, 2**24, (3, 16384)).astype(np.int32)
O.rmsnorm(h, np.full(16384, 8192, np.int16))
O.requant_rows(rng.integers(-(2**30), 2**30, (4, 100)).astype(np.int32))
O.softmax(rng.integers(-(2**20), 2**20, (5, 40)).astype(np.int32), np.array([1, 5, 40, 39, 2], np.int32),
          np.array([0, 3, 7, 9, 12], np.int32), 23637, 20)
O.swiglu(rng.integers(-(2**23), 2**23, (3, 64)).astype(np.int32), 12)
c, s_ = O.rope_tables(64, 64, 1000000)
O.rope(rng.integers(-(2**20), 2**20, (4, 2, 64)).astype(np.int32), np.array([0, 1, 33, 63], np.int32), c, s_)
lg = rng.integers(-(2**20), 2**20, (2, 500)).astype(np.int32)
O.sample(lg, 50, 23637, 15, np.array([1, 2**32 - 1], np.uint32), top_p=58982)
O.sample(lg, 0, 23637, 15, np.array([7, 9], np.uint32))
m = S.make_model("layer256", seed=1)
O.OracleModel(m, slots=1).layer(0, S.make_residual(64, 256, seed=2), [64], [0], [0], dump=True)
for name in ("tiny", "tiny_wide"):
    mm = S.make_model(name, seed=3)
    O.OracleModel(mm, slots=2).generate([S.make_prompt(1000, 20, 1), S.make_prompt(1000, 5, 2)], 4)
    O.OracleModel(mm, slots=1).embed(np.array([0, 999], np.int32))
mg = S.with_key_gains(S.make_model("tiny", seed=4), seed=5, gmax=3)
O.OracleModel(mg, slots=1).generate([S.make_prompt(1000, 17, 3)], 3)
print("ubsan driver done")
'''


def test_oracle_has_no_undefined_behaviour(tmp_path):
    src = ROOT / "oracle" / "detint_oracle.c"
    lib = tmp_path / "liboracle_ubsan.so"
    r = subprocess.run(["gcc", "-O1", "-g", "-std=gnu11", "-fopenmp", "-fPIC", "-shared",
                        "-fsanitize=undefined", "-fno-sanitize-recover=all", "-o", str(lib),
                        str(src), "-lm"], capture_output=True, text=True)
    if r.returncode != 0 and "ubsan" in (r.stderr or ""):
        pytest.skip("UndefinedBehaviorSanitizer runtime not available: " + r.stderr[-200:])
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, DETINT_ORACLE_LIB=str(lib), UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="4", PYTHONPATH=str(ROOT))
    p = subprocess.run([sys.executable, "-c", DRIVER], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    assert p.returncode == 0 and "ubsan driver done" in p.stdout, p.stderr[-3000:]
    assert "runtime error" not in p.stderr, p.stderr[-3000:]
