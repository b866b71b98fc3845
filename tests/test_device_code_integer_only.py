"""Float-leak guard over the built device code (DetLLM README, "Layout": a
guard makes any float in the forward pass an error; DetLLM blog, "DetLLM":
every op is integer arithmetic).

The gfx950 code objects inside the library's object files (built by
build.py) are disassembled with the ROCm LLVM tools and searched for any
floating-point instruction: float arithmetic, conversions, transcendental
and reciprocal ops (the compiler's expansion of a run-time integer `/` or `%`
seeds its quotient with a float reciprocal, so this also rejects such
divisions in kernels), packed fp32 ops, and matrix ops other than the int8
ones. Host set-up code (RoPE tables, offline multipliers) is not device code
and is not scanned."""
import re
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
BUILD = ROOT / "integer_only_deterministic_amd" / "_build"
LLVM = Path("/opt/rocm/llvm/bin")
KERNEL_SOURCES = ["gemm.hip", "decode.hip", "rowops.hip", "attention.hip"]

FLOAT_OP = re.compile(r"\b[vs]_\w*?(f16|f32|f64|bf16)\w*|\bv_(rcp|rsq|sqrt|exp|log|sin|cos|ldexp|"
                      r"frexp|fract|div_\w+)\w*")
MFMA = re.compile(r"\bv_(s?mfma|smfmac)\w*")


def _disassemble(obj: Path, tmp: Path) -> str:
    fat = tmp / (obj.name + ".fatbin")
    co = tmp / (obj.name + ".co")
    subprocess.run(["objcopy", f"--dump-section=.hip_fatbin={fat}", str(obj)], check=True,
                   capture_output=True)
    subprocess.run([str(LLVM / "clang-offload-bundler"), "--unbundle", "--type=o",
                    f"--input={fat}", "--targets=hipv4-amdgcn-amd-amdhsa--gfx950",
                    f"--output={co}"], check=True, capture_output=True)
    return subprocess.run([str(LLVM / "llvm-objdump"), "-d", str(co)], check=True,
                          capture_output=True, text=True).stdout


@pytest.mark.skipif(not (LLVM / "llvm-objdump").exists() or shutil.which("objcopy") is None,
                    reason="ROCm LLVM tools not installed")
@pytest.mark.parametrize("src", KERNEL_SOURCES)
def test_kernels_contain_no_floating_point_instruction(src, tmp_path):
    obj = BUILD / (src + ".o")
    if not obj.exists():
        pytest.skip(f"{obj} not built (run __graft_entry__.build())")
    text = _disassemble(obj, tmp_path)
    insts = [ln.split("//")[0].strip() for ln in text.splitlines() if ln.startswith("\t")]
    assert len(insts) > 1000, "disassembly looks empty"
    bad = sorted({m.group(0) for ln in insts for m in [FLOAT_OP.search(ln)] if m})
    assert not bad, f"{src}: floating-point instructions in device code: {bad[:20]}"
    mfma = sorted({m.group(0) for ln in insts for m in [MFMA.search(ln)] if m})
    assert all(re.fullmatch(r"v_mfma_i32_\w+_i8", op) for op in mfma), f"{src}: non-int8 matrix ops {mfma}"


def test_guard_detects_a_float_instruction():
    """The pattern recognises the instructions a leak would produce."""
    for op in ("v_add_f32_e32 v1, v2, v3", "v_cvt_f32_u32_e32 v0, v1", "v_rcp_iflag_f32_e32 v4, v4",
               "v_pk_fma_f32 v[0:1], v[2:3], v[4:5], v[6:7]", "v_fma_f64 v[0:1], v[2:3], v[4:5], v[6:7]",
               "v_sqrt_f32_e32 v0, v0", "v_div_scale_f64 v[0:1], vcc, v[2:3], v[2:3], v[4:5]"):
        assert FLOAT_OP.search(op), op
    for op in ("v_add_u32_e32 v1, v2, v3", "v_mad_u64_u32 v[0:1], s[0:1], v2, v3, v[4:5]",
               "v_dot4_i32_i8 v0, v1, v2, v0", "v_mfma_i32_32x32x32_i8 a[0:15], v[0:3], v[4:7], a[0:15]",
               "v_mul_hi_i32 v0, v1, v2", "global_load_dwordx4 v[0:3], v[4:5], off"):
        assert not FLOAT_OP.search(op), op
