"""Checks on the device code of the built library (host only, no GPU).

The library's gfx950 code objects are taken out of its offload bundles and
disassembled with ROCm's own LLVM tools; every check reads only code built
from this repository's sources.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "ragged_verification_amd", "librv.so")
LLVM = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"


def _tools():
    tools = {"bundler": os.path.join(LLVM, "clang-offload-bundler"),
             "objdump": os.path.join(LLVM, "llvm-objdump"),
             "objcopy": shutil.which("objcopy")}
    if not all(t and os.path.exists(t) for t in tools.values()):
        pytest.skip("ROCm LLVM tools or objcopy not available")
    if not os.path.exists(LIB):
        pytest.skip("librv.so not built (run __graft_entry__.build() first)")
    return tools


@pytest.fixture(scope="module")
def disassembly(tmp_path_factory):
    """Disassembly of every gfx950 code object in the library, one string per
    source file's bundle."""
    t = _tools()
    d = tmp_path_factory.mktemp("devcode")
    fat = d / "fatbin.bin"
    subprocess.run([t["objcopy"], "--dump-section", f".hip_fatbin={fat}", LIB, str(d / "stripped.so")],
                   check=True, capture_output=True)
    data = fat.read_bytes()
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)]
    assert starts, "no offload bundle in the library"
    out = []
    for n, a in enumerate(starts):
        b = starts[n + 1] if n + 1 < len(starts) else len(data)
        part, obj = d / f"b{n}.bin", d / f"c{n}.o"
        part.write_bytes(data[a:b])
        subprocess.run([t["bundler"], "--unbundle", "--type=o", f"--input={part}", f"--targets={TARGET}",
                        f"--output={obj}"], check=True, capture_output=True)
        r = subprocess.run([t["objdump"], "-d", str(obj)], check=True, capture_output=True, text=True)
        out.append(r.stdout)
    return out


def test_every_source_has_gfx950_code(disassembly):
    """One gfx950 code object per compiled source, and the kernels the
    launchers name are in them."""
    text = "\n".join(disassembly)
    assert len(disassembly) >= 9
    for kern in ("k_schedule", "k_pack", "k_pack_plan", "k_attn_mla_row", "k_attn_gqa_bal", "k_attn_combine",
                 "k_lm_gemm_tiled", "k_lm_gemm_rows", "k_lm_gemm_small", "k_accept", "k_scatter", "k_estimate",
                 "k_calibration"):
        assert kern in text, kern


def test_no_writes_through_the_scalar_cache(disassembly):
    """The device code writes memory only through vector stores: no scalar
    memory stores or atomics and no scalar-cache write-back anywhere."""
    pat = re.compile(r"^\s+s_(store|atomic|dcache_wb|scratch_store|buffer_store|buffer_atomic)\w*\s", re.M)
    hits = [m.group(0).strip() for text in disassembly for m in pat.finditer(text)]
    assert not hits, hits[:10]


def test_no_packed_fp32_arithmetic(disassembly):
    """Every source is built without packed-fp32 instruction selection, so no
    packed fp32 add, multiply or fma appears."""
    pat = re.compile(r"^\s+v_pk_(add|mul|fma)_f32\s", re.M)
    hits = [m.group(0).strip() for text in disassembly for m in pat.finditer(text)]
    assert not hits, hits[:10]
