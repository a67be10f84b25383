"""Host-only checks of the library's own gfx950 machine code (no GPU needed).

The grouped GEMM issues its stage loads (buffer_load ... lds) from inline
asm, where the compiler's hazard recognizer cannot see them: a vector
instruction that writes an SGPR (a readfirstlane of the resource base, an
SGPR spill reload) must be followed by five wait states before a
vector-memory instruction reads that SGPR, and each load statement pads
itself to five (a select plus `s_nop 3`, or `s_nop 4`).  This test
disassembles the code object built into libmxq.so and checks every such
load, so that an edit dropping the padding fails here rather than as a
memory fault on the GPU.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "swiglu_mxfp8_quant_amd", "libmxq.so")
LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"


def _tools():
    tools = {"objcopy": shutil.which("objcopy"),
             "bundler": os.path.join(LLVM, "clang-offload-bundler"),
             "objdump": os.path.join(LLVM, "llvm-objdump")}
    missing = [k for k, v in tools.items() if not v or not os.path.exists(v)]
    return tools, missing


def _device_code(tmp_path):
    """Instruction lists (mnemonic + operands) of every gfx950 code object in the library."""
    tools, missing = _tools()
    if missing:
        pytest.skip(f"tools not found: {missing}")
    if not os.path.exists(LIB):
        pytest.skip("libmxq.so is not built")
    fat = tmp_path / "fatbin.bin"
    # objcopy rewrites the file it reads in place: work on a copy, never on the
    # library this process (or another) has mapped
    lib_copy = tmp_path / "libmxq_copy.so"
    shutil.copyfile(LIB, lib_copy)
    subprocess.run([tools["objcopy"], "--dump-section", f".hip_fatbin={fat}", str(lib_copy)], check=True)
    blob = fat.read_bytes()
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    starts = [m.start() for m in re.finditer(re.escape(magic), blob)]
    assert starts, "no offload bundle in the library"
    objs = []
    for k, s in enumerate(starts):
        e = starts[k + 1] if k + 1 < len(starts) else len(blob)
        b = tmp_path / f"b{k}.bin"
        co = tmp_path / f"b{k}.co"
        b.write_bytes(blob[s:e])
        subprocess.run([tools["bundler"], "--unbundle", "--type=o", f"--input={b}", f"--targets={TARGET}",
                        f"--output={co}"], check=True)
        text = subprocess.run([tools["objdump"], "-d", "--mcpu=gfx950", str(co)], check=True,
                              capture_output=True, text=True).stdout
        objs.append([ln.strip().split("//")[0].strip() for ln in text.split("\n") if re.match(r"^\s+[a-z]", ln)])
    return objs


def _padded(prev):
    """The two instructions before an LDS-DMA load give it five wait states."""
    if prev and re.fullmatch(r"s_nop (0x)?[4-9a-f]", prev[-1]):
        return True
    return (len(prev) == 2 and re.fullmatch(r"s_nop (0x)?3", prev[-1]) is not None
            and prev[-2].startswith("v_cndmask_b32"))


def test_lds_dma_loads_are_padded(tmp_path):
    objs = _device_code(tmp_path)
    loads, bad = 0, []
    for seq in objs:
        for i, ins in enumerate(seq):
            if ins.startswith("buffer_load") and re.search(r"\blds\b", ins):
                loads += 1
                prev = seq[max(0, i - 2):i]
                if not _padded(prev):
                    bad.append((prev, ins))
    assert loads > 1000, f"expected the grouped GEMM's LDS-DMA loads, found {loads}"
    assert not bad, f"{len(bad)} LDS-DMA loads without five wait states, e.g. {bad[:3]}"
