"""Host check of the M0 invariant in the built library (no GPU needed).

The GEMM and attention kernels issue their global -> LDS loads as inline asm
pairs `s_mov_b32 m0, <lds address>` + `buffer_load_dwordx4 ... lds` and list
m0 as clobbered; the compiler treats m0 as reserved and does not promise to
save it around such a statement.  That is safe exactly when nothing but these
pairs touches m0: no compiler-generated instruction writes it or reads it
(explicitly, or implicitly as s_movrel*, v_movrel*, the *_addtid LDS ops,
GWS, append/consume, s_sendmsg, v_interp or compiler-emitted LDS-DMA loads
do), and every LDS-DMA load follows its own m0 write.  This test unbundles the
gfx950 code object from linear_layers_amd/libtpmlp.so and from the probe
library libtpmlp_probe.so (both built here from this repository's sources),
disassembles it with the ROCm LLVM tools and checks both properties over
every kernel.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBS = {"libtpmlp.so": 10000, "libtpmlp_probe.so": 100}   # library: fewest instructions it must hold
LLVM = "/opt/rocm/llvm/bin"
IMPLICIT_M0 = re.compile(r"s_movrel|v_movrel|_addtid|ds_gws|ds_append|ds_consume|s_sendmsg|global_load_lds|v_interp")


def _tool(name):
    path = os.path.join(LLVM, name)
    return path if os.path.exists(path) else shutil.which(name)


@pytest.mark.parametrize("lib", sorted(LIBS))
def test_m0_written_only_by_the_dma_pairs(tmp_path, lib):
    LIB = os.path.join(ROOT, "linear_layers_amd", lib)
    if not os.path.exists(LIB):
        pytest.skip(f"{lib} not built (run __graft_entry__.build())")
    objcopy, bundler, objdump = _tool("llvm-objcopy"), _tool("clang-offload-bundler"), _tool("llvm-objdump")
    if not (objcopy and bundler and objdump):
        pytest.skip("ROCm LLVM tools not found")
    fat, co = str(tmp_path / "fat.bin"), str(tmp_path / "gfx950.o")
    subprocess.run([objcopy, "--dump-section", f".hip_fatbin={fat}", LIB, str(tmp_path / "lib.so")], check=True,
                   capture_output=True)
    subprocess.run([bundler, "--type=o", f"--input={fat}", "--targets=hipv4-amdgcn-amd-amdhsa--gfx950",
                    f"--output={co}", "--unbundle"], check=True, capture_output=True)
    dis = subprocess.run([objdump, "-d", "--mcpu=gfx950", co], check=True, capture_output=True, text=True).stdout
    ins = []
    for line in dis.splitlines():
        text = line.split("//")[0].strip()
        if text and not text.endswith(":") and "file format" not in text and not text.startswith(("Disassembly", "<")):
            ins.append(text)
    assert len(ins) > LIBS[lib], "disassembly looks empty"
    pairs = 0
    for i, text in enumerate(ins):
        assert not IMPLICIT_M0.search(text), f"instruction that reads m0 implicitly: {text}"
        is_dma = text.startswith("buffer_load") and text.endswith(" lds")
        if re.search(r"\bm0\b", text):
            assert text.startswith("s_mov_b32 m0, s"), f"m0 used outside the DMA pairs: {text}"
            assert ins[i + 1].startswith("buffer_load") and ins[i + 1].endswith(" lds"), \
                f"m0 written but not followed by its LDS-DMA load: {text} | {ins[i + 1]}"
        if is_dma:
            assert ins[i - 1].startswith("s_mov_b32 m0, s"), f"LDS-DMA load without its m0 write: {ins[i - 1]} | {text}"
            pairs += 1
    assert pairs > 0, "no LDS-DMA loads found"
