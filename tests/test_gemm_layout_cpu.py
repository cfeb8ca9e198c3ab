"""Host check of the four-wave GEMM's LDS layouts (no GPU needed).

Builds tests/native/gemm_w4_layout_check.cpp with the host compiler against
linear_layers_amd/csrc/gemm_w4_layout.hpp and runs it: every wave, lane,
fragment block and K substep of 256- and 128-row tiles, both operand
orientations.  It checks that the DMA placement covers each tile chunk once,
that every fragment read hands each lane the 8 operand values the
v_mfma_f32_16x16x32_bf16 layout expects, that the kernel's base+immediate
offsets equal the direct formulas, that every access stays in the tile, and
that the reads are free of bank conflicts under the bank model fitted to
rocprofv3's conflict counts (stated in the header).
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_gemm_w4_layouts(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path / "layout_check")
    src = os.path.join(HERE, "native", "gemm_w4_layout_check.cpp")
    subprocess.run([cxx, "-O2", "-std=c++17", "-o", exe, src], check=True, capture_output=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("OK"), r.stdout + r.stderr
