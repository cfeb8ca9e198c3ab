"""The machine probes (libtpmlp_probe.so) on the GPU: one load-path case and
one LDS-read case run and report figures in a physical range (the per-CU
load path moves tens of bytes per clock, LDS reads between tens and a few
hundred; a figure outside 5-1000 would mean a broken clock or byte count).
The address check that precedes each launch is covered on the CPU by
test_probe_cpu.py."""
import ctypes
import os

import pytest

from tests.gpu_util import need_gpu

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "linear_layers_amd", "libtpmlp_probe.so")


def _lib():
    need_gpu()
    assert os.path.exists(LIB), "libtpmlp_probe.so is not built"
    h = ctypes.CDLL(LIB)
    h.tpmlp_probe_last_error.restype = ctypes.c_char_p
    return h


def test_load_path_probe_runs():
    lib = _lib()
    print("load-path probe: LDS DMA, the GEMM tiles' operand mix", flush=True)
    out = (ctypes.c_double * 4)()
    rc = lib.tpmlp_probe_load_path(0, 0, 4096, 8192, 3, out)
    assert rc == 0, lib.tpmlp_probe_last_error().decode()
    us, ghz, gbs, bpc = list(out)
    assert us > 0 and 0.5 < ghz < 3.0 and gbs > 0
    assert 5 < bpc < 1000, bpc


def test_lds_read_probe_runs():
    lib = _lib()
    print("LDS-read probe: ds_read_b128, 8 waves", flush=True)
    out = (ctypes.c_double * 2)()
    rc = lib.tpmlp_probe_lds_read(0, 8, 512, out)
    assert rc == 0, lib.tpmlp_probe_last_error().decode()
    assert out[0] > 0 and 5 < out[1] < 1000, list(out)
