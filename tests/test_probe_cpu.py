"""Host-side checks of the machine-probe library (no GPU needed).

libtpmlp_probe.so exports what include/tpmlp_probe.h declares, refuses bad
arguments before any HIP call, and every probe configuration that
`bench.py --probe` runs passes the probe's own host check of the addresses
its launch would form: without a GPU the call then stops at its first device
allocation (status 1), where an address outside the buffer would have given
status 3 before it.
"""
import ctypes
import os
import re

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "linear_layers_amd", "libtpmlp_probe.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.skip("libtpmlp_probe.so not built (run __graft_entry__.build())")
    h = ctypes.CDLL(LIB)
    h.tpmlp_probe_last_error.restype = ctypes.c_char_p
    return h


def test_exports_every_declared_symbol(lib):
    src = open(os.path.join(ROOT, "include", "tpmlp_probe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = set(re.findall(r"^\s*(?:const\s+)?(?:int|char\s*\*|const char\s*\*)\s*\*?\s*(\w+)\s*\(", src, flags=re.M))
    assert names == {"tpmlp_probe_load_path", "tpmlp_probe_lds_read", "tpmlp_probe_last_error"}
    for n in names:
        assert hasattr(lib, n), f"{n} declared but not exported"


@pytest.mark.parametrize("args", [(3, 0, 4096, 8192, 20), (0, 4, 4096, 8192, 20), (0, 0, 4095, 8192, 20),
                                  (0, 0, 4096, 2047, 20), (0, 0, 4096, 8192, 0), (0, 0, 70000, 8192, 20)])
def test_load_probe_refuses_bad_arguments(lib, args):
    out = (ctypes.c_double * 4)()
    assert lib.tpmlp_probe_load_path(*args, out) == 2
    assert b"bad arguments" in lib.tpmlp_probe_last_error()


@pytest.mark.parametrize("args", [(0, 5, 10), (1, 12, 10), (0, 4, 0)])
def test_lds_probe_refuses_bad_arguments(lib, args):
    out = (ctypes.c_double * 2)()
    assert lib.tpmlp_probe_lds_read(*args, out) == 2


@pytest.mark.parametrize("lda,ldb", [(4096, 8192), (4160, 8256)])
def test_every_bench_probe_passes_the_address_check(lib, lda, ldb):
    out = (ctypes.c_double * 4)()
    for mode, pat, _ in bench.PROBE_LOADS:
        rc = lib.tpmlp_probe_load_path(mode, pat, lda, ldb, 1, out)
        msg = lib.tpmlp_probe_last_error().decode()
        if rc == 0:   # a GPU is present: the probe ran
            assert out[3] > 0
            continue
        assert rc == 1, f"mode {mode} pattern {pat}: {msg}"
