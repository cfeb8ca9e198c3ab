"""Build libtpmlp.so (gfx950) in-tree with hipcc.

Usage: python -m linear_layers_amd.build   (or build() from Python)
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtpmlp.so")
SOURCES = [os.path.join(CSRC, "tpmlp.hip")]
# The machine probes (bench.py --probe) build into a library of their own.
PROBE_LIB = os.path.join(HERE, "libtpmlp_probe.so")
PROBE_SOURCES = [os.path.join(CSRC, "probes.hip")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # torch's bundled HIP runtime (ROCm 7.0) loads this library's code
    # objects, so the code-object version is pinned to one it reads.
    "-mcode-object-version=5",
    # Packed fp32 VALU forms stay off: the compiler would otherwise fuse pairs
    # of fp32 adds/multiplies into v_pk_* instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def _compile(out: str, sources, verbose: bool, extra) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra, "-o", tmp, *sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines()
            if "packed-fp32-ops" not in ln and ln.strip()]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)


def build(verbose: bool = False, extra=()) -> str:
    """Compile libtpmlp.so and the probe library libtpmlp_probe.so into
    linear_layers_amd/; returns the path of libtpmlp.so."""
    _compile(LIB, SOURCES, verbose, extra)
    _compile(PROBE_LIB, PROBE_SOURCES, verbose, extra)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, extra=sys.argv[1:]))
