"""CPU float64 oracle for the tensor-parallel MLP block.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check in
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or run anything in this package.  The GPU library never calls it and
shares no code with it; the two meet only through the seeded inputs of the
``synth`` package.

``ref``    numpy float64 implementation (library matmul as the only primitive).
``brute``  pure-Python loops for tiny inputs, used to pin ``ref``.

Every function in ``ref`` is pinned by CPU tests (``tests/test_oracle_*.py``):
a hand-worked integer example, torch's float64 GeLU and autograd, central
finite differences, brute-force loops and the block-matrix identities the
pages state.  No function is "parity unpinned".
"""
from . import ref, brute  # noqa: F401
