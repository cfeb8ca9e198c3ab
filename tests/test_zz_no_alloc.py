"""The allocation-free MLP backward (tp_mlp_bwd_noalloc) against tp_mlp_bwd.

tp_mlp_bwd_noalloc keeps its workspace in the library's static device array
instead of a caller buffer; it runs the same kernels in the same order, so
its outputs must equal tp_mlp_bwd's bit for bit.  Two calls in a row, the
second smaller, check that state left in the shared array by one call does
not leak into the next.  Sizes beyond the array are refused before anything
is written.
"""
from __future__ import annotations

import pytest
import torch

import synth
from tests.gpu_util import empty, empty_f32, need_gpu, sync, to_dev

pytestmark = pytest.mark.gpu

import linear_layers_amd as tl  # noqa: E402


def _case(T, h, F, tp, seed):
    print(f"noalloc case T={T} h={h} F={F} tp={tp}", flush=True)
    wl = synth.Workload("t", seed, "bf16", T=T, h=h, F=F, tp=tp, x_std=1.0, w_std=0.05, b_std=0.1, dz_std=1.0)
    raw = synth.mlp_inputs(wl)
    Fs = F // tp
    X, W1, W2, b1, dZ = (to_dev(raw[k], "bf16") for k in ("X", "W1", "W2", "b1", "dZ"))
    W1s, W2s, b1s = W1[:, :Fs], W2[:Fs].contiguous(), b1[:Fs]
    A, H, Z = empty((T, Fs), "bf16"), empty((T, Fs), "bf16"), empty_f32((T, h))
    tl.tp_mlp_fwd(X, W1s, b1s, W2s, tp, A, Z, H_save=H)
    outs = []
    for fn in (tl.tp_mlp_bwd, tl.tp_mlp_bwd_noalloc):
        dX, dW1, db1, dW2 = empty_f32((T, h)), empty_f32((h, Fs)), empty_f32((Fs,)), empty_f32((Fs, h))
        for t in (dX, dW1, db1, dW2):
            t.fill_(float("nan"))
        fn(X, W1s, W2s, H, A, dZ, tp, dX, dW1, dW2, db1_shard=db1)
        sync()
        outs.append((dX, dW1, db1, dW2))
    for name, a, b in zip(("dX", "dW1", "db1", "dW2"), *outs):
        assert torch.equal(a, b), f"{name} differs from tp_mlp_bwd (T={T})"


def test_noalloc_matches_workspace_entry_point_twice():
    need_gpu()
    assert tl.tpmlp_noalloc_scratch_bytes() == 64 << 20
    # the first call fills most of the array (8192 x 1536 shard: about 25 MiB of dH and column sums)
    _case(8192, 1024, 3072, 2, seed=41)
    # the second, smaller one (ragged T, the last tile row partial) reuses it
    _case(1000, 256, 1024, 2, seed=42)


def test_noalloc_refuses_sizes_beyond_the_array():
    need_gpu()
    T, h, F, tp = 32768, 256, 2048, 1   # dH alone is 128 MiB
    need = tl.tpmlp_bwd_workspace_bytes(tl.BF16, T, h, F, tp)
    assert need > tl.tpmlp_noalloc_scratch_bytes()
    X, W1, W2 = empty((T, h), "bf16"), empty((h, F), "bf16"), empty((F, h), "bf16")
    H, A, dZ = empty((T, F), "bf16"), empty((T, F), "bf16"), empty((T, h), "bf16")
    dX, dW1, dW2 = empty_f32((T, h)), empty_f32((h, F)), empty_f32((F, h))
    dX.fill_(3.0)
    with pytest.raises(tl.TpmlpError) as e:
        tl.tp_mlp_bwd_noalloc(X, W1, W2, H, A, dZ, tp, dX, dW1, dW2)
    assert e.value.status == 7 and "static scratch" in e.value.message
    sync()
    assert torch.all(dX == 3.0).item(), "a refused call must not write its outputs"
