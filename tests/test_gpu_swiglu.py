"""GPU parity of the gated MLP (SwiGLU) entry points against the float64 oracle.

Small shapes with ragged tails run the whole oracle: every shard's packed
weight (bit-exact: it is a copy), forward outputs, backward outputs, the
unpacked weight gradients (bit-exact), and the sum of the forward partials
against the unsharded block.  The Qwen3-8B-sized shard (T=8192, h=4096,
F=12288, tp=8) is checked on sampled rows and columns.  Tolerance for bf16
storage: max|err| / max|ref| <= 2e-2.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from oracle import swiglu as sw
from tests.gpu_util import assert_close, empty, empty_f32, need_gpu, sync, to_dev, to_f64

pytestmark = pytest.mark.gpu

import linear_layers_amd as tl  # noqa: E402


def _say(msg):
    print(msg, flush=True)


def _inputs(T, h, F, seed):
    wl = synth.Workload("t", seed, "bf16", T=T, h=h, F=F, tp=1, x_std=1.0, w_std=0.05, dz_std=1.0, kind="swiglu")
    raw = synth.swiglu_inputs(wl)
    return raw, {k: synth.to_f64(v, "bf16") for k, v in raw.items()}


SHAPES = [
    # T, h, F, tp   (F/tp a multiple of 8; packed widths not multiples of the tiles)
    (300, 264, 640, 2),
    (513, 512, 2048, 4),
    (1, 16, 32, 2),
    (77, 136, 48, 3),
    (200, 96, 192, 8),     # F/tp = 24: a 32-column block with only its gate/up pair 0 in range
]


@pytest.mark.parametrize("T,h,F,tp", SHAPES)
def test_tp_swiglu_fwd_bwd(T, h, F, tp):
    need_gpu()
    _say(f"swiglu T={T} h={h} F={F} tp={tp}")
    raw, f = _inputs(T, h, F, seed=T + h)
    Fs = F // tp
    X, Wg, Wu, Wd, dZ = (to_dev(raw[k], "bf16") for k in ("X", "W_gate", "W_up", "W_down", "dZ"))
    Zp = empty_f32((tp, T, h))
    dXp = empty_f32((tp, T, h))
    for i in range(tp):
        W_gu = empty((h, 2 * Fs), "bf16")
        tl.swiglu_pack_shard(Wg, Wu, tp, i, W_gu)
        Wd_i = Wd[i * Fs:(i + 1) * Fs]
        GU, A = empty((T, 2 * Fs), "bf16"), empty((T, Fs), "bf16")
        tl.tp_swiglu_fwd(X, W_gu, Wd_i, tp, A, Zp[i], GU_save=GU)
        dW_gu, dW_down = empty_f32((h, 2 * Fs)), empty_f32((Fs, h))
        tl.tp_swiglu_bwd(X, W_gu, Wd_i, GU, A, dZ, tp, dXp[i], dW_gu, dW_down)
        dWg_full, dWu_full = torch.zeros((h, F), device="cuda"), torch.zeros((h, F), device="cuda")
        tl.swiglu_unpack_grad(dW_gu, tp, i, dWg_full, dWu_full)
        sync()
        # the packed weight is a copy: bit-exact
        assert np.array_equal(to_f64(W_gu), sw.pack_shard(f["W_gate"], f["W_up"], tp, i)), f"packed shard {i}"
        o = sw.tp_swiglu_fwd_shard(f["X"], f["W_gate"], f["W_up"], f["W_down"], tp, i)
        assert_close(to_f64(GU), o["GU"], "bf16", f"GU shard {i}")
        assert_close(to_f64(A), o["A"], "bf16", f"A shard {i}")
        assert_close(to_f64(Zp[i]), o["Z"], "bf16", f"Z shard {i}")
        b = sw.tp_swiglu_bwd_shard(f["X"], f["W_gate"], f["W_up"], f["W_down"], f["dZ"], tp, i)
        assert_close(to_f64(dXp[i]), b["dX"], "bf16", f"dX shard {i}")
        assert_close(to_f64(dW_gu), b["dW_gu"], "bf16", f"dW_gu shard {i}")
        assert_close(to_f64(dW_down), b["dW_down"], "bf16", f"dW_down shard {i}")
        # unpacking moves the packed gradient's columns without arithmetic: bit-exact
        g_dev, u_dev = sw.deinterleave(to_f64(dW_gu))
        ug, uu = to_f64(dWg_full), to_f64(dWu_full)
        assert np.array_equal(ug[:, i * Fs:(i + 1) * Fs], g_dev) and np.array_equal(uu[:, i * Fs:(i + 1) * Fs], u_dev)
        assert not ug[:, :i * Fs].any() and not ug[:, (i + 1) * Fs:].any()
    # sum of partials on the device against the unsharded block
    Z, dX = empty_f32((T, h)), empty_f32((T, h))
    tl.shard_partial_sum(Zp, Z)
    tl.shard_partial_sum(dXp, dX)
    sync()
    full = sw.swiglu_fwd(f["X"], f["W_gate"], f["W_up"], f["W_down"])
    assert_close(to_f64(Z), full["Z"], "bf16", "sum of Z partials")
    g = sw.swiglu_bwd(f["X"], f["W_gate"], f["W_up"], f["W_down"], f["dZ"])
    assert_close(to_f64(dX), g["dX"], "bf16", "sum of dX partials")


def test_swiglu_empty_batch_and_f32_refused():
    need_gpu()
    h, F, tp = 64, 128, 2
    Fs = F // tp
    W_gu = torch.zeros((h, 2 * Fs), dtype=torch.bfloat16, device="cuda")
    Wd = torch.zeros((Fs, h), dtype=torch.bfloat16, device="cuda")
    X = torch.zeros((0, h), dtype=torch.bfloat16, device="cuda")
    A = torch.zeros((0, Fs), dtype=torch.bfloat16, device="cuda")
    Z = torch.zeros((0, h), dtype=torch.float32, device="cuda")
    tl.tp_swiglu_fwd(X, W_gu, Wd, tp, A, Z)
    dW_gu, dW_down = empty_f32((h, 2 * Fs)), empty_f32((Fs, h))
    tl.tp_swiglu_bwd(X, W_gu, Wd, torch.zeros((0, 2 * Fs), dtype=torch.bfloat16, device="cuda"), A,
                     torch.zeros((0, h), dtype=torch.bfloat16, device="cuda"), tp, Z, dW_gu, dW_down)
    sync()
    assert not to_f64(dW_gu).any() and not to_f64(dW_down).any()
    with pytest.raises(tl.TpmlpError) as e:
        tl.tp_swiglu_fwd(X.float(), W_gu.float(), Wd.float(), tp, A.float(), Z)
    assert e.value.status == 5


def _pick(n, k, seed):
    r = np.random.default_rng(seed)
    idx = set(r.choice(n, size=min(k, n), replace=False).tolist()) | {0, n - 1}
    return np.array(sorted(idx))


@pytest.mark.slow
def test_qwen3_swiglu_shard_sampled():
    """T=8192, h=4096, F=12288, tp=8 (Qwen3-8B sizes): shard 0 fwd+bwd on sampled rows and columns."""
    need_gpu()
    wl = synth.WORKLOADS["qwen3_swiglu_bf16"]
    _say(f"workload {wl.name}")
    raw = synth.swiglu_inputs(wl)
    T, h, Fs, tp = wl.T, wl.h, wl.Fs, wl.tp
    X, dZ = to_dev(raw["X"], "bf16"), to_dev(raw["dZ"], "bf16")
    Wg, Wu = to_dev(raw["W_gate"], "bf16"), to_dev(raw["W_up"], "bf16")
    W_gu = empty((h, 2 * Fs), "bf16")
    tl.swiglu_pack_shard(Wg, Wu, tp, 0, W_gu)
    del Wg, Wu
    Wd0 = to_dev(raw["W_down"][:Fs], "bf16")
    GU, A, Z = empty((T, 2 * Fs), "bf16"), empty((T, Fs), "bf16"), empty_f32((T, h))
    tl.tp_swiglu_fwd(X, W_gu, Wd0, tp, A, Z, GU_save=GU)
    dX, dW_gu, dW_down = empty_f32((T, h)), empty_f32((h, 2 * Fs)), empty_f32((Fs, h))
    tl.tp_swiglu_bwd(X, W_gu, Wd0, GU, A, dZ, tp, dX, dW_gu, dW_down)
    sync()
    fX, fdZ = synth.to_f64(raw["X"], "bf16"), synth.to_f64(raw["dZ"], "bf16")
    fW_gu = sw.pack_shard(synth.to_f64(raw["W_gate"], "bf16"), synth.to_f64(raw["W_up"], "bf16"), tp, 0)
    fWd0 = synth.to_f64(raw["W_down"][:Fs], "bf16")
    rows, cols = _pick(T, 96, 61), _pick(Fs, 48, 62)
    ri = torch.as_tensor(rows, device="cuda")
    o = sw.shard_fwd_rows(fX, fW_gu, fWd0, rows)
    assert_close(to_f64(GU[ri]), o["GU"], "bf16", "GU rows")
    assert_close(to_f64(A[ri]), o["A"], "bf16", "A rows")
    assert_close(to_f64(Z[ri]), o["Z"], "bf16", "Z rows")
    ob = sw.shard_bwd_rows(fX, fW_gu, fWd0, fdZ, rows)
    assert_close(to_f64(dX[ri]), ob["dX"], "bf16", "dX rows")
    oc = sw.shard_bwd_cols(fX, fW_gu, fWd0, fdZ, cols)
    gc = torch.as_tensor(oc["gate_cols"], device="cuda")
    uc = torch.as_tensor(oc["up_cols"], device="cuda")
    assert_close(to_f64(dW_gu[:, gc]), oc["dW_gate_cols"], "bf16", "dW_gate cols")
    assert_close(to_f64(dW_gu[:, uc]), oc["dW_up_cols"], "bf16", "dW_up cols")
    assert_close(to_f64(dW_down[torch.as_tensor(cols, device="cuda")]), oc["dW_down_rows"], "bf16", "dW_down rows")
