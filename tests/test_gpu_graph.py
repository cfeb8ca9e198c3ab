"""The MLP entry points under HIP graph capture (torch.cuda.CUDAGraph on a side
stream): the library's launches record into the graph like any stream work
(no allocation, no memset node, no host synchronisation inside a call), and
each replay computes what the same calls compute eagerly.

Each case captures one step (forward, the partial sum of the output, backward,
the partial sum of dX), then three times overwrites the inputs in place with a
new seeded draw, replays, and compares every output bit for bit with an eager
run of the same calls on the same inputs (the kernels are deterministic, so a
replay that read a stale or wrong buffer would differ).  The eager path itself
is held to the oracle by the parity tests; one replay here is also compared
with the oracle at the bf16 bar.
"""
from __future__ import annotations

import pytest
import torch

import synth
from oracle import ref
from oracle import swiglu as sw
from tests.gpu_util import assert_close, empty, empty_f32, need_gpu, to_dev, to_f64

pytestmark = pytest.mark.gpu

import linear_layers_amd as tl  # noqa: E402


def _say(msg):
    print(msg, flush=True)


def _replays_match_eager(inputs, fresh, step, outputs, check_oracle):
    """Capture step() on a side stream, then per replay: refill inputs from
    fresh(r), replay, copy the outputs aside, run step() eagerly, compare."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(s)   # first use of every code path outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step(s)
    torch.cuda.synchronize()
    for r in range(3):
        new = fresh(r)
        for name, t in inputs.items():
            t.copy_(new[name])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = {k: v.clone() for k, v in outputs.items()}
        for v in outputs.values():
            v.fill_(float("nan"))
        torch.cuda.synchronize()
        step(torch.cuda.current_stream())
        torch.cuda.synchronize()
        for k in outputs:
            assert torch.equal(got[k], outputs[k]), f"replay {r}: {k} differs from the eager result"
        if r == 0:
            check_oracle(got)


@pytest.mark.parametrize("T,h,F,joined", [(700, 1000, 4000, "128x128 trio"), (3400, 4000, 4000, "256x256 trio")])
def test_mlp_step_in_a_graph(T, h, F, joined):
    """tp = 2 (shard 0 computed, shard 1's partials precomputed), bias; the backward's weight gradients
    and dX run as the joined launch named in the case."""
    need_gpu()
    tp = 2
    _say(f"graph mlp T={T} h={h} F={F} tp={tp} ({joined})")
    wl = synth.Workload("g", 51, "bf16", T=T, h=h, F=F, tp=tp, x_std=1.0, w_std=0.05, b_std=0.1, dz_std=1.0)
    raw = synth.mlp_inputs(wl)
    Fs = F // tp
    X, dZ = to_dev(raw["X"], "bf16"), to_dev(raw["dZ"], "bf16")
    W1 = to_dev(raw["W1"][:, :Fs].copy(), "bf16")
    W2 = to_dev(raw["W2"][:Fs].copy(), "bf16")
    b1 = to_dev(raw["b1"][:Fs].copy(), "bf16")
    A, H = empty((T, Fs), "bf16"), empty((T, Fs), "bf16")
    Zp, dXp = empty_f32((tp, T, h), 0.0), empty_f32((tp, T, h), 0.0)
    Zp[1].normal_()
    dXp[1].normal_()
    Zsum, dXsum = empty_f32((T, h)), empty_f32((T, h))
    dW1, dW2, db1 = empty_f32((h, Fs)), empty_f32((Fs, h)), empty_f32((Fs,))
    ws = torch.empty(tl.tpmlp_bwd_workspace_bytes(tl.BF16, T, h, F, tp), dtype=torch.uint8, device="cuda")

    def step(s):
        tl.tp_mlp_fwd(X, W1, b1, W2, tp, A, Zp[0], H_save=H, stream=s)
        tl.shard_partial_sum(Zp, Zsum, stream=s)
        tl.tp_mlp_bwd(X, W1, W2, H, A, dZ, tp, dXp[0], dW1, dW2, db1_shard=db1, workspace=ws, stream=s)
        tl.shard_partial_sum(dXp, dXsum, stream=s)

    def fresh(r):
        w = synth.Workload("g", 60 + r, "bf16", T=T, h=h, F=F, tp=tp, x_std=1.0, w_std=0.05, b_std=0.1,
                           dz_std=1.0)
        d = synth.mlp_inputs(w)
        return {"X": to_dev(d["X"], "bf16"), "dZ": to_dev(d["dZ"], "bf16")}

    def check_oracle(got):
        x, dz = to_f64(X), to_f64(dZ)
        w1, w2, b = to_f64(W1), to_f64(W2), to_f64(b1)
        o = ref.tp_mlp_fwd_shard(x, w1, b, w2, 1, 0)
        assert_close(to_f64(got["Zsum"]), o["Z"] + to_f64(Zp[1]), "bf16", "Z sum")
        gb = ref.tp_mlp_bwd_shard(x, w1, b, w2, dz, 1, 0)
        for k in ("dW1", "dW2", "db1"):
            assert_close(to_f64(got[k]), gb[k], "bf16", k)
        assert_close(to_f64(got["dXsum"]), gb["dX"] + to_f64(dXp[1]), "bf16", "dX sum")

    outputs = {"A": A, "H": H, "Zsum": Zsum, "dW1": dW1, "dW2": dW2, "db1": db1, "dXsum": dXsum}
    _replays_match_eager({"X": X, "dZ": dZ}, fresh, step, outputs, check_oracle)


def test_swiglu_step_in_a_graph():
    """The gated MLP, T = 8000, h = 136, F = 2000, tp = 1: its backward joins the down-projection
    weight gradient and dA in one launch."""
    need_gpu()
    T, h, F = 8000, 136, 2000
    _say(f"graph swiglu T={T} h={h} F={F}")
    wl = synth.Workload("g", 52, "bf16", T=T, h=h, F=F, tp=1, x_std=1.0, w_std=0.05, dz_std=1.0, kind="swiglu")
    raw = synth.swiglu_inputs(wl)
    X, Wg, Wu, Wd, dZ = (to_dev(raw[k], "bf16") for k in ("X", "W_gate", "W_up", "W_down", "dZ"))
    W_gu = empty((h, 2 * F), "bf16")
    tl.swiglu_pack_shard(Wg, Wu, 1, 0, W_gu)
    GU, A, Z = empty((T, 2 * F), "bf16"), empty((T, F), "bf16"), empty_f32((T, h))
    dX, dW_gu, dW_down = empty_f32((T, h)), empty_f32((h, 2 * F)), empty_f32((F, h))
    ws = torch.empty(tl.tp_swiglu_bwd_workspace_bytes(tl.BF16, T, h, F, 1), dtype=torch.uint8, device="cuda")

    def step(s):
        tl.tp_swiglu_fwd(X, W_gu, Wd, 1, A, Z, GU_save=GU, stream=s)
        tl.tp_swiglu_bwd(X, W_gu, Wd, GU, A, dZ, 1, dX, dW_gu, dW_down, workspace=ws, stream=s)

    def fresh(r):
        w = synth.Workload("g", 70 + r, "bf16", T=T, h=h, F=F, tp=1, x_std=1.0, w_std=0.05, dz_std=1.0,
                           kind="swiglu")
        d = synth.swiglu_inputs(w)
        return {"X": to_dev(d["X"], "bf16"), "dZ": to_dev(d["dZ"], "bf16")}

    def check_oracle(got):
        f = {"X": to_f64(X), "dZ": to_f64(dZ), "W_gate": synth.to_f64(raw["W_gate"], "bf16"),
             "W_up": synth.to_f64(raw["W_up"], "bf16"), "W_down": synth.to_f64(raw["W_down"], "bf16")}
        o = sw.tp_swiglu_fwd_shard(f["X"], f["W_gate"], f["W_up"], f["W_down"], 1, 0)
        assert_close(to_f64(got["Z"]), o["Z"], "bf16", "Z")
        b = sw.tp_swiglu_bwd_shard(f["X"], f["W_gate"], f["W_up"], f["W_down"], f["dZ"], 1, 0)
        for k, name in (("dX", "dX"), ("dW_gu", "dW_gu"), ("dW_down", "dW_down")):
            assert_close(to_f64(got[k]), b[name], "bf16", name)

    outputs = {"A": A, "GU": GU, "Z": Z, "dX": dX, "dW_gu": dW_gu, "dW_down": dW_down}
    _replays_match_eager({"X": X, "dZ": dZ}, fresh, step, outputs, check_oracle)
