"""The library's entry points under HIP graph capture (torch.cuda.CUDAGraph on
a side stream): the MLP, the gated MLP, the head-sharded attention block and
one rank's step of the sequence-parallel MLP.  The launches record into the
graph like any stream work (no allocation, no memset node, no host
synchronisation inside a call), and each replay computes what the same calls
compute eagerly.

Each case captures one step (forward, the partial sum of the output, backward,
the partial sum of dX), then three times overwrites the inputs in place with a
new seeded draw, replays, and compares every output bit for bit with an eager
run of the same calls on the same inputs (the kernels are deterministic, so a
replay that read a stale or wrong buffer would differ).  The eager path itself
is held to the oracle by the parity tests; for the MLP, the gated MLP and the
attention block one replay here is also compared with the oracle at the bf16
bar.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from oracle import attn as oat
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


def test_attn_block_step_in_a_graph():
    """The head-sharded attention block, forward and backward: one causal sequence of 2500 tokens,
    4 heads of 128 (h = 512), tp = 2, shard 1.  Query blocks past key 2048 split their keys into two
    chunks, so the chunk merge runs in the graph too."""
    need_gpu()
    batch, seq, heads, tp, shard, D = 1, 2500, 4, 2, 1, 128
    T, h = batch * seq, heads * D
    hs, w = heads // tp, heads // tp * D
    _say(f"graph attention block T={T} heads={heads} tp={tp}")
    r = np.random.default_rng(77)
    Wf = {n: synth.bf16_round_bits((r.standard_normal((h, h)) / np.sqrt(h)).astype(np.float32))
          for n in ("Wq", "Wk", "Wv", "Wo")}
    c = slice(shard * w, (shard + 1) * w)
    Wqkv = to_dev(np.ascontiguousarray(np.concatenate([Wf[n][:, c] for n in ("Wq", "Wk", "Wv")], axis=1)), "bf16")
    Wo = to_dev(np.ascontiguousarray(Wf["Wo"][c]), "bf16")

    def draw(seed):
        q = np.random.default_rng(seed)
        return {"X": to_dev(synth.bf16_round_bits(q.standard_normal((T, h)).astype(np.float32)), "bf16"),
                "dZ": to_dev(synth.bf16_round_bits(q.standard_normal((T, h)).astype(np.float32)), "bf16")}

    first = draw(80)
    X, dZ = first["X"], first["dZ"]
    QKV, O, lse = empty((T, 3 * w), "bf16"), empty((T, w), "bf16"), empty_f32((hs, T))
    Z, dX, dWqkv, dWo = empty_f32((T, h)), empty_f32((T, h)), empty_f32((h, 3 * w)), empty_f32((w, h))
    wsf = torch.empty(max(1, tl.tp_attn_fwd_workspace_bytes(batch, seq, heads, tp)), dtype=torch.uint8, device="cuda")
    wsb = torch.empty(tl.tp_attn_bwd_workspace_bytes(batch, seq, heads, tp), dtype=torch.uint8, device="cuda")

    def step(s):
        tl.tp_attn_fwd(X, Wqkv, Wo, QKV, O, lse, Z, batch, seq, heads, tp, causal=True, workspace=wsf, stream=s)
        tl.tp_attn_bwd(X, Wqkv, Wo, QKV, O, lse, dZ, dX, dWqkv, dWo, batch, seq, heads, tp, causal=True,
                       workspace=wsb, stream=s)

    def check_oracle(got):
        f = {k: synth.to_f64(v, "bf16") for k, v in Wf.items()}
        want = oat.tp_attn_block_bwd_shard(to_f64(X), f["Wq"], f["Wk"], f["Wv"], f["Wo"], to_f64(dZ), batch, seq,
                                           heads, D, tp, shard, True, D ** -0.5)
        for k in ("QKV", "O", "Z", "dX", "dWqkv", "dWo"):
            assert_close(to_f64(got[k]), want[k], "bf16", k)

    outputs = {"QKV": QKV, "O": O, "lse": lse, "Z": Z, "dX": dX, "dWqkv": dWqkv, "dWo": dWo}
    _replays_match_eager({"X": X, "dZ": dZ}, lambda rr: draw(81 + rr), step, outputs, check_oracle)


def test_sp_rank_step_in_a_graph():
    """Rank 0's step of the MLP inside the sequence-parallel region, tp = 2: LayerNorm of its rows into
    its block of the gathered input, shard 0's MLP forward, its rows of the partial sum with dropout
    and the residual, dropout' into its block of the gathered gradient, the shard's backward, its rows
    of the dX partial sum, and LayerNorm backward with the residual gradient.  (The other rank's
    blocks and shard 1's partials are filled once, outside the graph; the eager chain is held to the
    oracle by test_gpu_sp.py, so the replays are compared with it.)"""
    need_gpu()
    T, h, F, tp, p, seed = 512, 256, 1024, 2, 0.1, 99
    rows, Fs = T // tp, F // tp
    _say(f"graph sp step T={T} h={h} F={F} tp={tp}")
    wl = synth.Workload("g", 53, "bf16", T=T, h=h, F=F, tp=1, x_std=1.0, w_std=0.05, b_std=0.1, dz_std=1.0)
    raw = synth.mlp_inputs(wl)
    r = np.random.default_rng(6)
    gam = torch.from_numpy((1.0 + 0.1 * r.standard_normal(h)).astype(np.float32)).cuda()
    bet = torch.from_numpy((0.1 * r.standard_normal(h)).astype(np.float32)).cuda()
    X, dOut = to_dev(raw["X"], "bf16"), to_dev(raw["dZ"], "bf16")
    W1 = [to_dev(np.ascontiguousarray(raw["W1"][:, j * Fs:(j + 1) * Fs]), "bf16") for j in range(tp)]
    W2 = [to_dev(np.ascontiguousarray(raw["W2"][j * Fs:(j + 1) * Fs]), "bf16") for j in range(tp)]
    b1 = [to_dev(raw["b1"][j * Fs:(j + 1) * Fs].copy(), "bf16") for j in range(tp)]
    Yg, dZg = empty((T, h), "bf16"), empty((T, h), "bf16")
    mean, rstd = empty_f32((T,)), empty_f32((T,))
    A, H = empty((T, Fs), "bf16"), empty((T, Fs), "bf16")
    Zp, dXp = empty_f32((tp, T, h)), empty_f32((tp, T, h))
    out, dY, dX = empty((rows, h), "bf16"), empty_f32((rows, h)), empty_f32((rows, h))
    dW1, dW2, db1 = empty_f32((h, Fs)), empty_f32((Fs, h)), empty_f32((Fs,))
    dgam, dbet = empty_f32((h,)), empty_f32((h,))
    ws = torch.empty(tl.tpmlp_bwd_workspace_bytes(tl.BF16, T, h, F, tp), dtype=torch.uint8, device="cuda")
    r0 = slice(0, rows)
    # rank 1's gathered blocks and shard 1's partials, once
    tl.layernorm_fwd(X[rows:], gam, bet, Yg[rows:], mean[rows:], rstd[rows:])
    tl.sp_dropout_bwd(dOut[rows:], dZg[rows:], p, seed, rows)

    def shard1():
        A1, H1 = empty((T, Fs), "bf16"), empty((T, Fs), "bf16")
        tl.layernorm_fwd(X[r0], gam, bet, Yg[r0], mean[r0], rstd[r0])
        tl.sp_dropout_bwd(dOut[r0], dZg[r0], p, seed, 0)
        tl.tp_mlp_fwd(Yg, W1[1], b1[1], W2[1], tp, A1, Zp[1], H_save=H1)
        d1, d2 = empty_f32((h, Fs)), empty_f32((Fs, h))
        tl.tp_mlp_bwd(Yg, W1[1], W2[1], H1, A1, dZg, tp, dXp[1], d1, d2, workspace=ws)

    shard1()
    torch.cuda.synchronize()

    def step(s):
        tl.layernorm_fwd(X[r0], gam, bet, Yg[r0], mean[r0], rstd[r0], stream=s)
        tl.tp_mlp_fwd(Yg, W1[0], b1[0], W2[0], tp, A, Zp[0], H_save=H, stream=s)
        tl.sp_partial_sum_dropout_residual(Zp[:, r0], X[r0], out, p, seed, 0, stream=s)
        tl.sp_dropout_bwd(dOut[r0], dZg[r0], p, seed, 0, stream=s)
        tl.tp_mlp_bwd(Yg, W1[0], W2[0], H, A, dZg, tp, dXp[0], dW1, dW2, db1_shard=db1, workspace=ws, stream=s)
        tl.shard_partial_sum(dXp[:, r0], dY, stream=s)
        tl.layernorm_bwd(X[r0], gam, mean[r0], rstd[r0], dY, dX, dgamma=dgam, dbeta=dbet, dRes=dOut[r0], stream=s)

    def fresh(rr):
        # new rows for rank 0 (its input and upstream gradient); rank 1's blocks stay
        q = np.random.default_rng(90 + rr)
        x = X.clone()
        x[r0] = to_dev(synth.bf16_round_bits(q.standard_normal((rows, h)).astype(np.float32)), "bf16")
        d = dOut.clone()
        d[r0] = to_dev(synth.bf16_round_bits(q.standard_normal((rows, h)).astype(np.float32)), "bf16")
        return {"X": x, "dOut": d}

    # rank 0's rows of the gathered buffers only: rank 1's rows are inputs of the step
    outputs = {"Yg rank 0": Yg[r0], "A": A, "H": H, "out": out, "dZg rank 0": dZg[r0], "dW1": dW1, "dW2": dW2,
               "db1": db1, "dY": dY, "dX": dX, "dgamma": dgam, "dbeta": dbet}
    _replays_match_eager({"X": X, "dOut": dOut}, fresh, step, outputs, lambda got: None)
