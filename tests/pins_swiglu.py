"""Checks that pin the float64 gated-MLP oracle (oracle.swiglu) to things
other than itself.

Each ``pin_*`` takes the oracle module (or a planted mutant of it) and raises
when the oracle disagrees with:
  * torch's float64 SiLU and its autograd derivative,
  * closed forms: silu(0) = 0, silu'(0) = 1/2, silu(x) - silu(-x) = x,
    sigmoid(-x) = 1 - sigmoid(x),
  * the storage order written out index by index,
  * pure-Python loops of the page's four-line listing,
  * the unsharded definition (the block must not depend on tp_size),
  * torch float64 autograd through the unsharded block,
  * central finite differences.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import brute
from oracle import ref as mlp_ref


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, rtol, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    scale = max(1e-300, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= rtol * scale, f"{what}: max err {err:.3e} > {rtol:.1e} * {scale:.3e}"


def _block(seed, T, h, F, w=0.3):
    r = _rng(seed)
    return (r.standard_normal((T, h)), w * r.standard_normal((h, F)), w * r.standard_normal((h, F)),
            w * r.standard_normal((F, h)), r.standard_normal((T, h)))


def pin_silu_closed_forms(sw):
    assert sw.silu(np.array([0.0]))[0] == 0.0
    assert abs(sw.silu_grad(np.array([0.0]))[0] - 0.5) < 1e-15
    x = np.concatenate([_rng(1).standard_normal(200) * 6.0, [-800.0, -40.0, 40.0, 800.0]])
    _close(sw.silu(x) - sw.silu(-x), x, 1e-14, "silu(x) - silu(-x) = x")
    _close(sw.sigmoid(-x), 1.0 - sw.sigmoid(x), 1e-14, "sigmoid symmetry")
    _close(sw.silu(np.array([800.0, -800.0])), np.array([800.0, 0.0]), 1e-15, "silu saturation")


def pin_silu_vs_torch(sw):
    x = torch.tensor(np.concatenate([_rng(2).standard_normal(500) * 5.0, [-30.0, 30.0]]), dtype=torch.float64,
                     requires_grad=True)
    y = torch.nn.functional.silu(x)
    (g,) = torch.autograd.grad(y.sum(), x)
    xs = x.detach().numpy()
    _close(sw.silu(xs), y.detach().numpy(), 1e-14, "silu")
    _close(sw.silu_grad(xs), g.numpy(), 1e-13, "silu'")


def pin_silu_grad_differences(sw):
    x = np.linspace(-8.0, 8.0, 161)
    e = 1e-6
    fd = (sw.silu(x + e) - sw.silu(x - e)) / (2 * e)
    _close(sw.silu_grad(x), fd, 1e-8, "silu' by differences")


def pin_storage_order(sw):
    r = _rng(3)
    T, Fs = 3, 24
    G, U = r.standard_normal((T, Fs)), r.standard_normal((T, Fs))
    P = sw.interleave(G, U)
    assert P.shape == (T, 2 * Fs)
    for t in range(T):
        for c in range(2 * Fs):
            q, rr = divmod(c, 16)
            want = G[t, 8 * q + rr] if rr < 8 else U[t, 8 * q + rr - 8]
            assert P[t, c] == want, (t, c)
    g2, u2 = sw.deinterleave(P)
    assert np.array_equal(g2, G) and np.array_equal(u2, U)
    # the packed shard holds shard i's columns of both weights
    h, F, tp = 4, 48, 2
    Wg, Wu = r.standard_normal((h, F)), r.standard_normal((h, F))
    for i in range(tp):
        g3, u3 = sw.deinterleave(sw.pack_shard(Wg, Wu, tp, i))
        assert np.array_equal(g3, Wg[:, 24 * i:24 * (i + 1)]) and np.array_equal(u3, Wu[:, 24 * i:24 * (i + 1)])
    try:
        sw.interleave(np.zeros((1, 12)), np.zeros((1, 12)))
    except ValueError:
        pass
    else:
        raise AssertionError("a shard width that is not a multiple of 8 must be refused")


def pin_brute_force(sw):
    X, Wg, Wu, Wd, _ = _block(4, 3, 5, 16)
    G, U, A, Z = brute.swiglu_fwd(X, Wg, Wu, Wd)
    f = sw.swiglu_fwd(X, Wg, Wu, Wd)
    _close(f["G"], G, 1e-13, "gate")
    _close(f["U"], U, 1e-13, "up")
    _close(f["A"], A, 1e-13, "silu(gate) * up")
    _close(f["Z"], Z, 1e-13, "down")


def pin_tp_invariance(sw):
    X, Wg, Wu, Wd, _ = _block(5, 7, 12, 64)
    f = sw.swiglu_fwd(X, Wg, Wu, Wd)
    for tp in (1, 2, 4, 8):
        _close(sw.tp_swiglu_fwd(X, Wg, Wu, Wd, tp), f["Z"], 1e-12, f"tp={tp} sum of partials")
        Fs = 64 // tp
        for i in range(tp):
            s = sw.tp_swiglu_fwd_shard(X, Wg, Wu, Wd, tp, i)
            _close(s["A"], f["A"][:, i * Fs:(i + 1) * Fs], 1e-13, f"tp={tp} shard {i} activation")
    try:
        sw.tp_swiglu_fwd(X, Wg, Wu, Wd, 3)
    except ValueError:
        pass
    else:
        raise AssertionError("F=64 over tp=3 must be refused")


def _torch_grads(X, Wg, Wu, Wd, dZ):
    t = [torch.tensor(m, dtype=torch.float64, requires_grad=True) for m in (X, Wg, Wu, Wd)]
    Z = (torch.nn.functional.silu(t[0] @ t[1]) * (t[0] @ t[2])) @ t[3]
    gs = torch.autograd.grad((Z * torch.tensor(dZ, dtype=torch.float64)).sum(), t)
    return [g.numpy() for g in gs]


def pin_autograd(sw):
    X, Wg, Wu, Wd, dZ = _block(6, 9, 16, 64)
    dX, dWg, dWu, dWd = _torch_grads(X, Wg, Wu, Wd, dZ)
    g = sw.swiglu_bwd(X, Wg, Wu, Wd, dZ)
    _close(g["dX"], dX, 1e-12, "dX")
    _close(g["dW_gate"], dWg, 1e-12, "dW_gate")
    _close(g["dW_up"], dWu, 1e-12, "dW_up")
    _close(g["dW_down"], dWd, 1e-12, "dW_down")
    for tp in (2, 4):
        Fs = 64 // tp
        parts = [sw.tp_swiglu_bwd_shard(X, Wg, Wu, Wd, dZ, tp, i) for i in range(tp)]
        _close(mlp_ref.shard_partial_sum([p["dX"] for p in parts]), dX, 1e-12, f"tp={tp} dX")
        for i, p in enumerate(parts):
            gg, gu = sw.unpack_grad_shard(p["dW_gu"], 64, tp, i)
            _close(gg[:, i * Fs:(i + 1) * Fs], dWg[:, i * Fs:(i + 1) * Fs], 1e-12, f"dW_gate shard {i}")
            _close(gu[:, i * Fs:(i + 1) * Fs], dWu[:, i * Fs:(i + 1) * Fs], 1e-12, f"dW_up shard {i}")
            _close(p["dW_down"], dWd[i * Fs:(i + 1) * Fs], 1e-12, f"dW_down shard {i}")


def pin_finite_differences(sw):
    X, Wg, Wu, Wd, dZ = _block(7, 2, 3, 8, w=0.5)
    fd = brute.swiglu_bwd_by_differences(X, Wg, Wu, Wd, dZ)
    g = sw.swiglu_bwd(X, Wg, Wu, Wd, dZ)
    for k in ("dX", "dW_gate", "dW_up", "dW_down"):
        _close(g[k], fd[k], 1e-7, f"{k} by differences")


def pin_sampled_views(sw):
    """The sampled row and column views agree with the whole shard."""
    X, Wg, Wu, Wd, dZ = _block(8, 11, 16, 64)
    tp, i = 2, 1
    W_gu = sw.pack_shard(Wg, Wu, tp, i)
    Wd_i = Wd[32:64]
    f = sw.tp_swiglu_fwd_shard(X, Wg, Wu, Wd, tp, i)
    b = sw.tp_swiglu_bwd_shard(X, Wg, Wu, Wd, dZ, tp, i)
    rows = [0, 3, 10]
    fr = sw.shard_fwd_rows(X, W_gu, Wd_i, rows)
    for k in ("GU", "A", "Z"):
        _close(fr[k], f[k][rows], 1e-13, f"rows {k}")
    br = sw.shard_bwd_rows(X, W_gu, Wd_i, dZ, rows)
    _close(br["dGU"], b["dGU"][rows], 1e-13, "rows dGU")
    _close(br["dX"], b["dX"][rows], 1e-13, "rows dX")
    cols = [0, 7, 8, 19, 31]
    bc = sw.shard_bwd_cols(X, W_gu, Wd_i, dZ, cols)
    _close(bc["dW_gate_cols"], b["dW_gu"][:, bc["gate_cols"]], 1e-13, "cols dW_gate")
    _close(bc["dW_up_cols"], b["dW_gu"][:, bc["up_cols"]], 1e-13, "cols dW_up")
    _close(bc["dW_down_rows"], b["dW_down"][cols], 1e-13, "cols dW_down")


ALL_PINS = [pin_silu_closed_forms, pin_silu_vs_torch, pin_silu_grad_differences, pin_storage_order,
            pin_brute_force, pin_tp_invariance, pin_autograd, pin_finite_differences, pin_sampled_views]
