"""Checks that pin the float64 oracle to things other than itself.

Each ``pin_*`` function takes an oracle module (``oracle.ref`` or a planted
mutant of it) and raises AssertionError (or any exception) when the oracle
disagrees with:
  * a hand-worked integer example of the block splits (tests/golden),
  * torch's float64 GeLU (tanh form) and its autograd derivative,
  * the exact GeLU x*Phi(x), within the tanh approximation's known error,
  * pure-Python brute-force loops,
  * central finite differences,
  * torch float64 autograd through the whole block,
  * the identities the pages state: column shards concatenate to XW, row
    partials sum to XW, the block does not depend on tp_size, every row
    shard sees the same upstream gradient.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

from oracle import brute

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, rtol, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    scale = max(1e-300, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= rtol * scale, f"{what}: max err {err:.3e} > {rtol:.1e} * {scale:.3e}"


def _frac_matmul(A, B):
    return [[sum((Fraction(A[r][t]) * Fraction(B[t][c]) for t in range(len(B))), Fraction(0))
             for c in range(len(B[0]))] for r in range(len(A))]


def load_example():
    with open(os.path.join(GOLDEN, "block_split_example.json")) as f:
        ex = json.load(f)
    # Re-derive the hand-worked values with exact rational loops first.
    X, W, dY = ex["X"], ex["W"], ex["dY"]
    assert _frac_matmul(X, W) == [[Fraction(v) for v in r] for r in ex["Y"]]
    WT = [list(c) for c in zip(*W)]
    XT = [list(c) for c in zip(*X)]
    assert _frac_matmul(dY, WT) == [[Fraction(v) for v in r] for r in ex["dX"]]
    assert _frac_matmul(XT, dY) == [[Fraction(v) for v in r] for r in ex["dW"]]
    assert [sum(c) for c in zip(*dY)] == ex["db"]
    return {k: (np.array(v, dtype=np.float64) if isinstance(v, list) else v) for k, v in ex.items()}


# ---------------------------------------------------------------- pins ----
def pin_worked_example(ref):
    ex = load_example()
    X, W, tp = ex["X"], ex["W"], ex["tp"]
    for i in range(tp):
        H, Y = ref.column_parallel_fwd(X, W, None, tp, i, ref.ACT_NONE)
        assert np.array_equal(Y, ex["Y_col_shards"][i]), f"column shard {i}"
        assert np.array_equal(H, ex["Y_col_shards"][i])
        assert np.array_equal(ref.row_parallel_fwd(X, W, tp, i), ex["Z_row_partials"][i]), f"row shard {i}"
    Z = ref.shard_partial_sum([ref.row_parallel_fwd(X, W, tp, i) for i in range(tp)])
    assert np.array_equal(Z, ex["Y"])
    g = ref.column_parallel_bwd(X, W, ex["dY"], with_bias=True)
    assert np.array_equal(g["dX"], ex["dX"]) and np.array_equal(g["dW"], ex["dW"])
    assert np.array_equal(g["db"], ex["db"])
    r = ref.row_parallel_bwd(X, W, ex["dY"])
    assert np.array_equal(r["dX"], ex["dX"]) and np.array_equal(r["dW"], ex["dW"])
    # Column-split backward over shards: dX is the sum, dW the concatenation.
    parts = [ref.column_parallel_bwd(X, ref.col_shard(W, tp, i), ref.col_shard(ex["dY"], tp, i), True)
             for i in range(tp)]
    assert np.array_equal(ref.shard_partial_sum([p["dX"] for p in parts]), ex["dX"])
    assert np.array_equal(np.concatenate([p["dW"] for p in parts], axis=1), ex["dW"])
    assert np.array_equal(np.concatenate([p["db"] for p in parts]), ex["db"])


def pin_gelu_vs_torch(ref):
    import torch
    x = np.concatenate([np.linspace(-12, 12, 2401), _rng(7).standard_normal(2000) * 3])
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    y = torch.nn.functional.gelu(xt, approximate="tanh")
    (g,) = torch.autograd.grad(y.sum(), xt)
    _close(ref.gelu_tanh(x), y.detach().numpy(), 1e-14, "gelu vs torch")
    _close(ref.gelu_tanh_grad(x), g.numpy(), 1e-13, "gelu' vs torch autograd")


def pin_gelu_exact_form(ref):
    """tanh GeLU stays within its known distance of x*Phi(x); odd-part identity; limits."""
    x = np.linspace(-8, 8, 3201)
    exact = np.array([v * 0.5 * (1.0 + math.erf(v / math.sqrt(2.0))) for v in x])
    d = np.max(np.abs(ref.gelu_tanh(x) - exact))
    assert 1e-5 < d < 5e-4, f"tanh GeLU deviates {d:.2e} from x*Phi(x)"
    g = ref.gelu_tanh(x)
    _close(g - ref.gelu_tanh(-x), x, 1e-15, "gelu(x) - gelu(-x) = x")
    assert abs(ref.gelu_tanh(np.array([0.0]))[0]) == 0.0
    assert abs(ref.gelu_tanh_grad(np.array([0.0]))[0] - 0.5) < 1e-15
    big = np.array([30.0, 50.0])
    _close(ref.gelu_tanh(big), big, 1e-15, "gelu -> x")
    assert np.all(np.abs(ref.gelu_tanh(-big)) < 1e-300 + 1e-12)
    # derivative against central differences of gelu itself
    e = 1e-6
    fd = (ref.gelu_tanh(x + e) - ref.gelu_tanh(x - e)) / (2 * e)
    _close(ref.gelu_tanh_grad(x), fd, 1e-8, "gelu' vs differences")


def _tiny(seed, T=3, h=5, F=8, bias=True):
    r = _rng(seed)
    X = r.standard_normal((T, h))
    W1 = r.standard_normal((h, F)) * 0.7
    b1 = r.standard_normal(F) * 0.3 if bias else None
    W2 = r.standard_normal((F, h)) * 0.7
    dZ = r.standard_normal((T, h))
    return X, W1, b1, W2, dZ


def pin_brute_forward(ref):
    for seed in (1, 2):
        X, W1, b1, W2, _ = _tiny(seed)
        H, A, Z = brute.mlp_fwd(X, W1, list(b1), W2)
        f = ref.mlp_fwd(X, W1, b1, W2)
        _close(f["H"], H, 1e-13, "H vs loops")
        _close(f["A"], A, 1e-13, "A vs loops")
        _close(f["Z"], Z, 1e-13, "Z vs loops")
        for tp in (1, 2, 4):
            for i in range(tp):
                s = ref.tp_mlp_fwd_shard(X, W1, b1, W2, tp, i)
                Fs = W1.shape[1] // tp
                _close(s["A"], np.array(A)[:, i * Fs:(i + 1) * Fs], 1e-13, "A_i vs loops")
                Zi = brute.matmul(brute.to_lists(np.array(A)[:, i * Fs:(i + 1) * Fs]),
                                  brute.to_lists(W2[i * Fs:(i + 1) * Fs]))
                _close(s["Z"], Zi, 1e-13, "Z_i vs loops")


def pin_split_identities(ref):
    r = _rng(11)
    X = r.standard_normal((6, 16))
    W = r.standard_normal((16, 24))
    full = X @ W  # library routine
    for tp in (1, 2, 4, 8):
        cols = np.concatenate([ref.column_parallel_fwd(X, W, None, tp, i, ref.ACT_NONE)[1] for i in range(tp)], axis=1)
        _close(cols, full, 1e-14, f"column concat tp={tp}")
        _close(ref.shard_partial_sum([ref.row_parallel_fwd(X, W, tp, i) for i in range(tp)]), full, 1e-13,
               f"row sum tp={tp}")
    X, W1, b1, W2, _ = _tiny(3, T=7, h=16, F=32)
    Z1 = ref.mlp_fwd(X, W1, b1, W2)["Z"]
    for tp in (1, 2, 4, 8):
        _close(ref.tp_mlp_fwd(X, W1, b1, W2, tp), Z1, 1e-13, f"tp invariance tp={tp}")
    # Activation is elementwise, so it commutes with the column split.
    H = ref.mlp_fwd(X, W1, b1, W2)["H"]
    for i in range(4):
        assert np.array_equal(ref.gelu_tanh(H)[:, i * 8:(i + 1) * 8], ref.gelu_tanh(H[:, i * 8:(i + 1) * 8]))
    # No activation and no bias: the block is X (W1 W2).
    _close(ref.tp_mlp_fwd(X, W1, None, W2, 4, ref.ACT_NONE), X @ (W1 @ W2), 1e-13, "linear special case")


def pin_backward_autograd(ref):
    import torch
    for seed, (T, h, F) in ((4, (3, 5, 8)), (5, (9, 6, 12))):
        X, W1, b1, W2, dZ = _tiny(seed, T, h, F)
        t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True)
             for k, v in (("X", X), ("W1", W1), ("b1", b1), ("W2", W2))}
        Z = torch.nn.functional.gelu(t["X"] @ t["W1"] + t["b1"], approximate="tanh") @ t["W2"]
        grads = torch.autograd.grad((Z * torch.tensor(dZ)).sum(), [t["X"], t["W1"], t["b1"], t["W2"]])
        g = ref.mlp_bwd(X, W1, b1, W2, dZ)
        for name, tg in zip(("dX", "dW1", "db1", "dW2"), grads):
            _close(g[name], tg.numpy(), 1e-13, f"{name} vs autograd")


def pin_backward_differences(ref):
    X, W1, b1, W2, dZ = _tiny(6, 3, 5, 8)
    fd = brute.mlp_bwd_by_differences(X, W1, list(b1), W2, dZ, step=1e-6)
    g = ref.mlp_bwd(X, W1, b1, W2, dZ)
    for name in ("dX", "dW1", "db1", "dW2"):
        _close(g[name], fd[name], 1e-7, f"{name} vs differences")


def pin_backward_shards(ref):
    X, W1, b1, W2, dZ = _tiny(8, 7, 12, 16)
    full = ref.mlp_bwd(X, W1, b1, W2, dZ)
    for tp in (1, 2, 4):
        s = [ref.tp_mlp_bwd_shard(X, W1, b1, W2, dZ, tp, i) for i in range(tp)]
        _close(ref.shard_partial_sum([p["dX"] for p in s]), full["dX"], 1e-13, f"sum dX_i tp={tp}")
        _close(np.concatenate([p["dW1"] for p in s], axis=1), full["dW1"], 1e-13, "dW1 concat")
        _close(np.concatenate([p["db1"] for p in s]), full["db1"], 1e-13, "db1 concat")
        _close(np.concatenate([p["dW2"] for p in s], axis=0), full["dW2"], 1e-13, "dW2 stack")
        _close(np.concatenate([p["dH"] for p in s], axis=1), full["dH"], 1e-13, "dH concat")
    # Each layer on its own: column-parallel backward with the activation's
    # gradient applied, and row-parallel backward with the same dZ everywhere.
    tp = 2
    for i in range(tp):
        s = ref.tp_mlp_bwd_shard(X, W1, b1, W2, dZ, tp, i)
        f = ref.tp_mlp_fwd_shard(X, W1, b1, W2, tp, i)
        rb = ref.row_parallel_bwd(f["A"], ref.row_shard(W2, tp, i), dZ)
        _close(rb["dW"], s["dW2"], 1e-13, "row bwd dW")
        _close(rb["dX"], s["dA"], 1e-13, "row bwd dX")
        cb = ref.column_parallel_bwd(X, ref.col_shard(W1, tp, i), s["dH"], with_bias=True)
        _close(cb["dX"], s["dX"], 1e-13, "col bwd dX")
        _close(cb["dW"], s["dW1"], 1e-13, "col bwd dW")
        _close(cb["db"], s["db1"], 1e-13, "col bwd db")


def pin_sampled(ref):
    X, W1, b1, W2, dZ = _tiny(9, 10, 8, 16)
    tp, i = 2, 1
    W1_i, b1_i, W2_i = ref.col_shard(W1, tp, i), ref.vec_shard(b1, tp, i), ref.row_shard(W2, tp, i)
    f = ref.tp_mlp_fwd_shard(X, W1, b1, W2, tp, i)
    b = ref.tp_mlp_bwd_shard(X, W1, b1, W2, dZ, tp, i)
    rows = np.array([0, 3, 9])
    fr = ref.tp_mlp_fwd_shard_rows(X, W1_i, b1_i, W2_i, rows)
    for k in ("H", "A", "Z"):
        _close(fr[k], f[k][rows], 1e-14, f"sampled fwd {k}")
    cols = np.array([1, 5, 7])
    bc = ref.tp_mlp_bwd_shard_cols(X, W1_i, b1_i, W2_i, dZ, cols)
    _close(bc["dH"], b["dH"][:, cols], 1e-14, "sampled dH cols")
    _close(bc["db1"], b["db1"][cols], 1e-14, "sampled db1")
    _close(bc["dW1"], b["dW1"][:, cols], 1e-14, "sampled dW1")
    _close(bc["dW2"], b["dW2"][cols, :], 1e-14, "sampled dW2")
    br = ref.tp_mlp_bwd_shard_rows(X, W1_i, b1_i, W2_i, dZ, rows)
    _close(br["dH"], b["dH"][rows], 1e-14, "sampled dH rows")
    _close(br["dX"], b["dX"][rows], 1e-14, "sampled dX rows")


def pin_projections(ref):
    r = _rng(12)
    heads, hd, tp = 4, 3, 2
    h = heads * hd
    X = r.standard_normal((5, h))
    Wq, Wk, Wv, Wo = (r.standard_normal((h, h)) for _ in range(4))
    O_in = r.standard_normal((5, h))
    for i in range(tp):
        P = ref.qkv_fwd_shard(X, Wq, Wk, Wv, heads, hd, tp, i)
        c0, c1 = i * (h // tp), (i + 1) * (h // tp)
        _close(P[:, :h // tp], (X @ Wq)[:, c0:c1], 1e-13, "Q heads")
        _close(P[:, h // tp:2 * h // tp], (X @ Wk)[:, c0:c1], 1e-13, "K heads")
        _close(P[:, 2 * h // tp:], (X @ Wv)[:, c0:c1], 1e-13, "V heads")
    _close(ref.shard_partial_sum([ref.out_proj_fwd_shard(O_in, Wo, heads, hd, tp, i) for i in range(tp)]),
           O_in @ Wo, 1e-13, "O projection partials")
    try:
        ref.qkv_shard_weight(Wq, Wk, Wv, heads, hd, 3, 0)
    except ValueError:
        pass
    else:
        raise AssertionError("heads not divisible by tp must be refused")


def pin_divisibility(ref):
    W = np.zeros((6, 10))
    for bad in (lambda: ref.col_shard(W, 4, 0), lambda: ref.row_shard(W, 4, 0), lambda: ref.col_shard(W, 0, 0)):
        try:
            bad()
        except ValueError:
            continue
        raise AssertionError("indivisible split accepted")


ALL_PINS = [pin_worked_example, pin_gelu_vs_torch, pin_gelu_exact_form, pin_brute_forward,
            pin_split_identities, pin_backward_autograd, pin_backward_differences,
            pin_backward_shards, pin_sampled, pin_projections, pin_divisibility]
