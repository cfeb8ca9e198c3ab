"""Checks that pin the float64 sequence-parallel oracle (oracle.sp) to things
other than itself:
  * Philox4x32-10 known-answer vectors (tests/golden/philox4x32_10_kat.json),
  * the keep rate of the dropout mask against p (binomial bounds),
  * torch's float64 layer_norm and its autograd,
  * LayerNorm closed forms (constant rows, unit-variance outputs),
  * pure-Python loops and central finite differences,
  * the pages' statement that splitting along the sequence changes nothing:
    the per-rank SP path composed from row blocks equals the block computed
    on the whole sequence, forward and backward (torch autograd).
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

from oracle import brute
from oracle import ref

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _close(a, b, rtol, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    scale = max(1e-300, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= rtol * scale, f"{what}: max err {err:.3e} > {rtol:.1e} * {scale:.3e}"


def pin_philox_known_answers(sp):
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.json")) as f:
        kat = json.load(f)
    for v in kat["vectors"]:
        ctr = np.array([[int(x, 16) for x in v["ctr"]]], dtype=np.uint32)
        got = sp.philox4x32_10(ctr, [int(x, 16) for x in v["key"]])[0]
        assert [int(x) for x in got] == [int(x, 16) for x in v["out"]], v


def pin_dropout_rate_and_split(sp):
    rows, h = 256, 1024
    for p in (0.0, 0.1, 0.5):
        keep = sp.dropout_keep(1234, 7, rows, h, p)
        n = keep.size
        rate = keep.mean()
        assert abs(rate - (1 - p)) <= 6 * np.sqrt(p * (1 - p) / n) + 1e-12, (p, rate)
    a = sp.dropout_keep(99, 0, 48, 64, 0.3)
    b = np.concatenate([sp.dropout_keep(99, 0, 16, 64, 0.3), sp.dropout_keep(99, 16, 32, 64, 0.3)])
    assert np.array_equal(a, b), "the mask must depend on the global row only"
    assert not np.array_equal(sp.dropout_keep(99, 0, 16, 64, 0.3), sp.dropout_keep(100, 0, 16, 64, 0.3))
    d = np.ones((48, 64))
    _close(sp.dropout_bwd(d, 0.3, 99, 0), np.where(a, 1.0 / (1.0 - float(np.float32(0.3))), 0.0), 1e-15, "dropout bwd")
    try:
        sp.keep_threshold(1.0)
    except ValueError:
        pass
    else:
        raise AssertionError("p = 1 must be refused")


def _ln_case(seed, rows, h):
    r = np.random.default_rng(seed)
    return r.standard_normal((rows, h)) * 2.0 + 0.5, 1.0 + 0.1 * r.standard_normal(h), 0.1 * r.standard_normal(h), \
        r.standard_normal((rows, h))


def pin_layernorm_vs_torch(sp):
    X, g, b, dY = _ln_case(1, 37, 96)
    t = [torch.tensor(m, dtype=torch.float64, requires_grad=True) for m in (X, g, b)]
    Y = torch.nn.functional.layer_norm(t[0], (96,), t[1], t[2], eps=1e-5)
    gx, gg, gb = torch.autograd.grad((Y * torch.tensor(dY)).sum(), t)
    f = sp.layernorm_fwd(X, g, b)
    _close(f["Y"], Y.detach().numpy(), 1e-13, "LN forward")
    d = sp.layernorm_bwd(X, g, dY)
    _close(d["dX"], gx.numpy(), 1e-12, "LN dX")
    _close(d["dgamma"], gg.numpy(), 1e-12, "LN dgamma")
    _close(d["dbeta"], gb.numpy(), 1e-12, "LN dbeta")


def pin_layernorm_closed_forms(sp):
    h = 64
    X = np.full((3, h), 2.5)
    b = np.linspace(-1, 1, h)
    assert np.array_equal(sp.layernorm_fwd(X, np.ones(h), b)["Y"], np.tile(b, (3, 1))), "constant rows give beta"
    X, _, _, _ = _ln_case(2, 5, h)
    f = sp.layernorm_fwd(X, np.ones(h), np.zeros(h))
    var = X.var(axis=1)
    assert np.max(np.abs(f["Y"].mean(axis=1))) < 1e-12, "zero mean"
    _close((f["Y"] ** 2).mean(axis=1), var / (var + 1e-5), 1e-12, "unit variance up to eps")


def pin_layernorm_brute_and_differences(sp):
    X, g, b, dY = _ln_case(3, 3, 8)
    _close(sp.layernorm_fwd(X, g, b)["Y"], brute.layernorm_rows(X, g, b), 1e-13, "LN brute force")
    d = sp.layernorm_bwd(X, g, dY)
    e = 1e-6
    num = np.zeros_like(X)
    for r in range(X.shape[0]):
        for c in range(X.shape[1]):
            Xp, Xm = X.copy(), X.copy()
            Xp[r, c] += e
            Xm[r, c] -= e
            lp = (np.array(brute.layernorm_rows(Xp, g, b)) * dY).sum()
            lm = (np.array(brute.layernorm_rows(Xm, g, b)) * dY).sum()
            num[r, c] = (lp - lm) / (2 * e)
    _close(d["dX"], num, 1e-7, "LN dX by differences")


def _mlp_case(seed, T, h, F):
    r = np.random.default_rng(seed)
    return (r.standard_normal((T, h)), 1.0 + 0.1 * r.standard_normal(h), 0.1 * r.standard_normal(h),
            0.1 * r.standard_normal((h, F)), 0.1 * r.standard_normal(F), 0.1 * r.standard_normal((F, h)),
            r.standard_normal((T, h)))


def pin_sp_split_equals_whole(sp):
    """Forward: LN on each rank's rows, all-gather, TP MLP partials, reduce-scatter
    with dropout and residual per rank == the block on the whole sequence."""
    T, h, F, tp, p, seed = 32, 16, 64, 4, 0.2, 77
    X, g, b, W1, b1, W2, _ = _mlp_case(4, T, h, F)
    rows = T // tp
    Y = np.concatenate([sp.layernorm_fwd(X[i * rows:(i + 1) * rows], g, b)["Y"] for i in range(tp)])
    parts = [ref.tp_mlp_fwd_shard(Y, W1, b1, W2, tp, j)["Z"] for j in range(tp)]
    out = np.concatenate([sp.partial_sum_dropout_residual([P[i * rows:(i + 1) * rows] for P in parts],
                                                          X[i * rows:(i + 1) * rows], p, seed, i * rows)
                          for i in range(tp)])
    whole = sp.sp_block_fwd(X, g, b, lambda Yf: ref.mlp_fwd(Yf, W1, b1, W2)["Z"], p, seed)
    _close(out, whole["out"], 1e-12, "SP split vs whole sequence")


def pin_sp_backward_autograd(sp):
    """Backward composed per rank (dropout bwd into the gathered dZ, TP MLP bwd,
    reduce-scatter of dX partials, LN bwd, plus the residual path) == torch
    autograd through the whole block with the same mask."""
    T, h, F, tp, p, seed = 24, 16, 48, 3, 0.25, 5
    X, g, b, W1, b1, W2, dOut = _mlp_case(6, T, h, F)
    keep = sp.dropout_keep(seed, 0, T, h, p)
    t = [torch.tensor(m, dtype=torch.float64, requires_grad=True) for m in (X, g, b, W1, b1, W2)]
    Yln = torch.nn.functional.layer_norm(t[0], (h,), t[1], t[2], eps=1e-5)
    Hm = Yln @ t[3] + t[4]
    Z = torch.nn.functional.gelu(Hm, approximate="tanh") @ t[5]
    out = t[0] + torch.where(torch.tensor(keep), Z / (1.0 - float(np.float32(p))), torch.zeros_like(Z))
    gX, gg, gb = torch.autograd.grad((out * torch.tensor(dOut)).sum(), t[:3])
    rows = T // tp
    dZ = np.concatenate([sp.dropout_bwd(dOut[i * rows:(i + 1) * rows], p, seed, i * rows) for i in range(tp)])
    Yf = sp.layernorm_fwd(X, g, b)["Y"]
    dXp = [ref.tp_mlp_bwd_shard(Yf, W1, b1, W2, dZ, tp, j)["dX"] for j in range(tp)]
    dX = []
    dgam, dbet = np.zeros(h), np.zeros(h)
    for i in range(tp):
        dY_i = ref.shard_partial_sum([P[i * rows:(i + 1) * rows] for P in dXp])
        d = sp.layernorm_bwd(X[i * rows:(i + 1) * rows], g, dY_i)
        dX.append(d["dX"] + dOut[i * rows:(i + 1) * rows])
        dgam += d["dgamma"]
        dbet += d["dbeta"]
    _close(np.concatenate(dX), gX.numpy(), 1e-11, "SP dX")
    _close(dgam, gg.numpy(), 1e-11, "SP dgamma (sum over ranks)")
    _close(dbet, gb.numpy(), 1e-11, "SP dbeta (sum over ranks)")


def pin_sp_forward_torch(sp):
    """Forward values against torch (float64, independent of the oracle): the
    block out = X + Dropout(GeLU_tanh(LayerNorm(X) W1 + b1) W2) with the same
    keep mask, compared with sp_block_fwd on the whole sequence and with the
    per-rank reduce-scatter end (partial_sum_dropout_residual over each rank's
    rows of the TP partials).  The two oracle paths share their formula for
    the dropout and the residual, so this is the pin that fixes it: dropout
    applies to the MLP output only, kept values scaled by 1/(1-p), the
    residual added unscaled (zouht 2.2.2, Dropout and the residual add)."""
    T, h, F, tp, p, seed = 24, 16, 48, 3, 0.25, 9
    X, g, b, W1, b1, W2, _ = _mlp_case(8, T, h, F)
    keep = sp.dropout_keep(seed, 0, T, h, p)
    t = [torch.tensor(m, dtype=torch.float64) for m in (X, g, b, W1, b1, W2)]
    Yln = torch.nn.functional.layer_norm(t[0], (h,), t[1], t[2], eps=1e-5)
    Z = torch.nn.functional.gelu(Yln @ t[3] + t[4], approximate="tanh") @ t[5]
    out = (t[0] + torch.where(torch.tensor(keep), Z / (1.0 - float(np.float32(p))), torch.zeros_like(Z))).numpy()
    whole = sp.sp_block_fwd(X, g, b, lambda Yf: ref.mlp_fwd(Yf, W1, b1, W2)["Z"], p, seed)
    _close(whole["out"], out, 1e-12, "SP block forward vs torch")
    rows = T // tp
    parts = [ref.tp_mlp_fwd_shard(Yln.numpy(), W1, b1, W2, tp, j)["Z"] for j in range(tp)]
    for i in range(tp):
        r = slice(i * rows, (i + 1) * rows)
        got = sp.partial_sum_dropout_residual([P[r] for P in parts], X[r], p, seed, i * rows)
        _close(got, out[r], 1e-12, f"SP reduce-scatter end, rank {i}, vs torch")


ALL_PINS = [pin_philox_known_answers, pin_dropout_rate_and_split, pin_layernorm_vs_torch, pin_layernorm_closed_forms,
            pin_layernorm_brute_and_differences, pin_sp_split_equals_whole, pin_sp_backward_autograd,
            pin_sp_forward_torch]
