"""Checks that pin the float64 attention oracle (oracle.attn) to things other
than itself: torch's float64 scaled_dot_product_attention and its autograd,
closed forms (zero queries attend uniformly), pure-Python loops, central
finite differences, the pages' independence of heads (any split of the heads
over shards gives the same columns) and the key-block online softmax of the
CP section (a query block's output accumulated key block by key block equals
the whole softmax)."""
from __future__ import annotations

import math

import numpy as np
import torch

from oracle import brute


def _close(a, b, rtol, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    scale = max(1e-300, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= rtol * scale, f"{what}: max err {err:.3e} > {rtol:.1e} * {scale:.3e}"


def _case(seed, B, S, H, d, ld_extra=0):
    r = np.random.default_rng(seed)
    mk = lambda: r.standard_normal((B * S, H * d + ld_extra))  # noqa: E731
    return mk(), mk(), mk(), mk()


def _torch_heads(M, B, S, H, d):
    t = torch.tensor(np.asarray(M)[:, :H * d], dtype=torch.float64)
    return t.reshape(B, S, H, d).permute(0, 2, 1, 3).contiguous().requires_grad_(True)


def _from_torch(t):
    B, H, S, d = t.shape
    return t.detach().permute(0, 2, 1, 3).reshape(B * S, H * d).numpy()


def pin_vs_torch_sdpa(at):
    for causal in (False, True):
        B, S, H, d = 2, 37, 3, 16
        Q, K, V, dO = _case(1 + causal, B, S, H, d, ld_extra=5)
        scale = 0.3
        q, k, v = (_torch_heads(M, B, S, H, d) for M in (Q, K, V))
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=scale)
        gq, gk, gv = torch.autograd.grad((o * _torch_heads(dO, B, S, H, d).detach()).sum(), (q, k, v))
        f = at.attn_fwd(Q, K, V, B, S, H, d, causal, scale)
        _close(f["O"], _from_torch(o), 1e-12, f"O causal={causal}")
        g = at.attn_bwd(Q, K, V, dO, B, S, H, d, causal, scale)
        _close(g["dQ"], _from_torch(gq), 1e-11, f"dQ causal={causal}")
        _close(g["dK"], _from_torch(gk), 1e-11, f"dK causal={causal}")
        _close(g["dV"], _from_torch(gv), 1e-11, f"dV causal={causal}")
        # log-sum-exp of each query row, from torch's own masked scores
        s = (q @ k.transpose(-1, -2)).detach() * scale
        if causal:
            s = s.masked_fill(torch.ones(S, S, dtype=torch.bool).triu(1), float("-inf"))
        lse = torch.logsumexp(s, dim=-1).permute(1, 0, 2).reshape(H, B * S).numpy()
        _close(f["lse"], lse, 1e-12, f"lse causal={causal}")


def pin_closed_forms(at):
    B, S, H, d = 1, 9, 2, 8
    r = np.random.default_rng(3)
    Q = np.zeros((B * S, H * d))
    K, V = r.standard_normal((S, H * d)), r.standard_normal((S, H * d))
    f = at.attn_fwd(Q, K, V, B, S, H, d, False, 0.5)
    _close(f["O"], np.tile(V.mean(axis=0), (S, 1)), 1e-13, "zero queries attend uniformly")
    _close(f["lse"], np.full((H, S), math.log(S)), 1e-13, "lse of uniform attention")
    fc = at.attn_fwd(Q, K, V, B, S, H, d, True, 0.5)
    _close(fc["O"], np.cumsum(V, axis=0) / np.arange(1, S + 1)[:, None], 1e-13, "causal: running mean")
    _close(fc["O"][0], V[0], 1e-15, "causal: the first query sees only itself")


def pin_brute_force(at):
    B, S, H, d = 2, 5, 2, 3
    Q, K, V, _ = _case(4, B, S, H, d)
    for causal in (False, True):
        f = at.attn_fwd(Q, K, V, B, S, H, d, causal, 0.7)
        for b in range(B):
            for h in range(H):
                rs, cs = slice(b * S, (b + 1) * S), slice(h * d, (h + 1) * d)
                want = brute.attention_head(Q[rs, cs], K[rs, cs], V[rs, cs], 0.7, causal)
                _close(f["O"][rs, cs], want, 1e-13, f"brute b={b} h={h} causal={causal}")


def pin_finite_differences(at):
    B, S, H, d = 1, 4, 1, 3
    Q, K, V, dO = _case(5, B, S, H, d)
    for causal in (False, True):
        g = at.attn_bwd(Q, K, V, dO, B, S, H, d, causal, 0.9)
        for name, M in (("dQ", Q), ("dK", K), ("dV", V)):
            num = np.zeros_like(M)
            for i in range(M.shape[0]):
                for j in range(M.shape[1]):
                    e = 1e-6
                    Mp, Mm = M.copy(), M.copy()
                    Mp[i, j] += e
                    Mm[i, j] -= e
                    args = {"dQ": (Mp, K, V), "dK": (Q, Mp, V), "dV": (Q, K, Mp)}[name]
                    argm = {"dQ": (Mm, K, V), "dK": (Q, Mm, V), "dV": (Q, K, Mm)}[name]
                    lp = (at.attn_fwd(*args, B, S, H, d, causal, 0.9)["O"] * dO).sum()
                    lm = (at.attn_fwd(*argm, B, S, H, d, causal, 0.9)["O"] * dO).sum()
                    num[i, j] = (lp - lm) / (2 * e)
            _close(g[name], num, 1e-7, f"{name} by differences, causal={causal}")


def pin_heads_independent(at):
    """Any split of the heads over shards (csdn 1.2.2; zouht 2.2.1) gives the same columns."""
    B, S, H, d, tp = 1, 12, 4, 8, 2
    Q, K, V, dO = _case(6, B, S, H, d)
    f = at.attn_fwd(Q, K, V, B, S, H, d, True, 0.35)
    g = at.attn_bwd(Q, K, V, dO, B, S, H, d, True, 0.35)
    hs = H // tp
    for i in range(tp):
        cs = slice(i * hs * d, (i + 1) * hs * d)
        fi = at.attn_fwd(Q[:, cs], K[:, cs], V[:, cs], B, S, hs, d, True, 0.35)
        _close(fi["O"], f["O"][:, cs], 1e-14, f"shard {i} O")
        gi = at.attn_bwd(Q[:, cs], K[:, cs], V[:, cs], dO[:, cs], B, S, hs, d, True, 0.35)
        for k in ("dQ", "dK", "dV"):
            _close(gi[k], g[k][:, cs], 1e-14, f"shard {i} {k}")


def pin_online_softmax_and_rows(at):
    """Key blocks accumulated with a running max and sum (sunjinbo CP) reproduce
    the whole softmax; the sampled-row view agrees with the whole output."""
    B, S, H, d = 1, 40, 1, 8
    Q, K, V, _ = _case(7, B, S, H, d)
    scale = 0.4
    f = at.attn_fwd(Q, K, V, B, S, H, d, True, scale)
    m = np.full(S, -np.inf)
    l = np.zeros(S)
    acc = np.zeros((S, d))
    for j0 in range(0, S, 16):
        s = Q @ K[j0:j0 + 16].T * scale
        s = np.where(np.arange(j0, min(S, j0 + 16))[None, :] > np.arange(S)[:, None], -np.inf, s)
        m_new = np.maximum(m, s.max(axis=1))
        c = np.exp(m - m_new)
        p = np.exp(s - m_new[:, None])
        l = l * c + p.sum(axis=1)
        acc = acc * c[:, None] + p @ V[j0:j0 + 16]
        m = m_new
    _close(acc / l[:, None], f["O"], 1e-13, "online softmax")
    _close(m + np.log(l), f["lse"][0], 1e-13, "online lse")
    rows = [0, 5, 39]
    fr = at.attn_fwd_rows(Q, K, V, B, S, H, d, True, scale, 0, 0, rows)
    _close(fr["O"], f["O"][rows], 1e-13, "rows view")
    _close(fr["lse"], f["lse"][0][rows], 1e-13, "rows lse")
    # sampled backward rows against the whole backward, two sequences and two heads
    B, S, H = 2, 23, 2
    Q, K, V, dO = _case(9, B, S, H, d)
    for causal in (False, True):
        g = at.attn_bwd(Q, K, V, dO, B, S, H, d, causal, scale)
        for b, hd, rr in ((0, 1, [0, 7, 22]), (1, 0, [3, 4, 21])):
            gr = at.attn_bwd_rows(Q, K, V, dO, B, S, H, d, causal, scale, b, hd, rr)
            idx = [b * S + r for r in rr]
            for k in ("dQ", "dK", "dV"):
                _close(gr[k], g[k][idx, hd * d:(hd + 1) * d], 1e-12, f"rows view {k} causal={causal}")


def _block_case(seed, B, S, H, d):
    r = np.random.default_rng(seed)
    h = H * d
    X = r.standard_normal((B * S, h))
    Ws = [r.standard_normal((h, h)) / math.sqrt(h) for _ in range(4)]
    dZ = r.standard_normal((B * S, h))
    return X, Ws, dZ


def pin_block_vs_torch_mha(at):
    """The head-sharded block (sum over shards of the partials, and of the dX
    partials; the shards' weight gradients as column / row slices of the whole
    ones) against torch's float64 multi-head attention and its autograd, for
    tp = 1, 2, 4."""
    B, S, H, d = 2, 9, 4, 4
    h = H * d
    X, (Wq, Wk, Wv, Wo), dZ = _block_case(8, B, S, H, d)
    for causal in (False, True):
        tX = torch.tensor(X.reshape(B, S, h).transpose(1, 0, 2).copy(), requires_grad=True)   # (L, N, E)
        tw = [torch.tensor(W.T.copy(), requires_grad=True) for W in (Wq, Wk, Wv, Wo)]         # x @ W^T form
        mask = torch.ones(S, S, dtype=torch.bool).triu(1) if causal else None
        out, _ = torch.nn.functional.multi_head_attention_forward(
            tX, tX, tX, h, H, None, None, None, None, False, 0.0, tw[3], None, training=False,
            need_weights=False, attn_mask=mask, use_separate_proj_weight=True, q_proj_weight=tw[0],
            k_proj_weight=tw[1], v_proj_weight=tw[2])
        tdZ = torch.tensor(dZ.reshape(B, S, h).transpose(1, 0, 2).copy())
        grads = torch.autograd.grad((out * tdZ).sum(), [tX] + tw)
        Zt = out.detach().numpy().transpose(1, 0, 2).reshape(B * S, h)
        dXt = grads[0].numpy().transpose(1, 0, 2).reshape(B * S, h)
        dWt = [g.numpy().T for g in grads[1:]]                                                  # back to X @ W form
        for tp in (1, 2, 4):
            Z = at.tp_attn_block_fwd(X, Wq, Wk, Wv, Wo, B, S, H, d, tp, causal, d ** -0.5)
            _close(Z, Zt, 1e-12, f"block output tp={tp} causal={causal}")
            dX = np.zeros_like(X)
            w = H // tp * d
            for i in range(tp):
                g = at.tp_attn_block_bwd_shard(X, Wq, Wk, Wv, Wo, dZ, B, S, H, d, tp, i, causal, d ** -0.5)
                dX += g["dX"]
                c = slice(i * w, (i + 1) * w)
                for k, Wt in enumerate(dWt[:3]):
                    _close(g["dWqkv"][:, k * w:(k + 1) * w], Wt[:, c], 1e-11, f"dW{'qkv'[k]} shard {i}/{tp}")
                _close(g["dWo"], dWt[3][c, :], 1e-11, f"dWo shard {i}/{tp}")
            _close(dX, dXt, 1e-11, f"sum of dX partials tp={tp} causal={causal}")


ALL_PINS = [pin_vs_torch_sdpa, pin_closed_forms, pin_brute_force, pin_finite_differences, pin_heads_independent,
            pin_online_softmax_and_rows, pin_block_vs_torch_mha]
