"""float64 CPU oracle of the attention core between the head-sharded projections.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the CPU
baseline of the benchmark, never by the GPU library.

Pages cited:
  [csdn]     damodev.csdn.net/6a43867610ee7a33f284fb9e.html, 1.2.2 Self-Attention
             模块的张量并行: every head is computed on its own from its own Q, K, V
             projections, so heads can be placed on different GPUs; the head
             outputs are concatenated before the output projection.
  [zouht]    io.zouht.com/197.html, 2.2.1 多头注意力机制: Q/K/V split by columns,
             each GPU owns a group of heads (32 heads on 4 GPUs: 8 each).
  [wangyu]   wangyu.me/posts/llm/tensor-parallelism/, 注意力机制中的张量并行:
             Q, K, V from X, the per-head output O_i, then O W_O.
  [sunjinbo] sunjinbo.space/document/parallelism.html, CP · 上下文并行: the
             attention of a query block is softmax(Q K^T) V over all key
             blocks, accumulated block by block with an online softmax.

Readings where the pages leave a step open (their formulas were lost):
  * O = softmax(Q K^T * scale) V per head and per sequence, scale =
    1/sqrt(head_dim) (the standard scaled form; the CP text's shorthand
    drops the scale).  An optional causal mask lets query position i see key
    positions j <= i only.
  * Layout: T = batch * seq token rows; head h of the shard reads columns
    [h*d, (h+1)*d) of Q, K and V (each [T, heads*d] with its own row stride,
    e.g. the three blocks of the fused QKV projection output); O and the
    gradients use the same column layout.
  * The log-sum-exp of each query row, LSE = log(sum_j exp(s_ij)), is kept
    for the backward.
  * Backward from the chain rule through the softmax: with P = softmax(S),
    dV = P^T dO, dP = dO V^T, dS = P * (dP - D), D_i = sum_j P_ij dP_ij =
    sum_d dO_id O_id, dQ = dS K * scale, dK = dS^T Q * scale.
  * The head-sharded block around it: shard i of tp owns heads
    [i*H/tp, (i+1)*H/tp), i.e. columns c = [i*w, (i+1)*w), w = H/tp * d, of
    each of Wq, Wk, Wv (column split) and rows c of Wo (row split); its fused
    QKV weight is [Wq[:, c] | Wk[:, c] | Wv[:, c]].  Z_i = O_i Wo[c, :] is an
    fp32 partial and the block output is the sum over shards; no biases.
"""
from __future__ import annotations

import math
from typing import Dict

import numpy as np


def _heads(M: np.ndarray, batch: int, seq: int, heads: int, d: int) -> np.ndarray:
    """[T, >= heads*d] -> [batch, heads, seq, d]."""
    M = np.asarray(M, dtype=np.float64)[:, :heads * d]
    return M.reshape(batch, seq, heads, d).transpose(0, 2, 1, 3)


def _unheads(A: np.ndarray) -> np.ndarray:
    b, h, s, d = A.shape
    return A.transpose(0, 2, 1, 3).reshape(b * s, h * d)


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def _mask(seq: int, causal: bool) -> np.ndarray:
    if not causal:
        return np.zeros((seq, seq), dtype=bool)
    return np.triu(np.ones((seq, seq), dtype=bool), k=1)   # True where key j > query i


def attn_fwd(Q, K, V, batch: int, seq: int, heads: int, d: int, causal: bool, scale: float) -> Dict[str, np.ndarray]:
    """Plain definition: per (batch, head) S = Q K^T * scale (masked), P = softmax(S), O = P V."""
    q, k, v = (_heads(M, batch, seq, heads, d) for M in (Q, K, V))
    S = np.matmul(q, k.transpose(0, 1, 3, 2)) * scale
    S = np.where(_mask(seq, causal)[None, None], -np.inf, S)
    m = S.max(axis=-1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=-1, keepdims=True)
    P = E / l
    O = np.matmul(P, v)
    lse = (m + np.log(l))[..., 0]                     # [batch, heads, seq]
    return {"O": _unheads(O), "P": P, "lse": lse.transpose(1, 0, 2).reshape(heads, batch * seq)}


def attn_bwd(Q, K, V, dO, batch: int, seq: int, heads: int, d: int, causal: bool,
             scale: float) -> Dict[str, np.ndarray]:
    f = attn_fwd(Q, K, V, batch, seq, heads, d, causal, scale)
    q, k, v = (_heads(M, batch, seq, heads, d) for M in (Q, K, V))
    do = _heads(dO, batch, seq, heads, d)
    P = f["P"]
    o = _heads(f["O"], batch, seq, heads, d)
    dV = np.matmul(P.transpose(0, 1, 3, 2), do)
    dP = np.matmul(do, v.transpose(0, 1, 3, 2))
    D = (do * o).sum(axis=-1, keepdims=True)
    dS = P * (dP - D)
    dQ = np.matmul(dS, k) * scale
    dK = np.matmul(dS.transpose(0, 1, 3, 2), q) * scale
    return {"dQ": _unheads(dQ), "dK": _unheads(dK), "dV": _unheads(dV),
            "D": D[..., 0].transpose(1, 0, 2).reshape(heads, batch * seq), "O": f["O"], "lse": f["lse"]}


def attn_fwd_rows(Q, K, V, batch: int, seq: int, heads: int, d: int, causal: bool, scale: float,
                  b: int, h: int, rows) -> Dict[str, np.ndarray]:
    """Output rows (positions) of one (batch, head) at full sequence length: each
    query row needs every key, but only its own query."""
    rows = np.asarray(rows)
    q, k, v = (_heads(M, batch, seq, heads, d)[b, h] for M in (Q, K, V))
    S = np.matmul(q[rows], k.T) * scale
    if causal:
        S = np.where(np.arange(seq)[None, :] > rows[:, None], -np.inf, S)
    m = S.max(axis=-1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=-1, keepdims=True)
    return {"O": np.matmul(E / l, v), "lse": (m + np.log(l))[:, 0]}


def attn_bwd_rows(Q, K, V, dO, batch: int, seq: int, heads: int, d: int, causal: bool, scale: float,
                  b: int, h: int, rows) -> Dict[str, np.ndarray]:
    """dQ, dK, dV at positions ``rows`` of one (batch, head), at full sequence
    length.  The same sums as attn_bwd restricted to those rows: a dQ row
    needs its own row of P and dP; a dK or dV row needs the column of P and
    dP at that key, i.e. every query's log-sum-exp and D."""
    rows = np.asarray(rows)
    q, k, v, do = (_heads(M, batch, seq, heads, d)[b, h] for M in (Q, K, V, dO))
    f = attn_fwd(q, k, v, 1, seq, 1, d, causal, scale)
    lse, o = f["lse"][0], f["O"]
    D = (do * o).sum(axis=1)
    pos = np.arange(seq)
    Sr = np.matmul(q[rows], k.T) * scale
    Sc = np.matmul(q, k[rows].T) * scale
    if causal:
        Sr = np.where(pos[None, :] > rows[:, None], -np.inf, Sr)
        Sc = np.where(rows[None, :] > pos[:, None], -np.inf, Sc)
    Pr = np.exp(Sr - lse[rows][:, None])
    dSr = Pr * (np.matmul(do[rows], v.T) - D[rows][:, None])
    Pc = np.exp(Sc - lse[:, None])
    dSc = Pc * (np.matmul(do, v[rows].T) - D[:, None])
    return {"dQ": np.matmul(dSr, k) * scale, "dK": np.matmul(dSc.T, q) * scale, "dV": np.matmul(Pc.T, do)}

def _shard_cols(heads: int, d: int, tp: int, i: int) -> slice:
    if heads % tp:
        raise ValueError(f"heads={heads} is not divisible by tp={tp}")
    w = heads // tp * d
    return slice(i * w, (i + 1) * w)


def qkv_shard_weight(Wq, Wk, Wv, heads: int, d: int, tp: int, i: int) -> np.ndarray:
    """Shard i's fused QKV weight [h, 3w] = [Wq_i | Wk_i | Wv_i] (columns of its heads)."""
    c = _shard_cols(heads, d, tp, i)
    return np.concatenate([np.asarray(W, dtype=np.float64)[:, c] for W in (Wq, Wk, Wv)], axis=1)


def tp_attn_block_fwd_shard(X, Wq, Wk, Wv, Wo, batch: int, seq: int, heads: int, d: int, tp: int, i: int,
                            causal: bool, scale: float) -> Dict[str, np.ndarray]:
    """Shard i's forward: QKV = X Wqkv_i, O = attention over its heads, Z = O Wo_i (a partial)."""
    c = _shard_cols(heads, d, tp, i)
    w = c.stop - c.start
    X = np.asarray(X, dtype=np.float64)
    QKV = X @ qkv_shard_weight(Wq, Wk, Wv, heads, d, tp, i)
    f = attn_fwd(QKV[:, :w], QKV[:, w:2 * w], QKV[:, 2 * w:], batch, seq, heads // tp, d, causal, scale)
    Z = f["O"] @ np.asarray(Wo, dtype=np.float64)[c, :]
    return {"QKV": QKV, "O": f["O"], "lse": f["lse"], "Z": Z}


def tp_attn_block_bwd_shard(X, Wq, Wk, Wv, Wo, dZ, batch: int, seq: int, heads: int, d: int, tp: int, i: int,
                            causal: bool, scale: float) -> Dict[str, np.ndarray]:
    """Shard i's backward for the gradient dZ of the block output, which every
    shard receives whole (Z is a sum of partials): dO = dZ Wo_i^T, dWo_i =
    O^T dZ, the attention backward gives dQKV, dWqkv_i = X^T dQKV and the
    partial dX_i = dQKV Wqkv_i^T (the sum over shards is dX)."""
    c = _shard_cols(heads, d, tp, i)
    w = c.stop - c.start
    X, dZ = np.asarray(X, dtype=np.float64), np.asarray(dZ, dtype=np.float64)
    Wqkv = qkv_shard_weight(Wq, Wk, Wv, heads, d, tp, i)
    Wo_i = np.asarray(Wo, dtype=np.float64)[c, :]
    f = tp_attn_block_fwd_shard(X, Wq, Wk, Wv, Wo, batch, seq, heads, d, tp, i, causal, scale)
    QKV = f["QKV"]
    dO = dZ @ Wo_i.T
    g = attn_bwd(QKV[:, :w], QKV[:, w:2 * w], QKV[:, 2 * w:], dO, batch, seq, heads // tp, d, causal, scale)
    dQKV = np.concatenate([g["dQ"], g["dK"], g["dV"]], axis=1)
    return {"dO": dO, "dWo": f["O"].T @ dZ, "dQKV": dQKV, "dWqkv": X.T @ dQKV, "dX": dQKV @ Wqkv.T,
            "D": g["D"], **f}


def tp_attn_block_fwd(X, Wq, Wk, Wv, Wo, batch: int, seq: int, heads: int, d: int, tp: int, causal: bool,
                      scale: float) -> np.ndarray:
    """The block output: the sum of all tp shards' partials."""
    parts = [tp_attn_block_fwd_shard(X, Wq, Wk, Wv, Wo, batch, seq, heads, d, tp, i, causal, scale)["Z"]
             for i in range(tp)]
    out = np.zeros_like(parts[0])
    for p in parts:
        out += p
    return out
