"""float64 CPU oracle of the tensor-parallel MLP block (numpy).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the CPU
baseline of the benchmark, never by the GPU library.

Pages cited (address, title, section):
  [csdn]   damodev.csdn.net/6a43867610ee7a33f284fb9e.html, 1 张量并行
           (1.1 矩阵分块乘法, 1.2.1 MLP 模块的张量并行)
  [zouht]  io.zouht.com/197.html, 2 张量并行 (2.1 概念 block equations,
           2.2.1 在 LLM 中的应用方式, 2.3 代价)
  [wangyu] wangyu.me/posts/llm/tensor-parallelism/, 大语言模型并行策略（三）：张量并行
           (两种切分方式: 按列切分 / 按行切分; 通信模式; 注意力机制中的张量并行;
           多层感知机（MLP）中的张量并行)

Conventions.  Every matrix is row-major and every product is ``Y = X W`` with
X of shape B x M and W of shape M x N [wangyu 两种切分方式].  A column shard of
W holds N/tp contiguous columns; a row shard holds M/tp contiguous rows.  All
arithmetic is float64; inputs are passed in already rounded to the storage
type.  The only primitive taken from a library is the matrix product
(``numpy.matmul``); everything else is written out here.

Readings where the pages leave a step open:
  * The activation is GeLU in its tanh form (the pages only name "GeLU").
  * The first layer may carry a bias, sharded with W1's columns and added
    before the activation; the second layer has none.
  * The backward of Y = XW is dX = dY W^T and dW = X^T dY, with dW in W's
    own orientation (the pages' formulas were not preserved; the orientation
    follows from Y = XW and is pinned by finite differences).
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np

SQRT_2_OVER_PI = math.sqrt(2.0 / math.pi)
GELU_CUBIC = 0.044715

ACT_NONE = "none"
ACT_GELU = "gelu_tanh"


# --------------------------------------------------------------------------
# Activation.  The pages name GeLU as the elementwise activation between the
# two layers [csdn 1.2.1; zouht 2.2.1 前馈网络]; its tanh approximation is
#   gelu(x) = x/2 * (1 + tanh(u)),   u = sqrt(2/pi) * (x + 0.044715 x^3).
# --------------------------------------------------------------------------
def gelu_tanh(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    u = SQRT_2_OVER_PI * (x + GELU_CUBIC * x * x * x)
    return 0.5 * x * (1.0 + np.tanh(u))


def gelu_tanh_grad(x: np.ndarray) -> np.ndarray:
    """d gelu / dx = (1 + t)/2 + x/2 * (1 - t^2) * du/dx, t = tanh(u)."""
    x = np.asarray(x, dtype=np.float64)
    u = SQRT_2_OVER_PI * (x + GELU_CUBIC * x * x * x)
    t = np.tanh(u)
    du = SQRT_2_OVER_PI * (1.0 + 3.0 * GELU_CUBIC * x * x)
    return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * du


def act_fwd(x: np.ndarray, act: str) -> np.ndarray:
    if act == ACT_NONE:
        return np.asarray(x, dtype=np.float64)
    if act == ACT_GELU:
        return gelu_tanh(x)
    raise ValueError(f"unknown activation {act!r}")


def act_grad(x: np.ndarray, act: str) -> np.ndarray:
    if act == ACT_NONE:
        return np.ones_like(np.asarray(x, dtype=np.float64))
    if act == ACT_GELU:
        return gelu_tanh_grad(x)
    raise ValueError(f"unknown activation {act!r}")


# --------------------------------------------------------------------------
# Shards.  W is split by columns into tp blocks of N/tp columns, or by rows
# into tp blocks of M/tp rows; the matching input of a row split is the same
# column block of X [wangyu 按列切分, 按行切分].  A width that tp does not
# divide is an error, as in the pages' example of 32 heads on 5 GPUs
# [zouht 2.2.1].
# --------------------------------------------------------------------------
def _shard_width(n: int, tp: int) -> int:
    if tp < 1 or n % tp != 0:
        raise ValueError(f"width {n} is not divisible by tp_size {tp}")
    return n // tp


def col_shard(W: np.ndarray, tp: int, i: int) -> np.ndarray:
    w = _shard_width(W.shape[1], tp)
    return np.asarray(W, dtype=np.float64)[:, i * w:(i + 1) * w]


def row_shard(W: np.ndarray, tp: int, i: int) -> np.ndarray:
    w = _shard_width(W.shape[0], tp)
    return np.asarray(W, dtype=np.float64)[i * w:(i + 1) * w, :]


def vec_shard(b: Optional[np.ndarray], tp: int, i: int) -> Optional[np.ndarray]:
    if b is None:
        return None
    w = _shard_width(b.shape[0], tp)
    return np.asarray(b, dtype=np.float64)[i * w:(i + 1) * w]


def matmul(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """The one library primitive: float64 matrix product."""
    return np.matmul(np.asarray(A, dtype=np.float64), np.asarray(B, dtype=np.float64))


# --------------------------------------------------------------------------
# Column-parallel layer: Y_i = Act(X W_i + b_i).  Every shard sees the whole
# X and produces N/tp columns of Y; concatenating the shard outputs gives Y
# [zouht 2.1, first block equation; wangyu 按列切分; csdn 1.1 列切分].
# --------------------------------------------------------------------------
def column_parallel_fwd(X, W, b, tp: int, i: int, act: str = ACT_GELU):
    """Shard i of a column-parallel layer.  Returns (H_i, Y_i), H_i = X W_i + b_i."""
    H = matmul(X, col_shard(W, tp, i))
    bi = vec_shard(b, tp, i)
    if bi is not None:
        H = H + bi[None, :]
    return H, act_fwd(H, act)


# --------------------------------------------------------------------------
# Row-parallel layer: Z_i = X_i W_i, with X_i the matching column block of X
# and W_i a row block of W.  Each Z_i has the full output shape; Y is the sum
# of the Z_i [zouht 2.1, second block equation; wangyu 按行切分; csdn 1.1
# 外积和切分].
# --------------------------------------------------------------------------
def row_parallel_fwd(X, W, tp: int, i: int) -> np.ndarray:
    """Shard i of a row-parallel layer, X being the full (unsplit) input."""
    return matmul(col_shard(X, tp, i), row_shard(W, tp, i))


def row_parallel_fwd_shard(X_i, W_i) -> np.ndarray:
    """Same, with the shard's input block and weight block passed directly."""
    return matmul(X_i, W_i)


def shard_partial_sum(partials: Sequence[np.ndarray]) -> np.ndarray:
    """Sum of the tp shard partials, added in ascending shard order.

    This is the arithmetic of the All-Reduce that ends a row-parallel layer
    [wangyu 按行切分 通信模式; zouht 2.3, f* in the forward pass].
    """
    parts = [np.asarray(p, dtype=np.float64) for p in partials]
    if not parts:
        raise ValueError("need at least one partial")
    out = parts[0].copy()
    for p in parts[1:]:
        out = out + p
    return out


# --------------------------------------------------------------------------
# The MLP block: Z = Act(X W1 + b1) W2, W1 split by columns and W2 by rows so
# that each shard's activation output is already the row-split input of the
# second layer, and one sum of partials ends the block [csdn 1.2.1; zouht
# 2.2.1 前馈网络; wangyu 多层感知机（MLP）中的张量并行].
# --------------------------------------------------------------------------
def mlp_fwd(X, W1, b1, W2, act: str = ACT_GELU) -> Dict[str, np.ndarray]:
    """Unsharded definition: H = X W1 + b1, A = Act(H), Z = A W2."""
    H = matmul(X, W1)
    if b1 is not None:
        H = H + np.asarray(b1, dtype=np.float64)[None, :]
    A = act_fwd(H, act)
    return {"H": H, "A": A, "Z": matmul(A, W2)}


def tp_mlp_fwd_shard(X, W1, b1, W2, tp: int, i: int, act: str = ACT_GELU) -> Dict[str, np.ndarray]:
    """Shard i: H_i, A_i from the column-parallel layer, then the fp64 partial Z_i."""
    H_i, A_i = column_parallel_fwd(X, W1, b1, tp, i, act)
    return {"H": H_i, "A": A_i, "Z": row_parallel_fwd_shard(A_i, row_shard(W2, tp, i))}


def tp_mlp_fwd(X, W1, b1, W2, tp: int, act: str = ACT_GELU) -> np.ndarray:
    """All tp shards in turn, then the sum of their partials."""
    return shard_partial_sum([tp_mlp_fwd_shard(X, W1, b1, W2, tp, i, act)["Z"] for i in range(tp)])


# --------------------------------------------------------------------------
# Backward.  For Y = X W with upstream gradient dY the chain rule gives
# dX = dY W^T and dW = X^T dY.  A row-split layer's partials all receive the
# same dY because Y is their sum [wangyu 按行切分, 反向传播]; a column-split
# layer's input gradient is the sum over shards of dY_i W_i^T, which needs an
# All-Reduce [wangyu 按列切分, 反向传播; zouht 2.3, f in the backward pass].
# --------------------------------------------------------------------------
def mlp_bwd(X, W1, b1, W2, dZ, act: str = ACT_GELU) -> Dict[str, np.ndarray]:
    """Unsharded backward of Z = Act(X W1 + b1) W2 for upstream gradient dZ."""
    f = mlp_fwd(X, W1, b1, W2, act)
    dZ = np.asarray(dZ, dtype=np.float64)
    dA = matmul(dZ, np.asarray(W2, dtype=np.float64).T)
    dW2 = matmul(f["A"].T, dZ)
    dH = dA * act_grad(f["H"], act)
    db1 = dH.sum(axis=0)
    dW1 = matmul(np.asarray(X, dtype=np.float64).T, dH)
    dX = matmul(dH, np.asarray(W1, dtype=np.float64).T)
    return {"dA": dA, "dH": dH, "db1": db1, "dW1": dW1, "dW2": dW2, "dX": dX}


def tp_mlp_bwd_shard(X, W1, b1, W2, dZ, tp: int, i: int, act: str = ACT_GELU) -> Dict[str, np.ndarray]:
    """Shard i's backward: the row-parallel layer first, then the column-parallel one.

    Returns dH_i, db1_i, dW1_i [h, F/tp], dW2_i [F/tp, h] and the partial
    input gradient dX_i [T, h] whose sum over shards is dX.
    """
    X = np.asarray(X, dtype=np.float64)
    dZ = np.asarray(dZ, dtype=np.float64)
    W1_i = col_shard(W1, tp, i)
    W2_i = row_shard(W2, tp, i)
    H_i, A_i = column_parallel_fwd(X, W1, b1, tp, i, act)
    dA_i = matmul(dZ, W2_i.T)                 # same dZ on every shard
    dW2_i = matmul(A_i.T, dZ)
    dH_i = dA_i * act_grad(H_i, act)
    return {"dA": dA_i, "dH": dH_i, "db1": dH_i.sum(axis=0), "dW1": matmul(X.T, dH_i),
            "dW2": dW2_i, "dX": matmul(dH_i, W1_i.T)}


def column_parallel_bwd(X, W_i, dY_i, with_bias: bool = False) -> Dict[str, np.ndarray]:
    """Backward of one column shard Y_i = X W_i (+ b_i), dY_i the gradient of Y_i.

    dX_partial = dY_i W_i^T (summed over shards to give dX), dW_i = X^T dY_i,
    db_i = column sums of dY_i.
    """
    dY_i = np.asarray(dY_i, dtype=np.float64)
    out = {"dX": matmul(dY_i, np.asarray(W_i, dtype=np.float64).T),
           "dW": matmul(np.asarray(X, dtype=np.float64).T, dY_i)}
    if with_bias:
        out["db"] = dY_i.sum(axis=0)
    return out


def row_parallel_bwd(X_i, W_i, dY) -> Dict[str, np.ndarray]:
    """Backward of one row shard Z_i = X_i W_i with the full upstream dY.

    dX_i = dY W_i^T is shard i's column block of dX; dW_i = X_i^T dY.
    """
    dY = np.asarray(dY, dtype=np.float64)
    return {"dX": matmul(dY, np.asarray(W_i, dtype=np.float64).T),
            "dW": matmul(np.asarray(X_i, dtype=np.float64).T, dY)}


# --------------------------------------------------------------------------
# Head-sharded attention projections.  Q, K and V are split by heads, which
# is a column split of each projection; the output projection is split by
# rows and ends in a sum of partials [zouht 2.2.1 多头注意力机制; wangyu
# 注意力机制中的张量并行].  Shard i owns heads [i*H/tp, (i+1)*H/tp).
# --------------------------------------------------------------------------
def qkv_shard_weight(Wq, Wk, Wv, heads: int, head_dim: int, tp: int, i: int) -> np.ndarray:
    """Shard i's fused QKV weight [h, 3*h/tp] = [Wq_i | Wk_i | Wv_i]."""
    hp = _shard_width(heads, tp)
    c0, c1 = i * hp * head_dim, (i + 1) * hp * head_dim
    return np.concatenate([np.asarray(W, dtype=np.float64)[:, c0:c1] for W in (Wq, Wk, Wv)], axis=1)


def qkv_fwd_shard(X, Wq, Wk, Wv, heads: int, head_dim: int, tp: int, i: int) -> np.ndarray:
    return matmul(X, qkv_shard_weight(Wq, Wk, Wv, heads, head_dim, tp, i))


def out_proj_fwd_shard(O_in, Wo, heads: int, head_dim: int, tp: int, i: int) -> np.ndarray:
    """Partial of the row-split output projection from shard i's heads."""
    hp = _shard_width(heads, tp)
    r0, r1 = i * hp * head_dim, (i + 1) * hp * head_dim
    return matmul(np.asarray(O_in, dtype=np.float64)[:, r0:r1], np.asarray(Wo, dtype=np.float64)[r0:r1, :])


# --------------------------------------------------------------------------
# Sampled evaluation for workloads too large to evaluate whole: exact for the
# entries it returns (each is the same sum of products as in the full
# definition, restricted to the rows or columns asked for).
# --------------------------------------------------------------------------
def tp_mlp_fwd_shard_rows(X, W1_i, b1_i, W2_i, rows, act: str = ACT_GELU) -> Dict[str, np.ndarray]:
    """Rows ``rows`` of H_i, A_i and Z_i for one shard (weights already sliced)."""
    Xr = np.asarray(X, dtype=np.float64)[np.asarray(rows)]
    H = matmul(Xr, W1_i)
    if b1_i is not None:
        H = H + np.asarray(b1_i, dtype=np.float64)[None, :]
    A = act_fwd(H, act)
    return {"H": H, "A": A, "Z": matmul(A, W2_i)}


def tp_mlp_bwd_shard_cols(X, W1_i, b1_i, W2_i, dZ, cols, act: str = ACT_GELU) -> Dict[str, np.ndarray]:
    """Columns ``cols`` of dH_i, db1_i and dW1_i, and rows ``cols`` of dW2_i.

    Column j of dH_i needs only column j of H_i and of dA_i = dZ W2_i^T.
    """
    X = np.asarray(X, dtype=np.float64)
    dZ = np.asarray(dZ, dtype=np.float64)
    c = np.asarray(cols)
    W1c = np.asarray(W1_i, dtype=np.float64)[:, c]
    H = matmul(X, W1c)
    if b1_i is not None:
        H = H + np.asarray(b1_i, dtype=np.float64)[c][None, :]
    A = act_fwd(H, act)
    dA = matmul(dZ, np.asarray(W2_i, dtype=np.float64)[c, :].T)
    dH = dA * act_grad(H, act)
    return {"dH": dH, "db1": dH.sum(axis=0), "dW1": matmul(X.T, dH), "dW2": matmul(A.T, dZ)}


def tp_mlp_bwd_shard_rows(X, W1_i, b1_i, W2_i, dZ, rows, act: str = ACT_GELU) -> Dict[str, np.ndarray]:
    """Rows ``rows`` of dH_i and of the partial input gradient dX_i."""
    r = np.asarray(rows)
    Xr = np.asarray(X, dtype=np.float64)[r]
    H = matmul(Xr, W1_i)
    if b1_i is not None:
        H = H + np.asarray(b1_i, dtype=np.float64)[None, :]
    dA = matmul(np.asarray(dZ, dtype=np.float64)[r], np.asarray(W2_i, dtype=np.float64).T)
    dH = dA * act_grad(H, act)
    return {"dH": dH, "dX": matmul(dH, np.asarray(W1_i, dtype=np.float64).T)}
