"""float64 CPU oracle of the tensor-parallel gated MLP (SwiGLU) block.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the CPU
baseline of the benchmark, never by the GPU library.

Page cited: wangyu.me/posts/llm/tensor-parallelism/, 大语言模型并行策略（三）：
张量并行, section 多层感知机（MLP）中的张量并行.  There the gated MLP of
Qwen3 is: gate = X W_gate, up = X W_up, x = silu(gate) * up (elementwise),
down = x W_down; W_gate and W_up may be joined along their columns so that
one product gives both, and the block is split like the plain MLP: the first
product by columns, the second by rows, one sum of partials at the end.

Readings where the page leaves a step open:
  * silu(g) = g * sigmoid(g) (the page names F.silu, whose definition this is).
  * Neither layer has a bias (the page's listing has none).
  * Shard i of the joined first layer owns gate and up columns
    [i*F/tp, (i+1)*F/tp): the same columns of both, so that silu(gate) * up
    needs nothing from other shards.
  * The joined shard weight is stored interleaved in groups of 8 columns:
    packed column 16q + r is gate column 8q + r for r < 8 and up column
    8q + r - 8 for r >= 8 (F/tp must be a multiple of 8).  The same layout
    holds for the saved pre-activations, their gradient and the weight
    gradient of the joined layer.  It is a storage order only: the products
    and sums are those of the page's formulas.
  * Backward follows from the chain rule: with s = sigmoid(g),
    d silu/dg = s (1 + g (1 - s)), so dgate = dx * up * s (1 + g (1 - s)) and
    dup = dx * silu(gate).
"""
from __future__ import annotations

from typing import Dict

import numpy as np

from oracle.ref import _shard_width, col_shard, matmul, row_shard, shard_partial_sum

GROUP = 8  # columns per interleave group


def sigmoid(x: np.ndarray) -> np.ndarray:
    """1 / (1 + exp(-x)) without overflow for either sign."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    e = np.exp(x[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def silu(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return x * sigmoid(x)


def silu_grad(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    s = sigmoid(x)
    return s * (1.0 + x * (1.0 - s))


# --------------------------------------------------------------------------
# Storage order of the joined layer.
# --------------------------------------------------------------------------
def _check_group(Fs: int) -> None:
    if Fs % GROUP != 0:
        raise ValueError(f"shard width {Fs} is not a multiple of {GROUP}")


def interleave(G: np.ndarray, U: np.ndarray) -> np.ndarray:
    """[.., Fs] gate and up blocks -> [.., 2 Fs] in groups of 8 (gate 8, up 8)."""
    G = np.asarray(G)
    U = np.asarray(U)
    if G.shape != U.shape:
        raise ValueError("gate and up blocks differ in shape")
    Fs = G.shape[-1]
    _check_group(Fs)
    lead = G.shape[:-1]
    g = G.reshape(lead + (Fs // GROUP, 1, GROUP))
    u = U.reshape(lead + (Fs // GROUP, 1, GROUP))
    return np.concatenate([g, u], axis=-2).reshape(lead + (2 * Fs,))


def deinterleave(P: np.ndarray):
    """Inverse of interleave: [.., 2 Fs] -> (gate [.., Fs], up [.., Fs])."""
    P = np.asarray(P)
    Fs2 = P.shape[-1]
    if Fs2 % (2 * GROUP) != 0:
        raise ValueError(f"packed width {Fs2} is not a multiple of {2 * GROUP}")
    lead = P.shape[:-1]
    q = P.reshape(lead + (Fs2 // (2 * GROUP), 2, GROUP))
    Fs = Fs2 // 2
    return q[..., 0, :].reshape(lead + (Fs,)), q[..., 1, :].reshape(lead + (Fs,))


def pack_shard(W_gate: np.ndarray, W_up: np.ndarray, tp: int, i: int) -> np.ndarray:
    """Shard i of the joined first layer, [h, 2 F/tp] in the interleaved order."""
    return interleave(col_shard(W_gate, tp, i), col_shard(W_up, tp, i))


# --------------------------------------------------------------------------
# Forward.
# --------------------------------------------------------------------------
def swiglu_fwd(X, W_gate, W_up, W_down) -> Dict[str, np.ndarray]:
    """Unsharded definition: gate, up, x = silu(gate) * up, down = x W_down."""
    G = matmul(X, W_gate)
    U = matmul(X, W_up)
    A = silu(G) * U
    return {"G": G, "U": U, "A": A, "Z": matmul(A, W_down)}


def tp_swiglu_fwd_shard(X, W_gate, W_up, W_down, tp: int, i: int) -> Dict[str, np.ndarray]:
    """Shard i: the joined column-parallel product, the gated activation, the
    row-parallel partial.  GU is the packed pre-activation [T, 2 F/tp]."""
    GU = matmul(X, pack_shard(W_gate, W_up, tp, i))
    G, U = deinterleave(GU)
    A = silu(G) * U
    return {"GU": GU, "A": A, "Z": matmul(A, row_shard(W_down, tp, i))}


def tp_swiglu_fwd(X, W_gate, W_up, W_down, tp: int) -> np.ndarray:
    return shard_partial_sum([tp_swiglu_fwd_shard(X, W_gate, W_up, W_down, tp, i)["Z"] for i in range(tp)])


# --------------------------------------------------------------------------
# Backward.
# --------------------------------------------------------------------------
def swiglu_bwd(X, W_gate, W_up, W_down, dZ) -> Dict[str, np.ndarray]:
    """Unsharded backward for upstream gradient dZ of down."""
    f = swiglu_fwd(X, W_gate, W_up, W_down)
    X = np.asarray(X, dtype=np.float64)
    dZ = np.asarray(dZ, dtype=np.float64)
    dA = matmul(dZ, np.asarray(W_down, dtype=np.float64).T)
    dG = dA * f["U"] * silu_grad(f["G"])
    dU = dA * silu(f["G"])
    return {"dA": dA, "dG": dG, "dU": dU,
            "dW_down": matmul(f["A"].T, dZ), "dW_gate": matmul(X.T, dG), "dW_up": matmul(X.T, dU),
            "dX": matmul(dG, np.asarray(W_gate, dtype=np.float64).T)
                  + matmul(dU, np.asarray(W_up, dtype=np.float64).T)}


def tp_swiglu_bwd_shard(X, W_gate, W_up, W_down, dZ, tp: int, i: int) -> Dict[str, np.ndarray]:
    """Shard i's backward in the packed order: dGU [T, 2 F/tp], dW_gu [h, 2 F/tp],
    dW_down_i [F/tp, h] and the partial dX_i [T, h] (summed over shards)."""
    X = np.asarray(X, dtype=np.float64)
    dZ = np.asarray(dZ, dtype=np.float64)
    W_gu = pack_shard(W_gate, W_up, tp, i)
    Wd_i = row_shard(W_down, tp, i)
    GU = matmul(X, W_gu)
    G, U = deinterleave(GU)
    A = silu(G) * U
    dA = matmul(dZ, Wd_i.T)
    dGU = interleave(dA * U * silu_grad(G), dA * silu(G))
    return {"dA": dA, "dGU": dGU, "dW_gu": matmul(X.T, dGU), "dW_down": matmul(A.T, dZ),
            "dX": matmul(dGU, W_gu.T)}


def unpack_grad_shard(dW_gu: np.ndarray, F: int, tp: int, i: int):
    """Full-width [h, F] gate and up gradients holding shard i's columns (zeros elsewhere)."""
    Fs = _shard_width(F, tp)
    dg, du = deinterleave(dW_gu)
    h = dW_gu.shape[0]
    out_g = np.zeros((h, F))
    out_u = np.zeros((h, F))
    out_g[:, i * Fs:(i + 1) * Fs] = dg
    out_u[:, i * Fs:(i + 1) * Fs] = du
    return out_g, out_u


# --------------------------------------------------------------------------
# Sampled views for sizes where the whole shard is too large for the CPU.
# Rows of the forward and of dX depend only on the same rows of X (and dZ);
# a column of a weight gradient needs that column over every row.  These
# take the shard's packed weight W_gu and its W_down block directly.
# --------------------------------------------------------------------------
def shard_fwd_rows(X, W_gu, Wd_i, rows) -> Dict[str, np.ndarray]:
    Xr = np.asarray(X, dtype=np.float64)[np.asarray(rows)]
    GU = matmul(Xr, W_gu)
    G, U = deinterleave(GU)
    A = silu(G) * U
    return {"GU": GU, "A": A, "Z": matmul(A, Wd_i)}


def shard_bwd_rows(X, W_gu, Wd_i, dZ, rows) -> Dict[str, np.ndarray]:
    """dGU and dX of the given rows."""
    rows = np.asarray(rows)
    Xr = np.asarray(X, dtype=np.float64)[rows]
    G, U = deinterleave(matmul(Xr, W_gu))
    dA = matmul(np.asarray(dZ, dtype=np.float64)[rows], np.asarray(Wd_i, dtype=np.float64).T)
    dGU = interleave(dA * U * silu_grad(G), dA * silu(G))
    return {"dGU": dGU, "dX": matmul(dGU, np.asarray(W_gu, dtype=np.float64).T)}


def shard_bwd_cols(X, W_gu, Wd_i, dZ, cols) -> Dict[str, np.ndarray]:
    """For shard columns c (of the F/tp): dW_gu's packed gate and up columns
    16(c//8) + c%8 and 16(c//8) + 8 + c%8, and rows c of dW_down."""
    cols = np.asarray(cols)
    X = np.asarray(X, dtype=np.float64)
    W_gu = np.asarray(W_gu, dtype=np.float64)
    gcol = 16 * (cols // GROUP) + cols % GROUP
    ucol = gcol + GROUP
    G = matmul(X, W_gu[:, gcol])
    U = matmul(X, W_gu[:, ucol])
    A = silu(G) * U
    dZ = np.asarray(dZ, dtype=np.float64)
    dA = matmul(dZ, np.asarray(Wd_i, dtype=np.float64)[cols].T)
    return {"gate_cols": gcol, "up_cols": ucol,
            "dW_gate_cols": matmul(X.T, dA * U * silu_grad(G)), "dW_up_cols": matmul(X.T, dA * silu(G)),
            "dW_down_rows": matmul(A.T, dZ)}
