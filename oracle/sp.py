"""float64 CPU oracle of the sequence-parallel (SP) region around the MLP block.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the CPU
baseline of the benchmark, never by the GPU library.

Pages cited:
  [zouht]    io.zouht.com/197.html, 2.2.2 与序列并行（Sequence Parallel）结合:
             Dropout is elementwise and LayerNorm works on each hidden state
             on its own, so both can be split along the sequence; LayerNorm is
             mu = mean(h), sigma^2 = mean((h - mu)^2), h_hat = (h - mu) /
             sqrt(sigma^2 + eps), h' = gamma * h_hat + beta.  2.3 代价: with
             SP the forward's f* all-reduce becomes a reduce-scatter (g*) and
             the input all-gather (g); the backward swaps them.
  [sunjinbo] sunjinbo.space/document/parallelism.html, SP · 序列并行: the
             non-TP region (LayerNorm, Dropout, residual) holds 1/N of the
             sequence on each GPU.

Readings where the pages leave a step open:
  * eps = 1e-5; the variance is the biased one (1/d_model), as written.
  * The block on one GPU's rows [r0, r0 + T/tp) of the residual stream X:
        Y_i = LayerNorm(X_i)                      (seq-split)
        Y   = all-gather of the Y_i              (g)
        Z_j = shard j's MLP partial of Y          (the TP region)
        out_i = X_i + Dropout(sum_j Z_j[rows i])  (g* = reduce-scatter, then
                                                   the seq-split dropout and
                                                   residual)
  * Dropout keeps an element with probability 1 - p and scales kept values by
    1 / (1 - p).  Its random bits come from the counter-based generator
    Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
    Easy as 1, 2, 3", SC 2011), written here from that definition: element
    (r, c) of the [T, h] tensor, flat index e = r*h + c with r the global
    row, takes word e % 4 of the generator at counter (n mod 2^32, n >> 32,
    0, 0), n = e // 4, key (seed mod 2^32, seed >> 32); it is kept iff that
    word >= floor(p * 2^32).  The mask therefore does not depend on how the
    sequence is split.
  * Residual-stream activations are bf16, LayerNorm parameters and
    statistics fp32; the reduce-scatter sums in fp32 (ascending shards) and
    the output is rounded once.
"""
from __future__ import annotations

from typing import Dict, Sequence

import numpy as np

from oracle.ref import shard_partial_sum

EPS = 1e-5

# Philox4x32 constants from the SC 2011 paper: round multipliers and the
# Weyl-sequence key increments.
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(ctr: np.ndarray, key: Sequence[int]) -> np.ndarray:
    """Philox4x32 with 10 rounds.  ctr: [n, 4] uint32 counters; key: two 32-bit words.

    One round: (hi0, lo0) = M0 * c0, (hi1, lo1) = M1 * c2 (64-bit products),
    c <- (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); the key advances by
    (W0, W1) before every round but the first.
    """
    c = np.asarray(ctr, dtype=np.uint32).reshape(-1, 4).astype(np.uint64)
    k0, k1 = np.uint64(int(key[0]) & 0xFFFFFFFF), np.uint64(int(key[1]) & 0xFFFFFFFF)
    m0, m1 = np.uint64(PHILOX_M0), np.uint64(PHILOX_M1)
    for r in range(10):
        if r > 0:
            k0 = (k0 + np.uint64(PHILOX_W0)) & _MASK32
            k1 = (k1 + np.uint64(PHILOX_W1)) & _MASK32
        p0 = m0 * c[:, 0]
        p1 = m1 * c[:, 2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c = np.stack([hi1 ^ c[:, 1] ^ k0, lo1, hi0 ^ c[:, 3] ^ k1, lo0], axis=1)
    return c.astype(np.uint32)


def keep_threshold(p: float) -> int:
    """Words >= this are kept; p is taken as the float32 the C ABI receives."""
    p32 = float(np.float32(p))
    if not 0.0 <= p32 < 1.0:
        raise ValueError(f"dropout probability {p} outside [0, 1)")
    return int(np.floor(p32 * 4294967296.0))


def dropout_keep(seed: int, row0: int, rows: int, h: int, p: float) -> np.ndarray:
    """Boolean keep mask of rows [row0, row0 + rows) of a [T, h] tensor."""
    if h % 4 != 0:
        raise ValueError("h must be a multiple of 4")
    n0 = row0 * h // 4
    n = np.arange(n0, n0 + rows * h // 4, dtype=np.uint64)
    ctr = np.zeros((n.size, 4), dtype=np.uint32)
    ctr[:, 0] = (n & _MASK32).astype(np.uint32)
    ctr[:, 1] = (n >> np.uint64(32)).astype(np.uint32)
    words = philox4x32_10(ctr, (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)).reshape(rows, h)
    return words >= np.uint32(keep_threshold(p))


def dropout_scale(p: float) -> float:
    return 1.0 / (1.0 - float(np.float32(p)))


# --------------------------------------------------------------------------
# LayerNorm [zouht 2.2.2 LayerNorm].
# --------------------------------------------------------------------------
def layernorm_fwd(X, gamma, beta, eps: float = EPS) -> Dict[str, np.ndarray]:
    X = np.asarray(X, dtype=np.float64)
    h = X.shape[1]
    mu = X.sum(axis=1) / h
    var = ((X - mu[:, None]) ** 2).sum(axis=1) / h
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (X - mu[:, None]) * rstd[:, None]
    Y = np.asarray(gamma, dtype=np.float64)[None, :] * xhat + np.asarray(beta, dtype=np.float64)[None, :]
    return {"Y": Y, "mean": mu, "rstd": rstd, "xhat": xhat}


def layernorm_bwd(X, gamma, dY, eps: float = EPS) -> Dict[str, np.ndarray]:
    """Chain rule through h' = gamma * (h - mu) * rstd + beta, per row:
    dX = rstd * (g - mean(g) - xhat * mean(g * xhat)), g = dY * gamma;
    dgamma = sum over rows of dY * xhat, dbeta = sum over rows of dY."""
    f = layernorm_fwd(X, gamma, np.zeros_like(np.asarray(gamma, dtype=np.float64)), eps)
    dY = np.asarray(dY, dtype=np.float64)
    g = dY * np.asarray(gamma, dtype=np.float64)[None, :]
    xh = f["xhat"]
    dX = f["rstd"][:, None] * (g - g.mean(axis=1, keepdims=True) - xh * (g * xh).mean(axis=1, keepdims=True))
    return {"dX": dX, "dgamma": (dY * xh).sum(axis=0), "dbeta": dY.sum(axis=0)}


# --------------------------------------------------------------------------
# The reduce-scatter end of the TP region, then dropout and the residual
# [zouht 2.2.2 Dropout, 2.3 g*; sunjinbo SP].
# --------------------------------------------------------------------------
def partial_sum_dropout_residual(partial_rows: Sequence[np.ndarray], residual, p: float, seed: int,
                                 row0: int) -> np.ndarray:
    """out = residual + Dropout(sum_j partial_j) on rows [row0, row0 + rows)."""
    z = shard_partial_sum(partial_rows)
    rows, h = z.shape
    keep = dropout_keep(seed, row0, rows, h, p)
    return np.asarray(residual, dtype=np.float64) + np.where(keep, z * dropout_scale(p), 0.0)


def dropout_bwd(dOut, p: float, seed: int, row0: int) -> np.ndarray:
    """Gradient through Dropout for rows [row0, ...): kept entries scaled, others zero."""
    dOut = np.asarray(dOut, dtype=np.float64)
    keep = dropout_keep(seed, row0, dOut.shape[0], dOut.shape[1], p)
    return np.where(keep, dOut * dropout_scale(p), 0.0)


def sp_block_fwd(X, gamma, beta, mlp, p: float, seed: int, eps: float = EPS) -> Dict[str, np.ndarray]:
    """The whole block on the full sequence: out = X + Dropout(mlp(LayerNorm(X))).

    ``mlp`` maps the full [T, h] LayerNorm output to the full [T, h] block
    output (the sum of the shard partials).  The SP split changes where each
    row is computed, not what is computed, so the seq-split path must match
    this row for row."""
    ln = layernorm_fwd(X, gamma, beta, eps)
    Z = mlp(ln["Y"])
    T, h = Z.shape
    keep = dropout_keep(seed, 0, T, h, p)
    return {"Y": ln["Y"], "Z": Z, "out": np.asarray(X, dtype=np.float64) + np.where(keep, Z * dropout_scale(p), 0.0)}
