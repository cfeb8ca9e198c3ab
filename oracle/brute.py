"""Pure-Python loop evaluation of the MLP block for tiny inputs.

TEST INFRASTRUCTURE ONLY.  It uses lists and ``math`` only (no numpy), and
serves as the brute-force pin of ``oracle.ref``: every entry is the textbook
sum of products, one term at a time.

The block is Z = GeLU(X W1 + b1) W2 with rows of X as tokens (io.zouht.com/197,
2.2.1 在 LLM 中的应用方式, 前馈网络; wangyu.me 大语言模型并行策略（三）：张量并行,
多层感知机（MLP）中的张量并行).
"""
from __future__ import annotations

import math
from typing import List, Optional

Matrix = List[List[float]]


def to_lists(a) -> Matrix:
    return [[float(v) for v in row] for row in a]


def matmul(A: Matrix, B: Matrix) -> Matrix:
    n, k, m = len(A), len(B), len(B[0]) if B else 0
    assert all(len(r) == k for r in A)
    out = [[0.0] * m for _ in range(n)]
    for r in range(n):
        for c in range(m):
            s = 0.0
            for t in range(k):
                s += A[r][t] * B[t][c]
            out[r][c] = s
    return out


def transpose(A: Matrix) -> Matrix:
    return [list(col) for col in zip(*A)] if A else []


def gelu(x: float) -> float:
    u = math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)
    return 0.5 * x * (1.0 + math.tanh(u))


def mlp_fwd(X, W1, b1: Optional[list], W2):
    X, W1, W2 = to_lists(X), to_lists(W1), to_lists(W2)
    H = matmul(X, W1)
    if b1 is not None:
        H = [[v + float(b1[c]) for c, v in enumerate(row)] for row in H]
    A = [[gelu(v) for v in row] for row in H]
    return H, A, matmul(A, W2)


def mlp_bwd_by_differences(X, W1, b1, W2, dZ, step: float = 1e-5):
    """Gradients of L = sum(dZ * Z) by central differences, one entry at a time.

    Slow (O(params * T*h*F)) and only for tiny shapes; independent of any
    backward formula.
    """
    X, W1, W2, dZ = to_lists(X), to_lists(W1), to_lists(W2), to_lists(dZ)
    b = None if b1 is None else [float(v) for v in b1]

    def loss(Xv, W1v, bv, W2v):
        _, _, Z = mlp_fwd(Xv, W1v, bv, W2v)
        return sum(dZ[r][c] * Z[r][c] for r in range(len(Z)) for c in range(len(Z[0])))

    def grad_matrix(M, setter):
        g = [[0.0] * len(M[0]) for _ in M]
        for r in range(len(M)):
            for c in range(len(M[0])):
                old = M[r][c]
                e = step * max(1.0, abs(old))
                M[r][c] = old + e
                lp = setter()
                M[r][c] = old - e
                lm = setter()
                M[r][c] = old
                g[r][c] = (lp - lm) / (2.0 * e)
        return g

    f = lambda: loss(X, W1, b, W2)  # noqa: E731
    out = {"dX": grad_matrix(X, f), "dW1": grad_matrix(W1, f), "dW2": grad_matrix(W2, f)}
    if b is not None:
        bm = [b]
        out["db1"] = grad_matrix(bm, lambda: loss(X, W1, bm[0], W2))[0]
    return out


# ---------------------------------------------------------------------------
# Gated MLP (wangyu.me 大语言模型并行策略（三）：张量并行, 多层感知机（MLP）中的
# 张量并行): gate = X W_gate, up = X W_up, x = silu(gate) * up, down = x W_down.
# ---------------------------------------------------------------------------
def silu(x: float) -> float:
    if x >= 0.0:
        return x / (1.0 + math.exp(-x))
    e = math.exp(x)
    return x * e / (1.0 + e)


def swiglu_fwd(X, W_gate, W_up, W_down):
    X, Wg, Wu, Wd = to_lists(X), to_lists(W_gate), to_lists(W_up), to_lists(W_down)
    G = matmul(X, Wg)
    U = matmul(X, Wu)
    A = [[silu(g) * u for g, u in zip(gr, ur)] for gr, ur in zip(G, U)]
    return G, U, A, matmul(A, Wd)


def swiglu_bwd_by_differences(X, W_gate, W_up, W_down, dZ, step: float = 1e-5):
    """Gradients of L = sum(dZ * down) by central differences (tiny shapes only)."""
    X, Wg, Wu, Wd, dZ = (to_lists(m) for m in (X, W_gate, W_up, W_down, dZ))

    def loss():
        Z = swiglu_fwd(X, Wg, Wu, Wd)[3]
        return sum(dZ[r][c] * Z[r][c] for r in range(len(Z)) for c in range(len(Z[0])))

    def grad_matrix(M):
        g = [[0.0] * len(M[0]) for _ in M]
        for r in range(len(M)):
            for c in range(len(M[0])):
                old = M[r][c]
                e = step * max(1.0, abs(old))
                M[r][c] = old + e
                lp = loss()
                M[r][c] = old - e
                lm = loss()
                M[r][c] = old
                g[r][c] = (lp - lm) / (2.0 * e)
        return g

    return {"dX": grad_matrix(X), "dW_gate": grad_matrix(Wg), "dW_up": grad_matrix(Wu), "dW_down": grad_matrix(Wd)}


# ---------------------------------------------------------------------------
# LayerNorm of one hidden state (io.zouht.com/197, 2.2.2, LayerNorm): mean,
# biased variance, normalise with eps under the square root, scale and shift.
# ---------------------------------------------------------------------------
def layernorm_rows(X, gamma, beta, eps: float = 1e-5):
    out = []
    for row in to_lists(X):
        n = len(row)
        mu = sum(row) / n
        var = sum((v - mu) ** 2 for v in row) / n
        inv = 1.0 / math.sqrt(var + eps)
        out.append([float(gamma[c]) * (v - mu) * inv + float(beta[c]) for c, v in enumerate(row)])
    return out


# ---------------------------------------------------------------------------
# Attention of one head: o_i = sum_j softmax_j(q_i . k_j * scale) v_j, with
# keys j > i left out when causal.
# ---------------------------------------------------------------------------
def attention_head(q, k, v, scale: float, causal: bool):
    q, k, v = to_lists(q), to_lists(k), to_lists(v)
    out = []
    for i, qi in enumerate(q):
        js = range(i + 1) if causal else range(len(k))
        s = [scale * sum(a * b for a, b in zip(qi, k[j])) for j in js]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        z = sum(e)
        out.append([sum(e[t] / z * v[j][c] for t, j in enumerate(js)) for c in range(len(v[0]))])
    return out
