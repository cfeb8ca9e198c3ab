"""Seeded synthetic inputs for the tensor-parallel MLP workloads.

This module only draws random numbers and rounds them to the storage type.
It holds none of the MLP's arithmetic, so both the CPU oracle's tests and the
GPU path can take their inputs from here without sharing any computation.

Every tensor is drawn from its own PCG64 stream, seeded with
``(workload_seed, tensor_index)``, as float32 normal samples scaled by the
workload's standard deviation.  bf16 workloads then round each float32 to
bfloat16 with round-to-nearest-even on the bit pattern, so the oracle (which
upcasts those exact values to float64) and the GPU see identical inputs.

Workload shapes follow the block the pages describe: a hidden size ``h``, an
FFN width ``F`` split over ``tp`` shards by columns for the first weight and
by rows for the second (wangyu.me, "大语言模型并行策略（三）：张量并行",
section 多层感知机（MLP）中的张量并行), and ``T`` tokens (batch x sequence).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Tuple

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "bf16_round_bits",
    "bf16_bits_to_f32",
    "draw",
    "mlp_inputs",
    "proj_inputs",
    "swiglu_inputs",
    "sp_inputs",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, storage type and input distributions."""

    name: str
    seed: int
    dtype: str                  # "f32" or "bf16" storage; accumulation is always fp32
    T: int                      # tokens = batch * sequence
    h: int                      # hidden size
    F: int                      # full FFN width (MLP) or full projection width (attention)
    tp: int                     # tensor-parallel degree
    x_std: float = 1.0
    w_std: float = 0.02
    b_std: Optional[float] = None   # None: no bias; 0.0: a zero bias buffer
    dz_std: Optional[float] = None  # None: forward only
    kind: str = "mlp"           # "mlp", "proj" (head-sharded QKV / O projections), "swiglu" (gated MLP)
                                # or "sp_mlp" (the MLP inside the sequence-parallel region)
    heads: int = 0
    head_dim: int = 0

    @property
    def Fs(self) -> int:
        return self.F // self.tp


# Shapes and distributions of the five workloads the measurement covers.
WORKLOADS: Dict[str, Workload] = {
    "tiny_f32": Workload("tiny_f32", 1, "f32", T=128, h=256, F=1024, tp=2,
                         x_std=1.0, w_std=0.02, b_std=0.0),
    "gpt2m_bf16": Workload("gpt2m_bf16", 2, "bf16", T=4096, h=1024, F=4096, tp=2,
                           x_std=1.0, w_std=0.02, b_std=0.01, dz_std=1.0),
    "llama7b_bf16": Workload("llama7b_bf16", 3, "bf16", T=8192, h=4096, F=16384, tp=8,
                             x_std=1.0, w_std=0.02, b_std=None, dz_std=1.0),
    "attn_proj_bf16": Workload("attn_proj_bf16", 4, "bf16", T=4096, h=5120, F=5120, tp=4,
                               x_std=0.02, w_std=0.02, b_std=None, dz_std=1.0,
                               kind="proj", heads=40, head_dim=128),
    "gpt3_bf16": Workload("gpt3_bf16", 5, "bf16", T=2048, h=12288, F=49152, tp=8,
                          x_std=1.0, w_std=0.02, b_std=None, dz_std=1.0),
    # The gated MLP of the pages' Qwen3 example at Qwen3-8B's sizes (hidden
    # 4096, gate/up width 12288), 8 shards of F/tp = 1536 columns each.
    "qwen3_swiglu_bf16": Workload("qwen3_swiglu_bf16", 6, "bf16", T=8192, h=4096, F=12288, tp=8,
                                  x_std=1.0, w_std=0.02, b_std=None, dz_std=1.0, kind="swiglu"),
    # The Llama-7B-scale MLP inside the sequence-parallel region: LayerNorm
    # before it, dropout (p = 0.1) and the residual after it, each GPU holding
    # T/tp rows of the residual stream.
    "llama7b_sp_bf16": Workload("llama7b_sp_bf16", 7, "bf16", T=8192, h=4096, F=16384, tp=8,
                                x_std=1.0, w_std=0.02, b_std=None, dz_std=1.0, kind="sp_mlp"),
}

SP_DROPOUT_P = 0.1


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bfloat16 bit patterns, round-to-nearest-even.

    Inputs are finite normal samples, so no NaN handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> exactly equal float32 values."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw(seed: int, index: int, shape: Tuple[int, ...], std: float, dtype: str,
         chunk_rows: int = 4096) -> np.ndarray:
    """Draw one tensor.

    Returns float32 values for ``dtype == "f32"`` and uint16 bf16 bit patterns
    for ``dtype == "bf16"``.  Rows are drawn in chunks from one stream, so the
    result does not depend on ``chunk_rows``; chunking only bounds host memory.
    """
    rng = np.random.default_rng([int(seed), int(index)])
    if dtype == "f32":
        out = np.empty(shape, dtype=np.float32)
    elif dtype == "bf16":
        out = np.empty(shape, dtype=np.uint16)
    else:
        raise ValueError(f"unknown dtype {dtype!r}")
    if out.size == 0:
        return out
    flat = out.reshape(shape[0], -1) if len(shape) > 1 else out.reshape(1, -1)
    step = max(1, int(chunk_rows))
    for r0 in range(0, flat.shape[0], step):
        r1 = min(flat.shape[0], r0 + step)
        v = rng.standard_normal(size=(r1 - r0, flat.shape[1]), dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        flat[r0:r1] = v if dtype == "f32" else bf16_round_bits(v)
    return out


# Tensor indices inside a workload's stream family.
_IDX = {"X": 0, "W1": 1, "b1": 2, "W2": 3, "dZ": 4,
        "Wq": 10, "Wk": 11, "Wv": 12, "O_in": 13, "Wo": 14, "dQKV": 15, "dOut": 16,
        "W_gate": 20, "W_up": 21, "W_down": 22, "ln_gamma": 30, "ln_beta": 31}


def mlp_inputs(wl: Workload, which=("X", "W1", "b1", "W2", "dZ"), T: Optional[int] = None,
               h: Optional[int] = None, F: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Full (unsharded) MLP inputs of a workload, optionally at other sizes.

    X [T,h], W1 [h,F], b1 [F], W2 [F,h], dZ [T,h].  Absent tensors (no bias,
    forward-only) are left out.  Shapes may be overridden to make small cases
    with the same distributions.
    """
    T = wl.T if T is None else T
    h = wl.h if h is None else h
    F = wl.F if F is None else F
    shapes = {"X": (T, h), "W1": (h, F), "b1": (F,), "W2": (F, h), "dZ": (T, h)}
    stds = {"X": wl.x_std, "W1": wl.w_std, "b1": wl.b_std, "W2": wl.w_std, "dZ": wl.dz_std}
    out = {}
    for name in which:
        std = stds[name]
        if std is None:
            continue
        if name == "b1" and std == 0.0:
            out[name] = np.zeros(shapes[name], dtype=np.float32 if wl.dtype == "f32" else np.uint16)
            continue
        out[name] = draw(wl.seed, _IDX[name], shapes[name], std, wl.dtype)
    return out


def proj_inputs(wl: Workload, which=("X", "Wq", "Wk", "Wv", "O_in", "Wo", "dQKV", "dOut"),
                T: Optional[int] = None, heads: Optional[int] = None,
                head_dim: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Inputs of the head-sharded attention projections.

    X [T,h]; Wq, Wk, Wv [h,h]; O_in [T,h] (the attention output that feeds the
    output projection); Wo [h,h]; upstream gradients dQKV [T,3h/tp] for one
    shard and dOut [T,h].  h = heads * head_dim.
    """
    T = wl.T if T is None else T
    heads = wl.heads if heads is None else heads
    head_dim = wl.head_dim if head_dim is None else head_dim
    h = heads * head_dim
    shapes = {"X": (T, h), "Wq": (h, h), "Wk": (h, h), "Wv": (h, h), "O_in": (T, h),
              "Wo": (h, h), "dQKV": (T, 3 * h // wl.tp), "dOut": (T, h)}
    stds = {"X": wl.x_std, "Wq": wl.w_std, "Wk": wl.w_std, "Wv": wl.w_std, "O_in": wl.x_std,
            "Wo": wl.w_std, "dQKV": wl.dz_std, "dOut": wl.dz_std}
    return {n: draw(wl.seed, _IDX[n], shapes[n], stds[n], wl.dtype) for n in which}


def swiglu_inputs(wl: Workload, which=("X", "W_gate", "W_up", "W_down", "dZ"), T: Optional[int] = None,
                  h: Optional[int] = None, F: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Full (unsharded) gated-MLP inputs: X [T,h], W_gate and W_up [h,F], W_down [F,h], dZ [T,h]."""
    T = wl.T if T is None else T
    h = wl.h if h is None else h
    F = wl.F if F is None else F
    shapes = {"X": (T, h), "W_gate": (h, F), "W_up": (h, F), "W_down": (F, h), "dZ": (T, h)}
    stds = {"X": wl.x_std, "W_gate": wl.w_std, "W_up": wl.w_std, "W_down": wl.w_std, "dZ": wl.dz_std}
    return {n: draw(wl.seed, _IDX[n], shapes[n], stds[n], wl.dtype) for n in which if stds[n] is not None}


def sp_inputs(wl: Workload, T: Optional[int] = None, h: Optional[int] = None,
              F: Optional[int] = None) -> Dict[str, np.ndarray]:
    """MLP inputs plus the LayerNorm parameters: gamma = 1 + N(0, 0.1^2),
    beta = N(0, 0.1^2), both float32 [h].  X is the residual stream; dZ is the
    upstream gradient of the block output."""
    out = mlp_inputs(wl, T=T, h=h, F=F)
    h = wl.h if h is None else h
    out["ln_gamma"] = np.float32(1.0) + draw(wl.seed, _IDX["ln_gamma"], (h,), 0.1, "f32")
    out["ln_beta"] = draw(wl.seed, _IDX["ln_beta"], (h,), 0.1, "f32")
    return out


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of a drawn tensor (bf16 bits are decoded first)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)
