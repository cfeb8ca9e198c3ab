"""GPU parity of the standalone (unfused) GeLU epilogues against the float64 oracle.

bias_gelu_fwd and gelu_bwd apply the column-parallel layer's epilogues to an
fp32 product after the GEMM (the fusion ablation; GeLU is elementwise and
commutes with the column split, csdn 1.2.1).  Cases cover both storage
dtypes, empty and one-row batches, ragged widths, with and without bias and
the saved pre-activation.  The fused path and the unfused one (the same
GEMM with an fp32 output, then bias_gelu_fwd) run the same arithmetic, so
their outputs are equal bit for bit.  Bar: max|err|/max|ref| <= 2e-2 (bf16)
or 1e-5 (fp32).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from oracle import ref
from tests.gpu_util import assert_close, empty, empty_f32, need_gpu, sync, to_dev as _to_dev, to_f64


def to_dev(a: np.ndarray, dtype: str):
    """Upload float32 values, rounded to bf16 (nearest even) for bf16 storage."""
    a = np.asarray(a, dtype=np.float32)
    return _to_dev(synth.bf16_round_bits(a) if dtype == "bf16" else a, dtype)

pytestmark = pytest.mark.gpu

import linear_layers_amd as tl  # noqa: E402


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T,N,bias,save_h", [(777, 264, True, True), (1, 8, False, False), (0, 64, True, True),
                                              (4096, 2048, True, False)])
def test_bias_gelu_fwd(dtype, T, N, bias, save_h):
    need_gpu()
    print(f"bias_gelu_fwd {dtype} T={T} N={N}", flush=True)
    r = np.random.default_rng(T + N)
    Hin = (3.0 * r.standard_normal((T, N))).astype(np.float32)
    b = (0.5 * r.standard_normal(N)).astype(np.float32)
    bd = to_dev(b, dtype) if bias else None
    A, H = empty((T, N), dtype), (empty((T, N), dtype) if save_h else None)
    tl.bias_gelu_fwd(to_dev(Hin, "f32"), A, bias=bd, H_out=H)
    sync()
    hb = Hin.astype(np.float64) + (to_f64(bd)[None, :] if bias else 0.0)
    assert_close(to_f64(A), ref.gelu_tanh(hb), dtype, "A")
    if save_h:
        assert_close(to_f64(H), hb, dtype, "H")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T,N", [(777, 264), (1, 8), (0, 64), (4096, 2048)])
def test_gelu_bwd(dtype, T, N):
    need_gpu()
    print(f"gelu_bwd {dtype} T={T} N={N}", flush=True)
    r = np.random.default_rng(7 * T + N)
    dA = r.standard_normal((T, N)).astype(np.float32)
    Hd = to_dev((3.0 * r.standard_normal((T, N))).astype(np.float32), dtype)
    dH = empty((T, N), dtype)
    tl.gelu_bwd(to_dev(dA, "f32"), Hd, dH)
    sync()
    assert_close(to_f64(dH), dA.astype(np.float64) * ref.gelu_tanh_grad(to_f64(Hd)), dtype, "dH")


def test_fused_equals_unfused():
    """column_parallel_fwd's fused epilogue vs the same product with an fp32 output followed by bias_gelu_fwd."""
    need_gpu()
    T, K, N = 1000, 200, 520
    r = np.random.default_rng(3)
    X = to_dev(r.standard_normal((T, K)).astype(np.float32), "bf16")
    W = to_dev((0.05 * r.standard_normal((K, N))).astype(np.float32), "bf16")
    b = to_dev((0.1 * r.standard_normal(N)).astype(np.float32), "bf16")
    A1, H1 = empty((T, N), "bf16"), empty((T, N), "bf16")
    tl.column_parallel_fwd(X, W, 1, A1, bias_shard=b, H_save=H1)
    P, A2, H2 = empty_f32((T, N)), empty((T, N), "bf16"), empty((T, N), "bf16")
    tl.row_parallel_fwd(X, W, 1, P)
    tl.bias_gelu_fwd(P, A2, bias=b, H_out=H2)
    sync()
    assert torch.equal(A1, A2) and torch.equal(H1, H2)
