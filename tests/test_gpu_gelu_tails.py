"""fp32 parity of the GeLU epilogues in their saturated tails.

The device evaluates GeLU as x * s, s = 1 / (1 + 2^(-z)) with the hardware
base-2 exponential and reciprocal, and GeLU' with its argument clamped to
+-64 (R14 of the design notes: the tanh form of csdn 1.2.1 / zouht 2.2.1 in
its logistic shape).  Pre-activations of order one never reach the parts of
that code where the exponential overflows or underflows, where 1 - s cancels,
or where the clamp acts; here a per-column bias spreads each shard's
pre-activations over [-70, 70] (both tails and past the clamp in every
shard), with fp32 storage so the 1e-5 bar applies.

Bar: each output tensor within max|err| <= 1e-5 max|ref| of the float64
oracle, and each column within 1e-5 of max(1, max|ref| over the column) -
the per-column check sees a tail column go wrong (a NaN, the wrong
saturation value, a sign) even where the tensor's maximum is set by the
other tail.  (A floor of 1 rather than the column's own maximum: in the
negative tail the exact GeLU is below fp32's smallest normal, and fp32 must
round it to zero.)
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import ref
from tests.gpu_util import assert_close, empty, empty_f32, need_gpu, sync, to_dev, to_f64

pytestmark = pytest.mark.gpu

import linear_layers_amd as tl  # noqa: E402

T, h, F, tp = 256, 64, 256, 2
Fs = F // tp


def _inputs(seed):
    r = np.random.default_rng(seed)
    X = r.standard_normal((T, h)).astype(np.float32)
    W1 = (0.05 * r.standard_normal((h, F))).astype(np.float32)
    W2 = (0.05 * r.standard_normal((F, h))).astype(np.float32)
    dZ = r.standard_normal((T, h)).astype(np.float32)
    b1 = np.tile(np.linspace(-70.0, 70.0, Fs), tp).astype(np.float32)   # every shard spans both tails
    return X, W1, b1, W2, dZ


def _per_column(got, want, what, axis=0):
    """Each column (each entry for a vector) within 1e-5 of max(1, max|ref| over it)."""
    got, want = np.atleast_2d(got), np.atleast_2d(want)
    err = np.abs(got - want).max(axis=axis)
    scale = np.maximum(1.0, np.abs(want).max(axis=axis))
    bad = np.nonzero(~(err <= 1e-5 * scale))[0]
    assert bad.size == 0, f"{what}: columns {bad[:8].tolist()} off by {err[bad[:8]].tolist()}"


def test_column_parallel_gelu_tails_fp32():
    need_gpu()
    X, W1, b1, _, _ = _inputs(51)
    Xd, W1d, b1d = to_dev(X, "f32"), to_dev(W1, "f32"), to_dev(b1, "f32")
    for i in range(tp):
        print(f"column fwd shard {i}", flush=True)
        Y, H = empty_f32((T, Fs)), empty_f32((T, Fs))
        tl.column_parallel_fwd(Xd, W1d[:, i * Fs:(i + 1) * Fs], tp, Y, bias_shard=b1d[i * Fs:(i + 1) * Fs], H_save=H)
        sync()
        Hr, Yr = ref.column_parallel_fwd(X.astype(np.float64), W1.astype(np.float64), b1.astype(np.float64), tp, i)
        assert np.abs(Hr).max() > 64.0 and Hr.min() < -64.0, "the pre-activations must pass the clamp"
        assert_close(to_f64(H), Hr, "f32", "H")
        assert_close(to_f64(Y), Yr, "f32", "GeLU(H)")
        _per_column(to_f64(Y), Yr, f"GeLU(H) shard {i}")
        Yg = to_f64(Y)
        assert np.isfinite(Yg).all()
        neg = Hr < -12.0   # exact GeLU below fp32's normal range: must come out as (signed) zero
        assert np.all(np.abs(Yg[neg]) < 1e-30)


def test_mlp_fwd_bwd_gelu_tails_fp32():
    need_gpu()
    X, W1, b1, W2, dZ = _inputs(52)
    Xd, W1d, b1d, W2d, dZd = (to_dev(a, "f32") for a in (X, W1, b1, W2, dZ))
    f64 = [a.astype(np.float64) for a in (X, W1, b1, W2, dZ)]
    for i in range(tp):
        print(f"mlp fwd+bwd shard {i}", flush=True)
        cols = slice(i * Fs, (i + 1) * Fs)
        A, H, Z = empty_f32((T, Fs)), empty_f32((T, Fs)), empty_f32((T, h))
        tl.tp_mlp_fwd(Xd, W1d[:, cols], b1d[cols], W2d[cols], tp, A, Z, H_save=H)
        dX, dW1, db1, dW2 = empty_f32((T, h)), empty_f32((h, Fs)), empty_f32((Fs,)), empty_f32((Fs, h))
        tl.tp_mlp_bwd(Xd, W1d[:, cols], W2d[cols], H, A, dZd, tp, dX, dW1, dW2, db1_shard=db1)
        sync()
        o = ref.tp_mlp_fwd_shard(f64[0], f64[1], f64[2], f64[3], tp, i)
        g = ref.tp_mlp_bwd_shard(f64[0], f64[1], f64[2], f64[3], f64[4], tp, i)
        for name, got, want in (("A", A, o["A"]), ("Z", Z, o["Z"]), ("dX", dX, g["dX"]), ("dW1", dW1, g["dW1"]),
                                ("db1", db1, g["db1"]), ("dW2", dW2, g["dW2"])):
            assert_close(to_f64(got), want, "f32", f"{name} shard {i}")
        _per_column(to_f64(A), o["A"], f"A shard {i}")
        _per_column(to_f64(dW1), g["dW1"], f"dW1 shard {i}")
        _per_column(to_f64(db1)[None, :], g["db1"][None, :], f"db1 shard {i}")
        # saturated columns: GeLU' is 1 on the right (dH = dA) and 0 on the left (dH = 0)
        lo = b1[cols] < -12.0
        assert np.all(np.abs(to_f64(db1)[lo]) < 1e-30) and np.all(np.abs(to_f64(dW1)[:, lo]) < 1e-30)
