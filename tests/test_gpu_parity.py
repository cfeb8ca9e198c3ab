"""GPU parity of every libtpmlp entry point against the float64 oracle.

Sizes here are small enough for the full oracle, yet span several tiles with
ragged tails (T, widths not multiples of the 128/256 tiles), empty batches,
views with ld > width, and both storage types.  Tolerances: max|err|/max|ref|
<= 2e-2 for bf16 storage and <= 1e-5 for fp32 storage.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from oracle import ref
from tests.gpu_util import TOL, assert_close, empty, empty_f32, need_gpu, sync, to_dev, to_f64

pytestmark = pytest.mark.gpu

import linear_layers_amd as tl  # noqa: E402  (after the gpu mark; import needs the built library)


def _inputs(dtype, T, h, F, seed, bias=True, x_std=1.0, w_std=0.05):
    wl = synth.Workload("t", seed, dtype, T=T, h=h, F=F, tp=1, x_std=x_std, w_std=w_std,
                        b_std=0.1 if bias else None, dz_std=1.0)
    raw = synth.mlp_inputs(wl)
    f64 = {k: synth.to_f64(v, dtype) for k, v in raw.items()}
    return raw, f64


SHAPES = [
    # dtype, T, h, F, tp
    ("bf16", 300, 264, 656, 2),
    ("bf16", 513, 512, 2048, 4),
    ("bf16", 1, 16, 32, 2),
    ("bf16", 77, 136, 24, 3),
    # h = 4096, F/tp = 2048: the two weight gradients run as one paired launch
    # (128 + 128 tiles of 256x256), with a ragged K = T
    ("bf16", 300, 4096, 4096, 2),
    ("f32", 128, 256, 1024, 2),
    ("f32", 45, 20, 24, 2),
]


@pytest.mark.parametrize("dtype,T,h,F,tp", SHAPES)
@pytest.mark.parametrize("bias", [True, False])
def test_tp_mlp_fwd(dtype, T, h, F, tp, bias):
    need_gpu()
    raw, f = _inputs(dtype, T, h, F, seed=T + h + F, bias=bias)
    Fs = F // tp
    X, W1, W2 = to_dev(raw["X"], dtype), to_dev(raw["W1"], dtype), to_dev(raw["W2"], dtype)
    b1 = to_dev(raw["b1"], dtype) if bias else None
    for i in range(tp):
        W1_i = W1[:, i * Fs:(i + 1) * Fs]                   # view, ld = F
        W2_i = W2[i * Fs:(i + 1) * Fs]
        b1_i = b1[i * Fs:(i + 1) * Fs] if bias else None
        A, H, Z = empty((T, Fs), dtype), empty((T, Fs), dtype), empty_f32((T, h))
        tl.tp_mlp_fwd(X, W1_i, b1_i, W2_i, tp, A, Z, H_save=H)
        sync()
        o = ref.tp_mlp_fwd_shard(f["X"], f["W1"], f.get("b1"), f["W2"], tp, i)
        assert_close(to_f64(H), o["H"], dtype, f"H_{i}")
        assert_close(to_f64(A), o["A"], dtype, f"A_{i}")
        assert_close(to_f64(Z), o["Z"], dtype, f"Z_{i}")


@pytest.mark.parametrize("dtype,T,h,F,tp", SHAPES)
def test_tp_mlp_bwd(dtype, T, h, F, tp):
    need_gpu()
    raw, f = _inputs(dtype, T, h, F, seed=7 * T + h, bias=True)
    Fs = F // tp
    X, W1, W2 = to_dev(raw["X"], dtype), to_dev(raw["W1"], dtype), to_dev(raw["W2"], dtype)
    b1, dZ = to_dev(raw["b1"], dtype), to_dev(raw["dZ"], dtype)
    for i in range(tp):
        W1_i, W2_i, b1_i = W1[:, i * Fs:(i + 1) * Fs], W2[i * Fs:(i + 1) * Fs], b1[i * Fs:(i + 1) * Fs]
        A, H, Z = empty((T, Fs), dtype), empty((T, Fs), dtype), empty_f32((T, h))
        tl.tp_mlp_fwd(X, W1_i, b1_i, W2_i, tp, A, Z, H_save=H)
        dX, dW1, db1, dW2 = empty_f32((T, h)), empty_f32((h, Fs)), empty_f32((Fs,)), empty_f32((Fs, h))
        tl.tp_mlp_bwd(X, W1_i, W2_i, H, A, dZ, tp, dX, dW1, dW2, db1_shard=db1)
        sync()
        o = ref.tp_mlp_bwd_shard(f["X"], f["W1"], f["b1"], f["W2"], f["dZ"], tp, i)
        assert_close(to_f64(dX), o["dX"], dtype, f"dX_{i}")
        assert_close(to_f64(dW1), o["dW1"], dtype, f"dW1_{i}")
        assert_close(to_f64(db1), o["db1"], dtype, f"db1_{i}")
        assert_close(to_f64(dW2), o["dW2"], dtype, f"dW2_{i}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_tp_invariance_and_partial_sum(dtype):
    """Sum over shards of Z_i equals the unsharded block for tp in {1, 2, 4, 8}."""
    need_gpu()
    T, h, F = 200, 128, 512
    raw, f = _inputs(dtype, T, h, F, seed=99, bias=True)
    Zfull = ref.mlp_fwd(f["X"], f["W1"], f["b1"], f["W2"])["Z"]
    X, W1, W2, b1 = (to_dev(raw[k], dtype) for k in ("X", "W1", "W2", "b1"))
    sums = {}
    for tp in (1, 2, 4, 8):
        Fs = F // tp
        parts = empty_f32((tp, T, h))
        for i in range(tp):
            A = empty((T, Fs), dtype)
            tl.tp_mlp_fwd(X, W1[:, i * Fs:(i + 1) * Fs], b1[i * Fs:(i + 1) * Fs], W2[i * Fs:(i + 1) * Fs], tp, A,
                          parts[i])
        out = empty_f32((T, h))
        tl.shard_partial_sum(parts, out)
        sync()
        sums[tp] = to_f64(out)
        assert_close(sums[tp], Zfull, dtype, f"sum of partials tp={tp}")
        # The sum is fp32, ascending in shard index: bit-identical to numpy's.
        p = parts.cpu().numpy()
        acc = p[0].copy()
        for i in range(1, tp):
            acc = (acc + p[i]).astype(np.float32)
        assert np.array_equal(out.cpu().numpy(), acc), "partial sum is not the ascending fp32 sum"
    # A is computed identically for every tp (same K order), so tp-invariance
    # holds up to fp32 reassociation of the second product and the sum.
    for tp in (2, 4, 8):
        assert_close(sums[tp], sums[1], "f32", f"tp={tp} vs tp=1", tol=1e-5)


@pytest.mark.parametrize("tp,T,N", [(1, 5, 4), (2, 128, 256), (3, 77, 36), (8, 1000, 1032), (4, 0, 64)])
def test_shard_partial_sum(tp, T, N):
    need_gpu()
    rng = np.random.default_rng(tp * 1000 + T)
    P = rng.standard_normal((tp, T, N), dtype=np.float32)
    parts = torch.from_numpy(P).cuda()
    out = empty_f32((T, N))
    tl.shard_partial_sum(parts, out)
    sync()
    expect = ref.shard_partial_sum([P[i] for i in range(tp)])
    assert_close(to_f64(out), expect, "f32", "partial sum")
    # in place into partial 0
    tl.shard_partial_sum(parts, parts[0])
    sync()
    assert np.array_equal(parts[0].cpu().numpy(), out.cpu().numpy())


def test_partial_sum_row_subrange_and_strides():
    """One GPU's share of a reduce-scatter: rows [r0, r1) of each partial, interleaved layout."""
    need_gpu()
    tp, T, N = 4, 96, 64
    rng = np.random.default_rng(5)
    P = rng.standard_normal((T, tp, N), dtype=np.float32)  # [T][tp][N] layout
    dev = torch.from_numpy(P).cuda()
    view = dev.permute(1, 0, 2)                            # [tp, T, N], shard stride N, row stride tp*N
    out = empty_f32((24, N))
    tl.shard_partial_sum(view[:, 24:48], out)
    sync()
    expect = ref.shard_partial_sum([P[24:48, i] for i in range(tp)])
    assert_close(to_f64(out), expect, "f32", "row sub-range partial sum")


@pytest.mark.parametrize("dtype,T,K,N,tp", [("bf16", 300, 264, 656, 2), ("bf16", 64, 128, 3 * 128, 3),
                                            ("f32", 50, 36, 48, 2)])
@pytest.mark.parametrize("act", ["gelu_tanh", "none"])
def test_column_parallel_fwd(dtype, T, K, N, tp, act):
    need_gpu()
    wl = synth.Workload("c", 11, dtype, T=T, h=K, F=N, tp=tp, b_std=0.1)
    raw = synth.mlp_inputs(wl, which=("X", "W1", "b1"))
    f = {k: synth.to_f64(v, dtype) for k, v in raw.items()}
    X, W, b = (to_dev(raw[k], dtype) for k in ("X", "W1", "b1"))
    Ns = N // tp
    for i in range(tp):
        Wp = W[:, i * Ns:(i + 1) * Ns].contiguous()        # packed shard, ld = N/tp
        Y, H = empty((T, Ns), dtype), empty((T, Ns), dtype)
        tl.column_parallel_fwd(X, Wp, tp, Y, bias_shard=b[i * Ns:(i + 1) * Ns], H_save=H, act=act)
        Yv = empty((T, Ns), dtype)
        tl.column_parallel_fwd(X, W[:, i * Ns:(i + 1) * Ns], tp, Yv, bias_shard=b[i * Ns:(i + 1) * Ns], act=act)
        sync()
        Hr, Yr = ref.column_parallel_fwd(f["X"], f["W1"], f["b1"], tp, i, act)
        assert_close(to_f64(H), Hr, dtype, "H")
        assert_close(to_f64(Y), Yr, dtype, "Y")
        assert torch.equal(Y, Yv), "view and packed shard differ"


@pytest.mark.parametrize("dtype,T,K,N,tp", [("bf16", 300, 656, 264, 2), ("bf16", 1, 64, 64, 4), ("f32", 50, 48, 36, 3)])
def test_row_parallel_fwd_and_bwd(dtype, T, K, N, tp):
    need_gpu()
    Xr = synth.draw(12, 50, (T, K), 1.0, dtype)
    Wr = synth.draw(12, 51, (K, N), 0.05, dtype)
    dYr = synth.draw(12, 52, (T, N), 1.0, dtype)
    fX, fW, fdY = synth.to_f64(Xr, dtype), synth.to_f64(Wr, dtype), synth.to_f64(dYr, dtype)
    X, W, dY = to_dev(Xr, dtype), to_dev(Wr, dtype), to_dev(dYr, dtype)
    Ks = K // tp
    for i in range(tp):
        Z = empty_f32((T, N))
        tl.row_parallel_fwd(X[:, i * Ks:(i + 1) * Ks], W[i * Ks:(i + 1) * Ks], tp, Z)
        dX, dW = empty_f32((T, Ks)), empty_f32((Ks, N))
        tl.row_parallel_bwd(X[:, i * Ks:(i + 1) * Ks], W[i * Ks:(i + 1) * Ks], dY, tp, dX, dW)
        sync()
        assert_close(to_f64(Z), ref.row_parallel_fwd(fX, fW, tp, i), dtype, "Z_i")
        g = ref.row_parallel_bwd(fX[:, i * Ks:(i + 1) * Ks], ref.row_shard(fW, tp, i), fdY)
        assert_close(to_f64(dX), g["dX"], dtype, "dX_i")
        assert_close(to_f64(dW), g["dW"], dtype, "dW_i")


@pytest.mark.parametrize("dtype,T,K,N,tp", [("bf16", 300, 264, 656, 2), ("bf16", 130, 128, 384, 3),
                                            ("f32", 50, 36, 48, 2)])
@pytest.mark.parametrize("with_bias", [True, False])
def test_column_parallel_bwd(dtype, T, K, N, tp, with_bias):
    need_gpu()
    Xr = synth.draw(13, 0, (T, K), 1.0, dtype)
    Wr = synth.draw(13, 1, (K, N), 0.05, dtype)
    Ns = N // tp
    fX, fW = synth.to_f64(Xr, dtype), synth.to_f64(Wr, dtype)
    X, W = to_dev(Xr, dtype), to_dev(Wr, dtype)
    for i in range(tp):
        dYr = synth.draw(13, 10 + i, (T, Ns), 1.0, dtype)
        dY = to_dev(dYr, dtype)
        dX, dW = empty_f32((T, K)), empty_f32((K, Ns))
        db = empty_f32((Ns,)) if with_bias else None
        tl.column_parallel_bwd(X, W[:, i * Ns:(i + 1) * Ns], dY, tp, dX, dW, db_shard=db)
        sync()
        g = ref.column_parallel_bwd(fX, ref.col_shard(fW, tp, i), synth.to_f64(dYr, dtype), with_bias=True)
        assert_close(to_f64(dX), g["dX"], dtype, "dX_partial")
        assert_close(to_f64(dW), g["dW"], dtype, "dW")
        if with_bias:
            assert_close(to_f64(db), g["db"], dtype, "db")


def test_empty_batch():
    need_gpu()
    dtype, T, h, F, tp = "bf16", 0, 64, 128, 2
    Fs = F // tp
    X = torch.empty((0, h), dtype=torch.bfloat16, device="cuda")
    W1 = to_dev(synth.draw(1, 1, (h, Fs), 0.05, dtype), dtype)
    W2 = to_dev(synth.draw(1, 2, (Fs, h), 0.05, dtype), dtype)
    A, H, Z = empty((0, Fs), dtype), empty((0, Fs), dtype), empty_f32((0, h))
    tl.tp_mlp_fwd(X, W1, None, W2, tp, A, Z, H_save=H)
    dX, dW1, db1, dW2 = empty_f32((0, h)), empty_f32((h, Fs)), empty_f32((Fs,)), empty_f32((Fs, h))
    tl.tp_mlp_bwd(X, W1, W2, H, A, torch.empty((0, h), dtype=torch.bfloat16, device="cuda"), tp, dX, dW1, dW2,
                  db1_shard=db1)
    sync()
    # sums over an empty batch are zero
    assert torch.count_nonzero(dW1).item() == 0 and torch.count_nonzero(dW2).item() == 0
    assert torch.count_nonzero(db1).item() == 0


def test_errors_leave_outputs_untouched():
    need_gpu()
    dtype, T, h, F, tp = "bf16", 64, 64, 128, 2
    Fs = F // tp
    X = to_dev(synth.draw(2, 0, (T, h), 1.0, dtype), dtype)
    W1 = to_dev(synth.draw(2, 1, (h, Fs), 0.05, dtype), dtype)
    W2 = to_dev(synth.draw(2, 2, (Fs, h), 0.05, dtype), dtype)
    A, Z = empty((T, Fs), dtype, fill=7.0), empty_f32((T, h), fill=7.0)
    st = tl.lib.tp_mlp_fwd(torch.cuda.current_stream().cuda_stream, 1, T, h, F, 3, X.data_ptr(), W1.data_ptr(),
                           Fs, None, W2.data_ptr(), None, A.data_ptr(), Z.data_ptr())
    assert st == 3  # TPMLP_E_DIVISIBILITY
    st = tl.lib.tp_mlp_fwd(torch.cuda.current_stream().cuda_stream, 1, T, h, F, tp, X.data_ptr() + 2,
                           W1.data_ptr(), Fs, None, W2.data_ptr(), None, A.data_ptr(), Z.data_ptr())
    assert st == 4  # TPMLP_E_ALIGNMENT
    st = tl.lib.tp_mlp_fwd(torch.cuda.current_stream().cuda_stream, 7, T, h, F, tp, X.data_ptr(),
                           W1.data_ptr(), Fs, None, W2.data_ptr(), None, A.data_ptr(), Z.data_ptr())
    assert st == 5  # TPMLP_E_DTYPE
    sync()
    assert torch.all(A == 7.0).item() and torch.all(Z == 7.0).item()


def test_bitwise_deterministic():
    need_gpu()
    dtype, T, h, F, tp = "bf16", 515, 256, 1024, 2
    raw, _ = _inputs(dtype, T, h, F, seed=3, bias=True)
    Fs = F // tp
    X, W1, W2, b1, dZ = (to_dev(raw[k], dtype) for k in ("X", "W1", "W2", "b1", "dZ"))
    outs = []
    for _ in range(2):
        A, H, Z = empty((T, Fs), dtype), empty((T, Fs), dtype), empty_f32((T, h))
        tl.tp_mlp_fwd(X, W1[:, :Fs], b1[:Fs], W2[:Fs], tp, A, Z, H_save=H)
        dX, dW1, db1, dW2 = empty_f32((T, h)), empty_f32((h, Fs)), empty_f32((Fs,)), empty_f32((Fs, h))
        tl.tp_mlp_bwd(X, W1[:, :Fs], W2[:Fs], H, A, dZ, tp, dX, dW1, dW2, db1_shard=db1)
        sync()
        outs.append([t.clone() for t in (A, H, Z, dX, dW1, db1, dW2)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_profiler_times_and_clocks():
    """Profiling brackets each launch with events; bf16 GEMMs also report the
    shader clock of workgroup 0's main loop.  Results stay bitwise equal to
    an unprofiled run."""
    need_gpu()
    dtype, T, h, F, tp = "bf16", 515, 256, 1024, 2
    raw, _ = _inputs(dtype, T, h, F, seed=4, bias=True)
    Fs = F // tp
    X, W1, W2, b1 = (to_dev(raw[k], dtype) for k in ("X", "W1", "W2", "b1"))

    def run():
        A, Z = empty((T, Fs), dtype), empty_f32((T, h))
        tl.tp_mlp_fwd(X, W1[:, :Fs], b1[:Fs], W2[:Fs], tp, A, Z)
        sync()
        return A, Z

    A0, Z0 = run()
    tl.profile_enable("gemm")
    try:
        A1, Z1 = run()
        recs = tl.profile_collect()
    finally:
        tl.profile_enable(None)
    assert torch.equal(A0, A1) and torch.equal(Z0, Z1)
    roles = {k.split("|")[0] for k in recs}
    assert roles == {"gemm.mlp_fwd1", "gemm.mlp_fwd2"}
    for n, ms, sym, clocks in recs.values():
        assert n == 1 and ms > 0.0 and sym.startswith(("gemm_bf16_kernel<", "gemm_w4_kernel<"))
        assert len(clocks) == 1 and 0.05 < clocks[0] < 5.0
    assert tl.profile_collect() == {}
