"""GPU parity of the sequence-parallel region (LayerNorm, the reduce-scatter
fused with dropout and residual, the dropout backward) against the float64
oracle, and of the whole SP block chained through the tensor-parallel MLP.

Bars: bf16 outputs max|err|/max|ref| <= 2e-2.  fp32 outputs of fp32
reductions (row statistics, dX of LayerNorm, dgamma/dbeta): |err| <= 1e-5 of
the reduction's natural scale, i.e. the sum of the absolute values of its
terms (an fp32 sum of n terms accumulated in short chains is off by a few
units of 2^-24 of that scale).  Dropout keep decisions are integer results:
they must match the oracle's mask exactly.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from oracle import ref
from oracle import sp
from tests.gpu_util import assert_close, empty, empty_f32, need_gpu, sync, to_dev, to_f64

pytestmark = pytest.mark.gpu

import linear_layers_amd as tl  # noqa: E402


def _say(msg):
    print(msg, flush=True)


def _bf16(a):
    return synth.bf16_round_bits(np.asarray(a, dtype=np.float32))


def _f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _within(got, want, scale, what, tol=1e-5):
    err = float(np.max(np.abs(np.asarray(got) - np.asarray(want)) / np.maximum(scale, 1e-30)))
    assert np.all(np.isfinite(got)) and err <= tol, f"{what}: error {err:.3e} of the reduction scale > {tol:.0e}"


@pytest.mark.parametrize("rows,h,ld_extra", [(1, 8, 0), (37, 264, 16), (1024, 4096, 0), (5, 16384, 8), (0, 64, 0)])
def test_layernorm_fwd_bwd(rows, h, ld_extra):
    need_gpu()
    _say(f"layernorm rows={rows} h={h}")
    r = np.random.default_rng(rows * 7 + h)
    X = _bf16(r.standard_normal((rows, h)) * 1.5 + 0.3)
    g = (1.0 + 0.2 * r.standard_normal(h)).astype(np.float32)
    b = (0.1 * r.standard_normal(h)).astype(np.float32)
    dY = r.standard_normal((rows, h)).astype(np.float32)
    dRes = _bf16(r.standard_normal((rows, h)))
    fX = synth.to_f64(X, "bf16")
    ld = h + ld_extra
    Xd = empty((rows, ld), "bf16")[:, :h]
    Xd.copy_(to_dev(X, "bf16"))
    Y = empty((rows + 2, ld), "bf16")       # written into rows [1, rows + 1) of a larger buffer
    mean, rstd = empty_f32((rows,)), empty_f32((rows,))
    tl.layernorm_fwd(Xd, _f32(g), _f32(b), Y[1:rows + 1, :h], mean, rstd)
    dX = empty_f32((rows, h))
    dgam, dbet = empty_f32((h,)), empty_f32((h,))
    tl.layernorm_bwd(Xd, _f32(g), mean, rstd, _f32(dY), dX, dgamma=dgam, dbeta=dbet, dRes=to_dev(dRes, "bf16"))
    sync()
    assert torch.isnan(Y[0]).all() and torch.isnan(Y[rows + 1]).all(), "rows outside the block were written"
    f = sp.layernorm_fwd(fX, g, b)
    d = sp.layernorm_bwd(fX, g, dY)
    if rows == 0:
        assert not to_f64(dgam).any() and not to_f64(dbet).any()
        return
    assert_close(to_f64(Y[1:rows + 1, :h]), f["Y"], "bf16", "Y")
    _within(to_f64(mean), f["mean"], np.abs(fX).mean(axis=1), "mean")
    _within(to_f64(rstd), f["rstd"], f["rstd"], "rstd")
    gd = dY * g[None, :]
    dx_scale = f["rstd"][:, None] * (np.abs(gd).mean(axis=1) + np.abs(gd * f["xhat"]).mean(axis=1) * np.abs(
        f["xhat"]).max(axis=1))[:, None]
    _within(to_f64(dX), d["dX"] + synth.to_f64(dRes, "bf16"), dx_scale + np.abs(synth.to_f64(dRes, "bf16")), "dX")
    _within(to_f64(dgam), d["dgamma"], np.abs(dY * f["xhat"]).sum(axis=0), "dgamma")
    _within(to_f64(dbet), d["dbeta"], np.abs(dY).sum(axis=0), "dbeta")


@pytest.mark.parametrize("tp,rows,h,row0,p", [(1, 3, 8, 0, 0.0), (3, 77, 264, 5, 0.1), (8, 64, 1024, 1000, 0.5),
                                              (2, 0, 64, 0, 0.3)])
def test_sp_partial_sum_dropout_residual(tp, rows, h, row0, p):
    need_gpu()
    _say(f"sp sum+dropout tp={tp} rows={rows} h={h} row0={row0} p={p}")
    r = np.random.default_rng(tp * 100 + rows)
    seed = 0x1234_5678_9ABC + rows
    parts = r.standard_normal((tp, rows + 4, h)).astype(np.float32)   # this GPU's rows start at row 2
    res = _bf16(r.standard_normal((rows, h)))
    P = _f32(parts)
    out = empty((rows, h), "bf16")
    tl.sp_partial_sum_dropout_residual(P[:, 2:rows + 2], to_dev(res, "bf16"), out, p, seed, row0)
    # the keep decisions themselves, through the dropout backward of a ones tensor
    ones = torch.ones((rows, h), dtype=torch.bfloat16, device="cuda")
    dZ = empty((rows, h), "bf16")
    tl.sp_dropout_bwd(ones, dZ, p, seed, row0)
    sync()
    keep = sp.dropout_keep(seed, row0, rows, h, p)
    assert np.array_equal(to_f64(dZ) != 0.0, keep), "dropout mask differs from the oracle's"
    if rows == 0:
        return
    want = sp.partial_sum_dropout_residual([parts[s, 2:rows + 2].astype(np.float64) for s in range(tp)],
                                           synth.to_f64(res, "bf16"), p, seed, row0)
    assert_close(to_f64(out), want, "bf16", "out")


def test_sp_dropout_bwd_values():
    need_gpu()
    rows, h, row0, p, seed = 100, 512, 3, 0.2, 42
    r = np.random.default_rng(9)
    dOut = _bf16(r.standard_normal((rows, h)))
    dZ = empty((rows + 10, h), "bf16")
    tl.sp_dropout_bwd(to_dev(dOut, "bf16"), dZ[10:], p, seed, row0)
    sync()
    assert torch.isnan(dZ[:10]).all()
    assert_close(to_f64(dZ[10:]), sp.dropout_bwd(synth.to_f64(dOut, "bf16"), p, seed, row0), "bf16", "dZ")


@pytest.mark.parametrize("T,h,F,tp,p", [(64, 128, 512, 4, 0.1), (200, 264, 640, 2, 0.0)])
def test_sp_mlp_block_chain(T, h, F, tp, p):
    """The whole SP block on one GPU, rank by rank: LayerNorm of each rank's rows
    into the gathered input, every TP shard's MLP, each rank's reduce-scatter
    with dropout and residual; then the backward through the same chain."""
    need_gpu()
    _say(f"sp block T={T} h={h} F={F} tp={tp} p={p}")
    seed = 2024
    wl = synth.Workload("sp", 31, "bf16", T=T, h=h, F=F, tp=1, w_std=0.05, b_std=0.1, dz_std=1.0)
    raw = synth.mlp_inputs(wl)
    f = {k: synth.to_f64(v, "bf16") for k, v in raw.items()}
    r = np.random.default_rng(5)
    g = (1.0 + 0.1 * r.standard_normal(h)).astype(np.float32)
    b = (0.1 * r.standard_normal(h)).astype(np.float32)
    rows, Fs = T // tp, F // tp
    X, W1, b1, W2, dOut = (to_dev(raw[k], "bf16") for k in ("X", "W1", "b1", "W2", "dZ"))
    gd, bd = _f32(g), _f32(b)
    Ygath = empty((T, h), "bf16")
    means, rstds = empty_f32((T,)), empty_f32((T,))
    for i in range(tp):
        sl = slice(i * rows, (i + 1) * rows)
        tl.layernorm_fwd(X[sl], gd, bd, Ygath[sl], means[sl], rstds[sl])
    Zp = empty_f32((tp, T, h))
    As, Hs = [], []
    for j in range(tp):
        A, H = empty((T, Fs), "bf16"), empty((T, Fs), "bf16")
        tl.tp_mlp_fwd(Ygath, W1[:, j * Fs:(j + 1) * Fs], b1[j * Fs:(j + 1) * Fs], W2[j * Fs:(j + 1) * Fs].contiguous(),
                      tp, A, Zp[j], H_save=H)
        As.append(A)
        Hs.append(H)
    out = empty((T, h), "bf16")
    for i in range(tp):
        sl = slice(i * rows, (i + 1) * rows)
        tl.sp_partial_sum_dropout_residual(Zp[:, sl], X[sl], out[sl], p, seed, i * rows)
    # backward
    dZg = empty((T, h), "bf16")
    for i in range(tp):
        sl = slice(i * rows, (i + 1) * rows)
        tl.sp_dropout_bwd(dOut[sl], dZg[sl], p, seed, i * rows)
    dXp = empty_f32((tp, T, h))
    for j in range(tp):
        dW1, dW2 = empty_f32((h, Fs)), empty_f32((Fs, h))
        tl.tp_mlp_bwd(Ygath, W1[:, j * Fs:(j + 1) * Fs], W2[j * Fs:(j + 1) * Fs].contiguous(), Hs[j], As[j], dZg, tp,
                      dXp[j], dW1, dW2)
    dX = empty_f32((T, h))
    dgam, dbet = torch.zeros((h,), device="cuda"), torch.zeros((h,), device="cuda")
    for i in range(tp):
        sl = slice(i * rows, (i + 1) * rows)
        dY = empty_f32((rows, h))
        tl.shard_partial_sum(dXp[:, sl], dY)
        dg_i, db_i = empty_f32((h,)), empty_f32((h,))
        tl.layernorm_bwd(X[sl], gd, means[sl], rstds[sl], dY, dX[sl], dgamma=dg_i, dbeta=db_i, dRes=dOut[sl])
        dgam += dg_i
        dbet += db_i
    sync()
    whole = sp.sp_block_fwd(f["X"], g, b, lambda Yf: ref.mlp_fwd(Yf, f["W1"], f["b1"], f["W2"])["Z"], p, seed)
    assert_close(to_f64(Ygath), whole["Y"], "bf16", "gathered LayerNorm output")
    assert_close(to_f64(out), whole["out"], "bf16", "block output")
    # backward reference: the same composition in float64
    keep = sp.dropout_keep(seed, 0, T, h, p)
    dZ = np.where(keep, f["dZ"] * sp.dropout_scale(p), 0.0)
    mb = ref.mlp_bwd(whole["Y"], f["W1"], f["b1"], f["W2"], dZ)
    lb = sp.layernorm_bwd(f["X"], g, mb["dX"])
    assert_close(to_f64(dZg), dZ, "bf16", "gathered dZ")
    assert_close(to_f64(dX), lb["dX"] + f["dZ"], "bf16", "dX of the block")
    assert_close(to_f64(dgam), lb["dgamma"], "bf16", "dgamma")
    assert_close(to_f64(dbet), lb["dbeta"], "bf16", "dbeta")


@pytest.mark.slow
def test_sp_llama7b_rank_block():
    """One rank's SP kernels at the Llama-7B-scale shapes: 1024 of 8192 rows, h=4096, tp=8."""
    need_gpu()
    wl = synth.WORKLOADS["llama7b_bf16"]
    T, h, tp = wl.T, wl.h, wl.tp
    rows, row0, p, seed = T // tp, 3 * (T // tp), 0.1, 77
    _say(f"sp rank block rows={rows} h={h} row0={row0}")
    r = np.random.default_rng(11)
    X = _bf16(r.standard_normal((rows, h)))
    g = (1.0 + 0.1 * r.standard_normal(h)).astype(np.float32)
    b = (0.1 * r.standard_normal(h)).astype(np.float32)
    parts = (0.05 * r.standard_normal((tp, rows, h))).astype(np.float32)
    Xd = to_dev(X, "bf16")
    Y, mean, rstd = empty((rows, h), "bf16"), empty_f32((rows,)), empty_f32((rows,))
    tl.layernorm_fwd(Xd, _f32(g), _f32(b), Y, mean, rstd)
    out = empty((rows, h), "bf16")
    tl.sp_partial_sum_dropout_residual(_f32(parts), Xd, out, p, seed, row0)
    sync()
    fX = synth.to_f64(X, "bf16")
    assert_close(to_f64(Y), sp.layernorm_fwd(fX, g, b)["Y"], "bf16", "Y")
    want = sp.partial_sum_dropout_residual([parts[s].astype(np.float64) for s in range(tp)], fX, p, seed, row0)
    assert_close(to_f64(out), want, "bf16", "out")
