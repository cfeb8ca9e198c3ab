"""GPU parity of the attention core against the float64 oracle.

Small shapes (ragged sequence lengths, several heads and sequences, the fused
QKV layout and separate strided Q/K/V) run the whole oracle; the
workload-sized shard (one sequence of 4096 tokens, 10 heads of 128, causal)
is checked on sampled query rows of every head.  Bars: bf16 outputs
max|err|/max|ref| <= 2e-2; the fp32 log-sum-exp |err| <= 1e-4 * max(1, |lse|)
(scores from bf16 inputs, fp32 exp2/log2 and sums of up to seq terms).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from oracle import attn as oat
from tests.gpu_util import assert_close, empty, empty_f32, need_gpu, sync, to_dev, to_f64

pytestmark = pytest.mark.gpu

import linear_layers_amd as tl  # noqa: E402

D = 128


def _say(msg):
    print(msg, flush=True)


def _lse_close(got, want, what):
    err = np.abs(np.asarray(got) - want) / np.maximum(1.0, np.abs(want))
    assert np.all(np.isfinite(got)) and err.max() <= 1e-4, f"{what}: lse error {err.max():.3e}"


def _qkv(seed, T, heads, std=1.0):
    """A fused [T, 3*heads*128] QKV tensor (bf16 bits) as the column projection writes it."""
    r = np.random.default_rng(seed)
    return synth.bf16_round_bits((r.standard_normal((T, 3 * heads * D)) * std).astype(np.float32))


@pytest.mark.parametrize("batch,seq,heads,causal", [(1, 1, 1, True), (2, 77, 3, True), (2, 77, 3, False),
                                                    (1, 300, 2, True), (1, 300, 2, False), (3, 128, 1, True),
                                                    (1, 1000, 2, True)])
def test_attn_fwd_fused_qkv(batch, seq, heads, causal):
    need_gpu()
    _say(f"attn fwd batch={batch} seq={seq} heads={heads} causal={causal}")
    T, w = batch * seq, heads * D
    qkv = _qkv(batch * 1000 + seq, T, heads)
    dev = to_dev(qkv, "bf16")
    O = empty((T, w), "bf16")
    lse = empty_f32((heads, T))
    tl.attn_fwd(dev[:, :w], dev[:, w:2 * w], dev[:, 2 * w:], O, batch, seq, heads, causal=causal, lse=lse)
    sync()
    f = synth.to_f64(qkv, "bf16")
    ref = oat.attn_fwd(f[:, :w], f[:, w:2 * w], f[:, 2 * w:], batch, seq, heads, D, causal, D ** -0.5)
    assert_close(to_f64(O), ref["O"], "bf16", "O")
    _lse_close(to_f64(lse), ref["lse"], "lse")


def test_attn_fwd_separate_strided_and_scale():
    need_gpu()
    batch, seq, heads, scale = 2, 200, 2, 0.05
    T, w = batch * seq, heads * D
    r = np.random.default_rng(3)
    mats = [synth.bf16_round_bits(r.standard_normal((T, w + 64)).astype(np.float32)) for _ in range(3)]
    Q, K, V = (to_dev(m, "bf16")[:, :w] for m in mats)
    O = empty((T, w + 32), "bf16")
    tl.attn_fwd(Q, K, V, O[:, :w], batch, seq, heads, causal=False, scale=scale)
    sync()
    f = [synth.to_f64(m, "bf16")[:, :w] for m in mats]
    ref = oat.attn_fwd(*f, batch, seq, heads, D, False, scale)
    assert_close(to_f64(O[:, :w]), ref["O"], "bf16", "O")
    assert torch.isnan(O[:, w:]).all(), "columns past the heads were written"


def test_attn_empty_and_errors():
    need_gpu()
    O = torch.empty((0, D), dtype=torch.bfloat16, device="cuda")
    tl.attn_fwd(O, O, O, O, 0, 5, 1)
    Z = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(tl.TpmlpError) as e:
        tl.attn_fwd(Z, Z, Z, Z, 1, 4, 1, head_dim=64)
    assert e.value.status == 2


@pytest.mark.slow
def test_attn_fwd_workload_sampled():
    """One sequence of 4096 tokens, 10 heads of 128 (one of 4 shards of 40 heads), causal: sampled rows."""
    need_gpu()
    seq, heads = 4096, 10
    _say(f"attn fwd seq={seq} heads={heads} (sampled)")
    qkv = _qkv(77, seq, heads)
    dev = to_dev(qkv, "bf16")
    w = heads * D
    O = empty((seq, w), "bf16")
    lse = empty_f32((heads, seq))
    tl.attn_fwd(dev[:, :w], dev[:, w:2 * w], dev[:, 2 * w:], O, 1, seq, heads, causal=True, lse=lse)
    sync()
    f = synth.to_f64(qkv, "bf16")
    r = np.random.default_rng(5)
    rows = np.array(sorted(set(r.choice(seq, 24, replace=False).tolist()) | {0, 127, 128, seq - 1}))
    Og, Lg = to_f64(O), to_f64(lse)
    for hd in range(heads):
        ref = oat.attn_fwd_rows(f[:, :w], f[:, w:2 * w], f[:, 2 * w:], 1, seq, heads, D, True, D ** -0.5, 0, hd,
                                rows)
        assert_close(Og[rows, hd * D:(hd + 1) * D], ref["O"], "bf16", f"O head {hd}")
        _lse_close(Lg[hd, rows], ref["lse"], f"lse head {hd}")


def _bwd_case(batch, seq, heads, causal, seed, scale=None):
    T, w = batch * seq, heads * D
    qkv = _qkv(seed, T, heads)
    r = np.random.default_rng(seed + 1)
    dO = synth.bf16_round_bits(r.standard_normal((T, w)).astype(np.float32))
    dev, dOd = to_dev(qkv, "bf16"), to_dev(dO, "bf16")
    Q, K, V = dev[:, :w], dev[:, w:2 * w], dev[:, 2 * w:]
    O, lse = empty((T, w), "bf16"), empty_f32((heads, T))
    tl.attn_fwd(Q, K, V, O, batch, seq, heads, causal=causal, scale=scale, lse=lse)
    dqkv = empty((T, 3 * w), "bf16")
    tl.attn_bwd(Q, K, V, O, dOd, lse, dqkv[:, :w], dqkv[:, w:2 * w], dqkv[:, 2 * w:], batch, seq, heads,
                causal=causal, scale=scale)
    sync()
    return qkv, dO, dqkv


@pytest.mark.parametrize("batch,seq,heads,causal", [(1, 1, 1, True), (2, 77, 3, True), (2, 77, 3, False),
                                                    (1, 300, 2, True), (1, 130, 1, False), (3, 128, 1, True),
                                                    (1, 1000, 2, True), (1, 1000, 1, False)])
def test_attn_bwd(batch, seq, heads, causal):
    need_gpu()
    _say(f"attn bwd batch={batch} seq={seq} heads={heads} causal={causal}")
    qkv, dO, dqkv = _bwd_case(batch, seq, heads, causal, seed=batch * 100 + seq)
    w = heads * D
    f = synth.to_f64(qkv, "bf16")
    ref = oat.attn_bwd(f[:, :w], f[:, w:2 * w], f[:, 2 * w:], synth.to_f64(dO, "bf16"), batch, seq, heads, D, causal,
                       D ** -0.5)
    g = to_f64(dqkv)
    assert_close(g[:, :w], ref["dQ"], "bf16", "dQ")
    assert_close(g[:, w:2 * w], ref["dK"], "bf16", "dK")
    assert_close(g[:, 2 * w:], ref["dV"], "bf16", "dV")


def test_attn_bwd_deterministic_and_workspace():
    need_gpu()
    a = _bwd_case(1, 200, 2, True, seed=9)[2]
    b = _bwd_case(1, 200, 2, True, seed=9)[2]
    assert torch.equal(a, b)
    assert tl.attn_bwd_workspace_bytes(2, 100, 3) >= 2 * 100 * 3 * 4
    Z = torch.zeros((4, D), dtype=torch.bfloat16, device="cuda")
    L = torch.zeros((1, 4), device="cuda")
    small = torch.zeros(8, dtype=torch.uint8, device="cuda")
    with pytest.raises(tl.TpmlpError) as e:
        tl.attn_bwd(Z, Z, Z, Z, Z, L, Z, Z, Z, 1, 4, 1, workspace=small)
    assert e.value.status == 7


@pytest.mark.slow
def test_attn_bwd_workload_two_heads():
    """4096 tokens, 10 heads, causal: full dQ, dK, dV of heads 0 and 7 against the oracle (heads are
    independent, so each head's gradients come from the oracle run on that head's columns alone)."""
    need_gpu()
    seq, heads = 4096, 10
    _say(f"attn bwd seq={seq} heads={heads}")
    qkv, dO, dqkv = _bwd_case(1, seq, heads, True, seed=123)
    w = heads * D
    f, fd, g = synth.to_f64(qkv, "bf16"), synth.to_f64(dO, "bf16"), to_f64(dqkv)
    for hd in (0, 7):
        cs = slice(hd * D, (hd + 1) * D)
        ref = oat.attn_bwd(f[:, cs], f[:, w:2 * w][:, cs], f[:, 2 * w:][:, cs], fd[:, cs], 1, seq, 1, D, True,
                           D ** -0.5)
        assert_close(g[:, :w][:, cs], ref["dQ"], "bf16", f"dQ head {hd}")
        assert_close(g[:, w:2 * w][:, cs], ref["dK"], "bf16", f"dK head {hd}")
        assert_close(g[:, 2 * w:][:, cs], ref["dV"], "bf16", f"dV head {hd}")
