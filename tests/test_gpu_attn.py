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


def _lse_close(got, want, what, tol=1e-4):
    err = np.abs(np.asarray(got) - want) / np.maximum(1.0, np.abs(want))
    assert np.all(np.isfinite(got)) and err.max() <= tol, f"{what}: lse error {err.max():.3e}"


def _qkv(seed, T, heads, std=1.0):
    """A fused [T, 3*heads*128] QKV tensor (bf16 bits) as the column projection writes it."""
    r = np.random.default_rng(seed)
    return synth.bf16_round_bits((r.standard_normal((T, 3 * heads * D)) * std).astype(np.float32))


@pytest.mark.parametrize("batch,seq,heads,causal", [(1, 1, 1, True), (2, 77, 3, True), (2, 77, 3, False),
                                                    (1, 300, 2, True), (1, 300, 2, False), (3, 128, 1, True),
                                                    (1, 1000, 2, True),
                                                    # causal query blocks past row 1664 split their keys into
                                                    # chunks of 1664, merged by log-sum-exp (2 and 3 chunks,
                                                    # ragged last block)
                                                    (2, 1100, 1, True), (1, 2100, 2, True), (1, 2100, 1, False),
                                                    (1, 4200, 1, True)])
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


def test_attn_fwd_split_workspace():
    """Causal, 2100 tokens (two key chunks for the last query block): the chunked forward is bitwise
    repeatable; a workspace below attn_fwd_workspace_bytes is refused before anything is written."""
    need_gpu()
    batch, seq, heads = 1, 2100, 2
    T, w = batch * seq, heads * D
    dev = to_dev(_qkv(21, T, heads), "bf16")
    Q, K, V = dev[:, :w], dev[:, w:2 * w], dev[:, 2 * w:]
    outs = []
    for _ in range(2):
        O, lse = empty((T, w), "bf16"), empty_f32((heads, T))
        tl.attn_fwd(Q, K, V, O, batch, seq, heads, causal=True, lse=lse)
        sync()
        outs.append((O, lse))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    need = tl.attn_fwd_workspace_bytes(batch, seq, heads)
    assert need > 0
    O = empty((T, w), "bf16")
    small = torch.zeros(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(tl.TpmlpError) as e:
        tl.attn_fwd(Q, K, V, O, batch, seq, heads, causal=True, workspace=small)
    assert e.value.status == 7
    sync()
    assert torch.isnan(O).all(), "O was written by a refused call"


@pytest.mark.slow
@pytest.mark.parametrize("batch,seq,heads,chunk", [(2, 8400, 2, 1664), (1, 16500, 1, 2176)])
def test_attn_fwd_long_sequence_sampled(batch, seq, heads, chunk):
    """Long causal sequences (ragged): 8400 tokens take 6 key chunks of 1664; past 13312 tokens the chunks
    grow (34 key blocks of 64 at 16500, 8 chunks for the last query block).  Sampled rows of O and lse of
    every (sequence, head) against the oracle, on both sides of the chunk edges."""
    need_gpu()
    _say(f"attn fwd long batch={batch} seq={seq} heads={heads}")
    T, w = batch * seq, heads * D
    qkv = _qkv(8401, T, heads)
    dev = to_dev(qkv, "bf16")
    O, lse = empty((T, w), "bf16"), empty_f32((heads, T))
    tl.attn_fwd(dev[:, :w], dev[:, w:2 * w], dev[:, 2 * w:], O, batch, seq, heads, causal=True, lse=lse)
    sync()
    f = synth.to_f64(qkv, "bf16")
    Og, Lg = to_f64(O), to_f64(lse)
    edges = [e for c in range(1, 8) for e in (c * chunk - 1, c * chunk) if c * chunk < seq]
    rows = np.array(sorted({0, 1, seq // 2, seq - 129, seq - 128, seq - 2, seq - 1, *edges}))
    for b in range(batch):
        for hd in range(heads):
            ref = oat.attn_fwd_rows(f[:, :w], f[:, w:2 * w], f[:, 2 * w:], batch, seq, heads, D, True, D ** -0.5,
                                    b, hd, rows)
            r = b * seq + rows
            assert_close(Og[r, hd * D:(hd + 1) * D], ref["O"], "bf16", f"O seq {b} head {hd}")
            _lse_close(Lg[hd, r], ref["lse"], f"lse seq {b} head {hd}")


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
                                                    (1, 1000, 2, True), (1, 1000, 1, False),
                                                    # causal query blocks past row 1664 split their keys into
                                                    # chunks of 1664 (2 and 3 chunks here, ragged last block)
                                                    (2, 1100, 1, True), (1, 2100, 2, True), (1, 4200, 1, True)])
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
    for seq in (200, 2100):   # one key chunk; two (partials summed in order)
        a = _bwd_case(1, seq, 2, True, seed=9)[2]
        b = _bwd_case(1, seq, 2, True, seed=9)[2]
        assert torch.equal(a, b)
    assert tl.attn_bwd_workspace_bytes(2, 100, 3) >= 2 * 2 * 100 * 3 * 4
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


@pytest.mark.slow
def test_attn_bwd_long_sequence_sampled():
    """8400 tokens (ragged), 2 sequences, 2 heads, causal: 6 dQ key chunks of 1664 for the last query
    block.  Sampled rows of dQ, dK, dV of two (sequence, head) pairs against the oracle, rows on both sides
    of the chunk edges."""
    need_gpu()
    batch, seq, heads = 2, 8400, 2
    _say(f"attn bwd long batch={batch} seq={seq} heads={heads}")
    qkv, dO, dqkv = _bwd_case(batch, seq, heads, True, seed=8400)
    w = heads * D
    f, fd, g = synth.to_f64(qkv, "bf16"), synth.to_f64(dO, "bf16"), to_f64(dqkv)
    rows = np.array([0, 1, 127, 1663, 1664, 1665, 3327, 3328, 4991, 4992, 6655, 6656, 8191, 8192, 8270, 8271,
                     8399])
    for b, hd in ((0, 0), (1, 1)):
        ref = oat.attn_bwd_rows(f[:, :w], f[:, w:2 * w], f[:, 2 * w:], fd, batch, seq, heads, D, True, D ** -0.5,
                                b, hd, rows)
        r = b * seq + rows
        cs = slice(hd * D, (hd + 1) * D)
        assert_close(g[r][:, :w][:, cs], ref["dQ"], "bf16", f"dQ seq {b} head {hd}")
        assert_close(g[r][:, w:2 * w][:, cs], ref["dK"], "bf16", f"dK seq {b} head {hd}")
        assert_close(g[r][:, 2 * w:][:, cs], ref["dV"], "bf16", f"dV seq {b} head {hd}")


# ----------------------------------------------------------------------------
# The head-sharded attention block: QKV projection, attention over the shard's
# heads, O-projection partial, and its backward, through tp_attn_fwd/bwd.

def _block_run(raw, batch, seq, heads, tp, i, causal):
    """Shard i of the block on the GPU; returns every output as a device tensor."""
    T, h = raw["X"].shape
    w = heads // tp * D
    c = slice(i * w, (i + 1) * w)
    Wqkv = np.ascontiguousarray(np.concatenate([raw[n][:, c] for n in ("Wq", "Wk", "Wv")], axis=1))
    X, Wq, Wo, dZ = (to_dev(a, "bf16") for a in (raw["X"], Wqkv, np.ascontiguousarray(raw["Wo"][c]), raw["dZ"]))
    out = {"QKV": empty((T, 3 * w), "bf16"), "O": empty((T, w), "bf16"), "lse": empty_f32((heads // tp, T)),
           "Z": empty_f32((T, h)), "dX": empty_f32((T, h)), "dWqkv": empty_f32((h, 3 * w)),
           "dWo": empty_f32((w, h))}
    tl.tp_attn_fwd(X, Wq, Wo, out["QKV"], out["O"], out["lse"], out["Z"], batch, seq, heads, tp, causal=causal)
    tl.tp_attn_bwd(X, Wq, Wo, out["QKV"], out["O"], out["lse"], dZ, out["dX"], out["dWqkv"], out["dWo"], batch, seq,
                   heads, tp, causal=causal)
    sync()
    return out


@pytest.mark.parametrize("batch,seq,heads,tp,shard,causal", [(2, 77, 4, 2, 1, True), (1, 200, 2, 1, 0, False),
                                                             (3, 64, 4, 4, 3, True)])
def test_attn_block_small(batch, seq, heads, tp, shard, causal):
    need_gpu()
    _say(f"attn block batch={batch} seq={seq} heads={heads} tp={tp} shard={shard} causal={causal}")
    T, h = batch * seq, heads * D
    r = np.random.default_rng(seq + 7 * heads)
    raw = {"X": synth.bf16_round_bits(r.standard_normal((T, h)).astype(np.float32)),
           "dZ": synth.bf16_round_bits(r.standard_normal((T, h)).astype(np.float32))}
    for n in ("Wq", "Wk", "Wv", "Wo"):
        raw[n] = synth.bf16_round_bits((r.standard_normal((h, h)) / np.sqrt(h)).astype(np.float32))
    g = _block_run(raw, batch, seq, heads, tp, shard, causal)
    f = {k: synth.to_f64(v, "bf16") for k, v in raw.items()}
    ref = oat.tp_attn_block_bwd_shard(f["X"], f["Wq"], f["Wk"], f["Wv"], f["Wo"], f["dZ"], batch, seq, heads, D, tp,
                                      shard, causal, D ** -0.5)
    for k in ("QKV", "O", "Z", "dX", "dWqkv", "dWo"):
        assert_close(to_f64(g[k]), ref[k], "bf16", k)
    _block_lse_close(to_f64(g["lse"]), ref["QKV"], ref["lse"], batch, seq, heads // tp, causal)


def _block_lse_close(got, QKV, want, batch, seq, hs, causal):
    """The block's attention reads the bf16-rounded QKV its projection wrote, so
    each score q.k * scale may move by up to 2^-7 * scale * sum_d |q_d| |k_d|
    (two roundings of unit 2^-8), and the log-sum-exp, a softmax-weighted
    mean of those moves, by no more than their maximum over the row's keys;
    fp32 arithmetic adds the 1e-4 * max(1, |lse|) of the core's own bar."""
    w = hs * D
    for b in range(batch):
        rs = slice(b * seq, (b + 1) * seq)
        for hd in range(hs):
            cs = slice(hd * D, (hd + 1) * D)
            aq, ak = np.abs(QKV[rs, cs]), np.abs(QKV[rs, w:2 * w][:, cs])
            m = aq @ ak.T
            if causal:
                m = np.where(np.tril(np.ones((seq, seq), dtype=bool)), m, 0.0)
            bound = 2.0 ** -7 * D ** -0.5 * m.max(axis=1) + 1e-4 * np.maximum(1.0, np.abs(want[hd, rs]))
            err = np.abs(got[hd, rs] - want[hd, rs])
            assert np.all(np.isfinite(got[hd, rs])) and np.all(err <= bound), \
                f"lse b={b} head={hd}: worst err/bound {np.max(err / bound):.3f}"


@pytest.mark.slow
def test_attn_block_workload_sampled():
    """T=4096 (one causal sequence), h=5120, 40 heads of 128, tp=4, shard 0, the workload's own inputs:
    sampled rows of every output, sampled columns of the weight gradients."""
    need_gpu()
    wl = synth.WORKLOADS["attn_proj_bf16"]
    _say(f"attn block workload {wl.name}")
    raw = synth.proj_inputs(wl, which=("X", "Wq", "Wk", "Wv", "Wo", "dOut"))
    raw["dZ"] = raw.pop("dOut")
    T, heads, tp = wl.T, wl.heads, wl.tp
    hs, w = heads // tp, heads // tp * D
    g = _block_run(raw, 1, T, heads, tp, 0, True)
    f = {k: synth.to_f64(v, "bf16") for k, v in raw.items()}
    rows = np.array(sorted(set(np.random.default_rng(11).choice(T, 20, replace=False).tolist()) | {0, 127, T - 1}))
    Wqkv = oat.qkv_shard_weight(f["Wq"], f["Wk"], f["Wv"], heads, D, tp, 0)
    Wo = f["Wo"][:w]
    QKV = f["X"] @ Wqkv
    assert_close(to_f64(g["QKV"][torch.as_tensor(rows, device="cuda")]), QKV[rows], "bf16", "QKV rows")
    Q, K, V = QKV[:, :w], QKV[:, w:2 * w], QKV[:, 2 * w:]
    dO = f["dZ"] @ Wo.T
    O_rows = np.zeros((len(rows), w))
    dQKV_rows = np.zeros((len(rows), 3 * w))
    for hd in range(hs):
        cs = slice(hd * D, (hd + 1) * D)
        fr = oat.attn_fwd_rows(Q, K, V, 1, T, hs, D, True, D ** -0.5, 0, hd, rows)
        O_rows[:, cs] = fr["O"]
        _lse_close(to_f64(g["lse"])[hd, rows], fr["lse"], f"lse head {hd}")
        br = oat.attn_bwd_rows(Q, K, V, dO, 1, T, hs, D, True, D ** -0.5, 0, hd, rows)
        for k, name in enumerate(("dQ", "dK", "dV")):
            dQKV_rows[:, k * w + hd * D:k * w + (hd + 1) * D] = br[name]
    sel = torch.as_tensor(rows, device="cuda")
    assert_close(to_f64(g["O"][sel]), O_rows, "bf16", "O rows")
    assert_close(to_f64(g["Z"][sel]), O_rows @ Wo, "bf16", "Z rows")
    assert_close(to_f64(g["dX"][sel]), dQKV_rows @ Wqkv.T, "bf16", "dX rows")
    # weight-gradient columns: dWo needs all of O, dWqkv the whole dQ/dK/dV of head 3
    cols = np.random.default_rng(12).choice(wl.h, 24, replace=False)
    O_full = np.concatenate([oat.attn_fwd(Q[:, hd * D:(hd + 1) * D], K[:, hd * D:(hd + 1) * D],
                                          V[:, hd * D:(hd + 1) * D], 1, T, 1, D, True, D ** -0.5)["O"]
                             for hd in range(hs)], axis=1)
    assert_close(to_f64(g["dWo"][:, torch.as_tensor(cols, device="cuda")]), O_full.T @ f["dZ"][:, cols], "bf16",
                 "dWo cols")
    cs = slice(3 * D, 4 * D)
    b3 = oat.attn_bwd(Q[:, cs], K[:, cs], V[:, cs], dO[:, cs], 1, T, 1, D, True, D ** -0.5)
    for k, name in enumerate(("dQ", "dK", "dV")):
        qc = k * w + 3 * D + np.array([0, 17, 64, 127])
        assert_close(to_f64(g["dWqkv"][:, torch.as_tensor(qc, device="cuda")]),
                     f["X"].T @ b3[name][:, [0, 17, 64, 127]], "bf16", f"dWqkv {name} cols of head 3")
