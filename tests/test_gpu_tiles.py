"""GPU parity of the GEMM tile shapes that the common MLP cases do not reach,
against the float64 oracle, through the public entry points.

The 256x320 tile (eight waves as 4 x 2) serves fp32 outputs whose width
(5120 and the like) leaves 256x256 tiles part of a round idle; the four-wave
kernel's typed epilogues are also run here on ragged shapes whose last tile
column is partial, at 256x256 and at 128x128 (two workgroups per CU, for grids
too small for 256x256 tiles), as is the weight-gradient pair at 128x128.  Each case is sized so the planner picks the kernel
under test (checked through the launch records), with ragged M, N and K, and
covers one operand orientation or epilogue: the fp32 partial with a
K-contiguous A and an N-contiguous B, two K-contiguous operands, two
M/N-contiguous operands (weight gradients, B's K-rows of 40 chunks), GeLU'
with the bias-gradient column sums (two wave rows per tile), and the gated
MLP's backward epilogue.  Bar: max|err|/max|ref| <= 2e-2 (bf16 storage).
"""
from __future__ import annotations

import pytest

import synth
from oracle import ref
from oracle import swiglu as sw
from tests.gpu_util import assert_close, empty, empty_f32, need_gpu, sync, to_dev, to_f64

pytestmark = pytest.mark.gpu

import linear_layers_amd as tl  # noqa: E402


def _say(msg):
    print(msg, flush=True)


def _launched(fn):
    """Run fn with GEMM launch records on; returns the kernel symbols in launch order."""
    tl.profile_enable("gemm")
    try:
        fn()
        sync()
        recs = tl.profile_collect(ordered=True)
    finally:
        tl.profile_enable(None)
    return [sym for _, sym in recs]


def _has(syms, prefix):
    assert any(s.startswith(prefix) for s in syms), f"no {prefix}... among {syms}"


def test_row_parallel_fwd_256x320():
    """Z = X W (fp32 partial), M = 4000, N = 5096, K = 200: K-contiguous A, N-contiguous B."""
    need_gpu()
    T, K, N = 4000, 200, 5096
    _say(f"row fwd T={T} K={K} N={N}")
    Xr, Wr = synth.draw(31, 0, (T, K), 1.0, "bf16"), synth.draw(31, 1, (K, N), 0.05, "bf16")
    X, W = to_dev(Xr, "bf16"), to_dev(Wr, "bf16")
    Z = empty_f32((T, N))
    syms = _launched(lambda: tl.row_parallel_fwd(X, W, 1, Z))
    _has(syms, "gemm_bf16_kernel<256,320,1,0,0,")
    want = ref.row_parallel_fwd(synth.to_f64(Xr, "bf16"), synth.to_f64(Wr, "bf16"), 1, 0)
    assert_close(to_f64(Z), want, "bf16", "Z")


@pytest.mark.parametrize("T,K,tile", [(4000, 5096, "gemm_bf16_kernel<256,320"), (8000, 2000, "gemm_w4_kernel<256,256"),
                                       (2600, 3080, "gemm_w4_kernel<256,192")])
def test_row_parallel_bwd_dgrad_wide(T, K, tile):
    """dX = dY W^T with M = T, N = K, K = 200: both operands K-contiguous."""
    need_gpu()
    N = 200
    _say(f"row bwd T={T} K={K} N={N}")
    Xr, Wr, dYr = (synth.draw(32, 0, (T, K), 1.0, "bf16"), synth.draw(32, 1, (K, N), 0.05, "bf16"),
                   synth.draw(32, 2, (T, N), 1.0, "bf16"))
    X, W, dY = to_dev(Xr, "bf16"), to_dev(Wr, "bf16"), to_dev(dYr, "bf16")
    dX, dW = empty_f32((T, K)), empty_f32((K, N))
    syms = _launched(lambda: tl.row_parallel_bwd(X, W, dY, 1, dX, dW))
    _has(syms, f"{tile},1,1,0")
    g = ref.row_parallel_bwd(synth.to_f64(Xr, "bf16"), synth.to_f64(Wr, "bf16"), synth.to_f64(dYr, "bf16"))
    assert_close(to_f64(dX), g["dX"], "bf16", "dX")
    assert_close(to_f64(dW), g["dW"], "bf16", "dW")


def test_column_parallel_bwd_wgrad_256x320():
    """dW = X^T dY with M = 4000, N = 5096, K = T = 300 (a partial last K step): both operands
    M/N-contiguous, read through the transposing LDS reads, the B tile's rows not a multiple of 128."""
    need_gpu()
    T, K, Ns = 300, 4000, 5096
    _say(f"col bwd T={T} K={K} Ns={Ns}")
    Xr, Wr, dYr = (synth.draw(33, 0, (T, K), 1.0, "bf16"), synth.draw(33, 1, (K, Ns), 0.05, "bf16"),
                   synth.draw(33, 2, (T, Ns), 1.0, "bf16"))
    X, W, dY = to_dev(Xr, "bf16"), to_dev(Wr, "bf16"), to_dev(dYr, "bf16")
    dX, dW, db = empty_f32((T, K)), empty_f32((K, Ns)), empty_f32((Ns,))
    syms = _launched(lambda: tl.column_parallel_bwd(X, W, dY, 1, dX, dW, db_shard=db))
    _has(syms, "gemm_bf16_kernel<256,320,0,0,0,")
    g = ref.column_parallel_bwd(synth.to_f64(Xr, "bf16"), synth.to_f64(Wr, "bf16"), synth.to_f64(dYr, "bf16"),
                                with_bias=True)
    assert_close(to_f64(dW), g["dW"], "bf16", "dW")
    assert_close(to_f64(dX), g["dX"], "bf16", "dX")
    assert_close(to_f64(db), g["db"], "bf16", "db")


@pytest.mark.parametrize("F,tile", [(2000, "256,256"), (1496, "256,192")])
def test_tp_mlp_bwd_dgrad_act_ragged(F, tile):
    """The MLP backward with T = 8000, h = 200: dH = (dZ W2^T) * GeLU'(H) and the db1 column sums
    run on the four-wave kernel, at F/tp = 2000 on 256x256 tiles (the last tile column 208 wide),
    at F/tp = 1496 on 256x192 tiles (the last column 152 wide), where the forward's bias+GeLU
    product also runs on 256x192 tiles with the B tile's K-rows of 24 chunks."""
    need_gpu()
    T, h = 8000, 200
    _say(f"mlp bwd T={T} h={h} F={F}")
    wl = synth.Workload("t", 35, "bf16", T=T, h=h, F=F, tp=1, x_std=1.0, w_std=0.05, b_std=0.1, dz_std=1.0)
    raw = synth.mlp_inputs(wl)
    f = {k: synth.to_f64(v, "bf16") for k, v in raw.items()}
    X, W1, W2, b1, dZ = (to_dev(raw[k], "bf16") for k in ("X", "W1", "W2", "b1", "dZ"))
    A, H, Z = empty((T, F), "bf16"), empty((T, F), "bf16"), empty_f32((T, h))
    dX, dW1, db1, dW2 = empty_f32((T, h)), empty_f32((h, F)), empty_f32((F,)), empty_f32((F, h))

    def run():
        tl.tp_mlp_fwd(X, W1, b1, W2, 1, A, Z, H_save=H)
        tl.tp_mlp_bwd(X, W1, W2, H, A, dZ, 1, dX, dW1, dW2, db1_shard=db1)

    syms = _launched(run)
    _has(syms, f"gemm_w4_kernel<{tile},1,1,2>")
    if tile == "256,192":
        _has(syms, "gemm_w4_kernel<256,192,1,0,1>")
    o = ref.tp_mlp_fwd_shard(f["X"], f["W1"], f["b1"], f["W2"], 1, 0)
    assert_close(to_f64(A), o["A"], "bf16", "A")
    assert_close(to_f64(Z), o["Z"], "bf16", "Z")
    g = ref.tp_mlp_bwd_shard(f["X"], f["W1"], f["b1"], f["W2"], f["dZ"], 1, 0)
    for name, got in (("dX", dX), ("dW1", dW1), ("db1", db1), ("dW2", dW2)):
        assert_close(to_f64(got), g[name], "bf16", name)


@pytest.mark.parametrize("T,joined", [(700, "gemm_w4_trio_kernel<128,128>"), (4200, "gemm_w4_pair_kernel<128,128,0,0,0>")])
def test_tp_mlp_128x128_tiles_and_weight_gradient_pair(T, joined):
    """The MLP with h = 1000, F/tp = 2000: at T = 700 the four-wave kernel runs 128x128 tiles
    (bias+GeLU, GeLU' with column sums, the fp32 partials), and the two weight gradients (2000 x 1000 and 1000 x 2000,
    16 x 8 tiles each) run in one launch of 128x128 tiles: at T = 700 joined by dX = dH W1^T (48 more
    tiles, one round of two workgroups per CU), at T = 4200 (264 dX tiles, more than the round holds)
    as a pair, dX on its own; ragged M, N and K (a partial last K step of T)."""
    need_gpu()
    h, F = 1000, 2000
    _say(f"mlp 128x128 T={T} h={h} F={F}")
    wl = synth.Workload("t", 38, "bf16", T=T, h=h, F=F, tp=1, x_std=1.0, w_std=0.05, b_std=0.1, dz_std=1.0)
    raw = synth.mlp_inputs(wl)
    f = {k: synth.to_f64(v, "bf16") for k, v in raw.items()}
    X, W1, W2, b1, dZ = (to_dev(raw[k], "bf16") for k in ("X", "W1", "W2", "b1", "dZ"))
    A, H, Z = empty((T, F), "bf16"), empty((T, F), "bf16"), empty_f32((T, h))
    dX, dW1, db1, dW2 = empty_f32((T, h)), empty_f32((h, F)), empty_f32((F,)), empty_f32((F, h))

    def run():
        tl.tp_mlp_fwd(X, W1, b1, W2, 1, A, Z, H_save=H)
        tl.tp_mlp_bwd(X, W1, W2, H, A, dZ, 1, dX, dW1, dW2, db1_shard=db1)

    syms = _launched(run)
    _has(syms, joined)
    if "pair" in joined:      # the forward products are large enough for 256x192 tiles here
        _has(syms, "gemm_w4_kernel<128,128,1,1,0>")
    else:
        for k in ("gemm_w4_kernel<128,128,1,0,1>", "gemm_w4_kernel<128,128,1,0,0>", "gemm_w4_kernel<128,128,1,1,2>"):
            _has(syms, k)
    o = ref.tp_mlp_fwd_shard(f["X"], f["W1"], f["b1"], f["W2"], 1, 0)
    assert_close(to_f64(A), o["A"], "bf16", "A")
    assert_close(to_f64(H), o["H"], "bf16", "H")
    assert_close(to_f64(Z), o["Z"], "bf16", "Z")
    g = ref.tp_mlp_bwd_shard(f["X"], f["W1"], f["b1"], f["W2"], f["dZ"], 1, 0)
    for name, got in (("dX", dX), ("dW1", dW1), ("db1", db1), ("dW2", dW2)):
        assert_close(to_f64(got), g[name], "bf16", name)


def test_tp_mlp_bwd_trio_256x256_ragged():
    """The MLP backward with h = 4000, F/tp = 2000, T = 3400: the two weight gradients fill one round of
    256x256 tiles (128 + 128) and dX = dH W1^T plans 256x256 tiles too (14 x 16), so all three run in one
    launch of the 256x256 four-wave kernel, dX's tiles after the pair's; ragged M, N and K in every
    product (3400 = 13 x 256 + 72 rows, 4000 = 15 x 256 + 160, 2000 = 7 x 256 + 208; K = 3400 and 2000
    end in partial 64-deep steps)."""
    need_gpu()
    T, h, F = 3400, 4000, 2000
    _say(f"mlp 256x256 trio T={T} h={h} F={F}")
    wl = synth.Workload("t", 41, "bf16", T=T, h=h, F=F, tp=1, x_std=1.0, w_std=0.05, b_std=0.1, dz_std=1.0)
    raw = synth.mlp_inputs(wl)
    f = {k: synth.to_f64(v, "bf16") for k, v in raw.items()}
    X, W1, W2, b1, dZ = (to_dev(raw[k], "bf16") for k in ("X", "W1", "W2", "b1", "dZ"))
    A, H, Z = empty((T, F), "bf16"), empty((T, F), "bf16"), empty_f32((T, h))
    dX, dW1, db1, dW2 = empty_f32((T, h)), empty_f32((h, F)), empty_f32((F,)), empty_f32((F, h))
    tl.tp_mlp_fwd(X, W1, b1, W2, 1, A, Z, H_save=H)

    def run():
        tl.tp_mlp_bwd(X, W1, W2, H, A, dZ, 1, dX, dW1, dW2, db1_shard=db1)

    syms = _launched(run)
    _has(syms, "gemm_w4_trio_kernel<256,256>")
    assert not any("pair" in k or "1,1,0>" in k for k in syms), syms
    g = ref.tp_mlp_bwd_shard(f["X"], f["W1"], f["b1"], f["W2"], f["dZ"], 1, 0)
    for name, got in (("dX", dX), ("dW1", dW1), ("db1", db1), ("dW2", dW2)):
        assert_close(to_f64(got), g[name], "bf16", name)


def test_tp_mlp_bwd_wgrad_pair_several_rounds_ragged():
    """The MLP backward with T = 200, h = 12200, F/tp = 6104: each weight gradient is 24 x 48 tiles of
    256x256 (1152, five rounds of the 256 CUs with the last half full), so the two run in one launch of
    the four-wave pair kernel (nine rounds), the second's tiles after the first's; ragged M and N in
    both (12200 = 47 x 256 + 168, 6104 = 23 x 256 + 216) and K = 200 ending in a partial 64-deep
    step.  dX then runs on its own launch."""
    need_gpu()
    T, h, F = 200, 12200, 6104
    _say(f"mlp wgrad pair over several rounds T={T} h={h} F={F}")
    wl = synth.Workload("t", 43, "bf16", T=T, h=h, F=F, tp=1, x_std=1.0, w_std=0.05, b_std=0.1, dz_std=1.0)
    raw = synth.mlp_inputs(wl)
    f = {k: synth.to_f64(v, "bf16") for k, v in raw.items()}
    X, W1, W2, b1, dZ = (to_dev(raw[k], "bf16") for k in ("X", "W1", "W2", "b1", "dZ"))
    A, H, Z = empty((T, F), "bf16"), empty((T, F), "bf16"), empty_f32((T, h))
    dX, dW1, db1, dW2 = empty_f32((T, h)), empty_f32((h, F)), empty_f32((F,)), empty_f32((F, h))
    tl.tp_mlp_fwd(X, W1, b1, W2, 1, A, Z, H_save=H)

    def run():
        tl.tp_mlp_bwd(X, W1, W2, H, A, dZ, 1, dX, dW1, dW2, db1_shard=db1)

    syms = _launched(run)
    _has(syms, "gemm_w4_pair_kernel<256,256,0,0,0>")
    assert not any("trio" in k or "256,256,0,0,0>" in k and "pair" not in k for k in syms), syms
    g = ref.tp_mlp_bwd_shard(f["X"], f["W1"], f["b1"], f["W2"], f["dZ"], 1, 0)
    for name, got in (("dX", dX), ("dW1", dW1), ("db1", db1), ("dW2", dW2)):
        assert_close(to_f64(got), g[name], "bf16", name)


@pytest.mark.parametrize("T,h,F,tile,dact", [
    (8000, 136, 2000, "256,256", "gemm_w4_duo_kernel<256,256,0,0,0,1,1,4>"),
    (8000, 136, 1720, "256,256", "gemm_w4_kernel<256,256,1,1,4>"),
    (8000, 136, 1496, "256,192", "gemm_w4_kernel<256,192,1,1,4>"),
    (1000, 136, 296, "128,128", "gemm_w4_kernel<128,128,1,1,4>")])
def test_swiglu_bwd_ragged(T, h, F, tile, dact):
    """The gated MLP with h = 136: dA = dZ W_down^T with its gate/up epilogue runs on the four-wave
    kernel at 256x256 (T = 8000, F/tp = 2000 and 1720; the last tile column 208 and 184 wide), at
    256x192 (F/tp = 1496, with the forward's joined gate/up product: the last columns 152 and 112
    wide) and at 128x128 (T = 1000, F/tp = 296; the last columns 40 and 80 wide).  At F/tp = 2000 the
    weight gradient A^T dZ (8 tiles of 256x256 over K = 8000) leaves the chip nearly idle, and dA
    runs in the same launch, after it; at 1720 its 7 tiles are not a multiple of 8, and dA runs
    alone."""
    need_gpu()
    _say(f"swiglu T={T} h={h} F={F}")
    wl = synth.Workload("t", 36, "bf16", T=T, h=h, F=F, tp=1, x_std=1.0, w_std=0.05, dz_std=1.0, kind="swiglu")
    raw = synth.swiglu_inputs(wl)
    f = {k: synth.to_f64(v, "bf16") for k, v in raw.items()}
    X, Wg, Wu, Wd, dZ = (to_dev(raw[k], "bf16") for k in ("X", "W_gate", "W_up", "W_down", "dZ"))
    W_gu = empty((h, 2 * F), "bf16")
    tl.swiglu_pack_shard(Wg, Wu, 1, 0, W_gu)
    GU, A, Z = empty((T, 2 * F), "bf16"), empty((T, F), "bf16"), empty_f32((T, h))
    dX, dW_gu, dW_down = empty_f32((T, h)), empty_f32((h, 2 * F)), empty_f32((F, h))

    def run():
        tl.tp_swiglu_fwd(X, W_gu, Wd, 1, A, Z, GU_save=GU)
        tl.tp_swiglu_bwd(X, W_gu, Wd, GU, A, dZ, 1, dX, dW_gu, dW_down)

    syms = _launched(run)
    _has(syms, dact)
    if tile != "256,256":
        _has(syms, f"gemm_w4_kernel<{tile},1,0,3>")
    o = sw.tp_swiglu_fwd_shard(f["X"], f["W_gate"], f["W_up"], f["W_down"], 1, 0)
    assert_close(to_f64(GU), o["GU"], "bf16", "GU")
    assert_close(to_f64(A), o["A"], "bf16", "A")
    assert_close(to_f64(Z), o["Z"], "bf16", "Z")
    b = sw.tp_swiglu_bwd_shard(f["X"], f["W_gate"], f["W_up"], f["W_down"], f["dZ"], 1, 0)
    assert_close(to_f64(dX), b["dX"], "bf16", "dX")
    assert_close(to_f64(dW_gu), b["dW_gu"], "bf16", "dW_gu")
    assert_close(to_f64(dW_down), b["dW_down"], "bf16", "dW_down")


@pytest.mark.parametrize("T", [2048, 2100])
def test_tp_mlp_bwd_split_k_weight_gradients(T):
    """h = 512, F/tp = 1024: the weight gradients (1024 x 512 and 512 x 1024) fill a sixteenth of the
    chip, so each runs as two K slices of T/2 (a partial last K step at T = 2100), summed in order."""
    need_gpu()
    h, F = 512, 1024
    _say(f"mlp bwd split-K T={T} h={h} F={F}")
    wl = synth.Workload("t", 37, "bf16", T=T, h=h, F=F, tp=1, x_std=1.0, w_std=0.05, b_std=0.1, dz_std=1.0)
    raw = synth.mlp_inputs(wl)
    f = {k: synth.to_f64(v, "bf16") for k, v in raw.items()}
    X, W1, W2, b1, dZ = (to_dev(raw[k], "bf16") for k in ("X", "W1", "W2", "b1", "dZ"))
    A, H, Z = empty((T, F), "bf16"), empty((T, F), "bf16"), empty_f32((T, h))
    dX, dW1, db1, dW2 = empty_f32((T, h)), empty_f32((h, F)), empty_f32((F,)), empty_f32((F, h))
    tl.tp_mlp_fwd(X, W1, b1, W2, 1, A, Z, H_save=H)
    tl.profile_enable("")
    try:
        tl.tp_mlp_bwd(X, W1, W2, H, A, dZ, 1, dX, dW1, dW2, db1_shard=db1)
        sync()
        roles = [r for r, _ in tl.profile_collect(ordered=True)]
    finally:
        tl.profile_enable(None)
    assert roles.count("wgrad_split_sum") == 2, roles
    g = ref.tp_mlp_bwd_shard(f["X"], f["W1"], f["b1"], f["W2"], f["dZ"], 1, 0)
    for name, got in (("dX", dX), ("dW1", dW1), ("db1", db1), ("dW2", dW2)):
        assert_close(to_f64(got), g[name], "bf16", name)
