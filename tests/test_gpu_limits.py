"""Operands at the largest leading dimension the library accepts: 2^22 - 8
elements, the largest multiple of 8 below the 2^22 it refuses.  Inside one
256-row tile the byte offsets that the buffer descriptors carry then reach
(255 * (2^22 - 8) + K) * 2, about 2.1 GB, near the top of their 32-bit range
(each tile's own base address is formed in 64 bits).  The inputs are narrow
views of tensors that wide; the results are held to the oracle at the bf16
bar."""
import numpy as np
import pytest
import torch

import synth
from oracle import ref
from tests.gpu_util import assert_close, empty, empty_f32, need_gpu, sync, to_dev, to_f64

pytestmark = pytest.mark.gpu

import linear_layers_amd as tl  # noqa: E402

LD = (1 << 22) - 8


def _wide(a: np.ndarray, dtype: str) -> torch.Tensor:
    """A [rows, cols] view, row stride LD, of a device tensor holding a's values in its first cols columns."""
    rows, cols = a.shape
    base = torch.empty((rows, LD), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda")
    v = base[:, :cols]
    v.copy_(to_dev(a, dtype))
    assert v.stride(0) == LD
    return v


def test_column_parallel_layer_at_the_largest_leading_dimension():
    """Y = GeLU(X W) and its backward with X [300, 72], W [72, 48000] and dY [300, 48000] all at row
    stride 2^22 - 8: the forward runs 256x192 tiles (two tile rows, the second 44 rows), so its
    K-contiguous X tile spans 255 rows of 8 MB; W's K-rows and, in the weight gradient, X's and dY's
    rows are as far apart."""
    need_gpu()
    T, K, N = 300, 72, 48000
    print(f"largest leading dimension {LD}: T={T} K={K} N={N}", flush=True)
    Xr, Wr = synth.draw(61, 0, (T, K), 1.0, "bf16"), synth.draw(61, 1, (K, N), 0.05, "bf16")
    dYr = synth.draw(61, 2, (T, N), 1.0, "bf16")
    X, W, dY = _wide(Xr, "bf16"), _wide(Wr, "bf16"), _wide(dYr, "bf16")
    Y, H = empty((T, N), "bf16"), empty((T, N), "bf16")
    tl.profile_enable("gemm")
    try:
        tl.column_parallel_fwd(X, W, 1, Y, H_save=H)
        sync()
        syms = [sym for _, sym in tl.profile_collect(ordered=True)]
    finally:
        tl.profile_enable(None)
    assert any(s.startswith("gemm_w4_kernel<256,192,") for s in syms), syms
    dX, dW, db = empty_f32((T, K)), empty_f32((K, N)), empty_f32((N,))
    tl.column_parallel_bwd(X, W, dY, 1, dX, dW, db_shard=db)
    sync()
    fX, fW, fdY = (synth.to_f64(a, "bf16") for a in (Xr, Wr, dYr))
    Hr, Yr = ref.column_parallel_fwd(fX, fW, None, 1, 0)
    assert_close(to_f64(H), Hr, "bf16", "H")
    assert_close(to_f64(Y), Yr, "bf16", "Y")
    g = ref.column_parallel_bwd(fX, fW, fdY, with_bias=True)
    assert_close(to_f64(dX), g["dX"], "bf16", "dX")
    assert_close(to_f64(dW), g["dW"], "bf16", "dW")
    assert_close(to_f64(db), g["db"], "bf16", "db")


def test_outputs_past_two_to_the_31_elements():
    """Z = X W (fp32) and Y = GeLU(X W + b) with H saved (bf16), X [33000, 64], W [64, 65536]: the
    outputs hold 2.16e9 elements, so element indices pass 2^31 from row 32768 on, which is also where
    the last, ragged row of 256-row tiles starts (232 rows).  The first rows, rows on both sides of
    32768 and rows through the end of that tile row against the oracle, row by row."""
    need_gpu()
    T, K, N = 33000, 64, 65536
    print(f"outputs past 2^31 elements: T={T} K={K} N={N}", flush=True)
    Xr, Wr = synth.draw(62, 0, (T, K), 1.0, "bf16"), synth.draw(62, 1, (K, N), 0.05, "bf16")
    br = synth.draw(62, 2, (N,), 0.1, "bf16")
    X, W, b = to_dev(Xr, "bf16"), to_dev(Wr, "bf16"), to_dev(br, "bf16")
    rows = np.r_[0:3, 32766:32771, T - 105:T - 102, T - 3:T]
    fW, fb = synth.to_f64(Wr, "bf16"), synth.to_f64(br, "bf16")
    fX = synth.to_f64(Xr[rows], "bf16")
    Z = empty_f32((T, N))
    tl.row_parallel_fwd(X, W, 1, Z)
    sync()
    assert_close(to_f64(Z[torch.from_numpy(rows).cuda()]), ref.row_parallel_fwd_shard(fX, fW), "bf16", "Z rows")
    del Z
    Y, H = empty((T, N), "bf16"), empty((T, N), "bf16")
    tl.column_parallel_fwd(X, W, 1, Y, bias_shard=b, H_save=H)
    sync()
    Hr, Yr = ref.column_parallel_fwd(fX, fW, fb, 1, 0)
    idx = torch.from_numpy(rows).cuda()
    assert_close(to_f64(H[idx]), Hr, "bf16", "H rows")
    assert_close(to_f64(Y[idx]), Yr, "bf16", "Y rows")
