"""The Python binding checks every tensor argument before calling the library.

The C ABI sees pointers and sizes only, so a short buffer, a bf16 tensor
where fp32 is written, or a host tensor would be read or written past its
end on the device.  Every wrapper therefore checks exact shapes, dtypes and
that all tensors are on one CUDA (HIP) device, raising ValueError (shape,
device) or TypeError (dtype, non-tensor) before any library call.  These
tests run on the CPU: the library handle is replaced by one that fails the
test if it is ever touched, and the tensors are host tensors (which pass the
shape and dtype checks and must then be refused as not on a device).
"""
from __future__ import annotations

import pytest
import torch

import linear_layers_amd as tl

bf, f32, u8 = torch.bfloat16, torch.float32, torch.uint8


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def boom():
        raise AssertionError("the library was called before the arguments were checked")
    monkeypatch.setattr(tl, "_get_lib", boom)
    monkeypatch.setattr(tl, "_stream", lambda *a, **k: boom())


def z(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


T, h, F, tp = 8, 16, 64, 2
Fs = F // tp


def mlp_fwd_args(**over):
    a = dict(X=z(T, h), W1_shard=z(h, Fs), b1_shard=z(Fs), W2_shard=z(Fs, h), tp_size=tp, A_save=z(T, Fs),
             Z_partial=z(T, h, dtype=f32), H_save=z(T, Fs))
    a.update(over)
    return a


def mlp_bwd_args(**over):
    a = dict(X=z(T, h), W1_shard=z(h, Fs), W2_shard=z(Fs, h), H_save=z(T, Fs), A_save=z(T, Fs), dZ=z(T, h), tp_size=tp,
             dX_partial=z(T, h, dtype=f32), dW1_shard=z(h, Fs, dtype=f32), dW2_shard=z(Fs, h, dtype=f32),
             db1_shard=z(Fs, dtype=f32))
    a.update(over)
    return a


def test_host_tensors_are_refused_in_every_wrapper():
    w = 128
    calls = [
        lambda: tl.column_parallel_fwd(z(T, h), z(h, Fs), tp, z(T, Fs), bias_shard=z(Fs), H_save=z(T, Fs)),
        lambda: tl.row_parallel_fwd(z(T, Fs), z(Fs, h), tp, z(T, h, dtype=f32)),
        lambda: tl.shard_partial_sum(z(tp, T, h, dtype=f32), z(T, h, dtype=f32)),
        lambda: tl.tp_mlp_fwd(**mlp_fwd_args()),
        lambda: tl.tp_mlp_bwd(**mlp_bwd_args()),
        lambda: tl.tp_mlp_bwd_noalloc(**mlp_bwd_args()),
        lambda: tl.column_parallel_bwd(z(T, h), z(h, Fs), z(T, Fs), tp, z(T, h, dtype=f32), z(h, Fs, dtype=f32),
                                       db_shard=z(Fs, dtype=f32)),
        lambda: tl.row_parallel_bwd(z(T, Fs), z(Fs, h), z(T, h), tp, z(T, Fs, dtype=f32), z(Fs, h, dtype=f32)),
        lambda: tl.swiglu_pack_shard(z(h, F), z(h, F), tp, 0, z(h, 2 * Fs)),
        lambda: tl.swiglu_unpack_grad(z(h, 2 * Fs, dtype=f32), tp, 0, z(h, F, dtype=f32), z(h, F, dtype=f32)),
        lambda: tl.tp_swiglu_fwd(z(T, h), z(h, 2 * Fs), z(Fs, h), tp, z(T, Fs), z(T, h, dtype=f32)),
        lambda: tl.tp_swiglu_bwd(z(T, h), z(h, 2 * Fs), z(Fs, h), z(T, 2 * Fs), z(T, Fs), z(T, h), tp,
                                 z(T, h, dtype=f32), z(h, 2 * Fs, dtype=f32), z(Fs, h, dtype=f32)),
        lambda: tl.layernorm_fwd(z(T, h), z(h, dtype=f32), z(h, dtype=f32), z(T, h), z(T, dtype=f32), z(T, dtype=f32)),
        lambda: tl.layernorm_bwd(z(T, h), z(h, dtype=f32), z(T, dtype=f32), z(T, dtype=f32), z(T, h, dtype=f32),
                                 z(T, h, dtype=f32)),
        lambda: tl.sp_partial_sum_dropout_residual(z(tp, T, h, dtype=f32), z(T, h), z(T, h), 0.1, 1, 0),
        lambda: tl.sp_dropout_bwd(z(T, h), z(T, h), 0.1, 1, 0),
        lambda: tl.attn_fwd(z(T, w), z(T, w), z(T, w), z(T, w), 1, T, 1, lse=z(1, T, dtype=f32)),
        lambda: tl.attn_bwd(z(T, w), z(T, w), z(T, w), z(T, w), z(T, w), z(1, T, dtype=f32), z(T, w), z(T, w),
                            z(T, w), 1, T, 1),
        lambda: tl.tp_attn_fwd(z(T, h), z(h, 3 * w), z(w, h), z(T, 3 * w), z(T, w), z(1, T, dtype=f32),
                               z(T, h, dtype=f32), 1, T, 2, 2),
        lambda: tl.tp_attn_bwd(z(T, h), z(h, 3 * w), z(w, h), z(T, 3 * w), z(T, w), z(1, T, dtype=f32), z(T, h),
                               z(T, h, dtype=f32), z(h, 3 * w, dtype=f32), z(w, h, dtype=f32), 1, T, 2, 2),
    ]
    for i, call in enumerate(calls):
        with pytest.raises(ValueError, match="device"):
            call()


def test_wrong_output_dtype_is_a_type_error():
    # a bf16 Z_partial would receive T*h*4 bytes into T*h*2
    with pytest.raises(TypeError, match="Z_partial"):
        tl.tp_mlp_fwd(**mlp_fwd_args(Z_partial=z(T, h, dtype=bf)))
    with pytest.raises(TypeError, match="dX_partial"):
        tl.tp_mlp_bwd(**mlp_bwd_args(dX_partial=z(T, h, dtype=bf)))
    # typed outputs must share the inputs' storage dtype
    with pytest.raises(TypeError, match="A_save"):
        tl.tp_mlp_fwd(**mlp_fwd_args(A_save=z(T, Fs, dtype=f32)))
    with pytest.raises(TypeError, match="unsupported dtype"):
        tl.tp_mlp_fwd(**mlp_fwd_args(X=z(T, h, dtype=torch.float16)))


@pytest.mark.parametrize("name,bad", [
    ("W1_shard", z(h + 1, Fs)),       # one row short of h... or one too many
    ("W2_shard", z(Fs, h - 8)),
    ("b1_shard", z(Fs - 8)),
    ("A_save", z(T - 1, Fs)),
    ("H_save", z(T, Fs + 8)),
    ("Z_partial", z(T, h + 4, dtype=f32)),
])
def test_wrong_shapes_are_value_errors_forward(name, bad):
    with pytest.raises(ValueError, match=name):
        tl.tp_mlp_fwd(**mlp_fwd_args(**{name: bad}))


@pytest.mark.parametrize("name,bad", [
    ("W2_shard", z(h, Fs)),           # transposed
    ("H_save", z(T, 2 * Fs)),
    ("dZ", z(T + 1, h)),
    ("dW1_shard", z(Fs, h, dtype=f32)),
    ("dW2_shard", z(h, Fs, dtype=f32)),
    ("db1_shard", z(F, dtype=f32)),
])
def test_wrong_shapes_are_value_errors_backward(name, bad):
    with pytest.raises(ValueError, match=name):
        tl.tp_mlp_bwd(**mlp_bwd_args(**{name: bad}))
    with pytest.raises(ValueError, match=name):
        tl.tp_mlp_bwd_noalloc(**mlp_bwd_args(**{name: bad}))


def test_other_checks():
    with pytest.raises(TypeError, match="must be a torch.Tensor"):
        tl.row_parallel_fwd([[1.0]], z(Fs, h), tp, z(T, h, dtype=f32))
    with pytest.raises(ValueError, match="tp_size"):
        tl.shard_partial_sum(z(2, T, h, dtype=f32), z(T, h, dtype=f32), tp_size=3)
    with pytest.raises(ValueError, match="workspace"):
        tl.tp_mlp_bwd(**mlp_bwd_args(), workspace=z(4, 4, dtype=u8))
    with pytest.raises(TypeError, match="workspace"):
        tl.tp_mlp_bwd(**mlp_bwd_args(), workspace=z(16, dtype=f32))
    with pytest.raises(ValueError, match="lse"):
        tl.attn_fwd(z(T, 128), z(T, 128), z(T, 128), z(T, 128), 1, T, 1, lse=z(2, T, dtype=f32))
    with pytest.raises(ValueError, match="divisible"):
        tl.tp_attn_fwd(z(T, h), z(h, 384), z(128, h), z(T, 384), z(T, 128), z(1, T, dtype=f32),
                       z(T, h, dtype=f32), 1, T, 3, 2)
