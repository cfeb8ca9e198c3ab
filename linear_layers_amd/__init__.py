"""Python binding of libtpmlp, the gfx950 tensor-parallel MLP library.

Argument marshalling only: every function turns torch tensors into device
pointers, leading dimensions and the current HIP stream, and calls the C
entry point of the same name (declared in include/tpmlp.h).  All arithmetic
runs in the library's HIP kernels; there is no fallback.  If libtpmlp.so is
not built this module refuses to import.

torch is imported before the library is loaded so that the library binds to
the HIP runtime torch already loaded (one runtime per process; its soname is
the same as the system runtime's).
"""
from __future__ import annotations

import ctypes
import json
import os
from typing import Optional

import torch

__all__ = [
    "TpmlpError", "lib", "LIB_PATH", "F32", "BF16", "ACT_NONE", "ACT_GELU_TANH",
    "column_parallel_fwd", "row_parallel_fwd", "shard_partial_sum", "tp_mlp_fwd", "tp_mlp_bwd",
    "tp_mlp_bwd_noalloc", "tpmlp_noalloc_scratch_bytes", "tpmlp_bwd_workspace_bytes", "bias_gelu_fwd", "gelu_bwd", "column_parallel_bwd", "row_parallel_bwd", "swiglu_pack_shard",
    "swiglu_unpack_grad", "tp_swiglu_fwd", "tp_swiglu_bwd", "tp_swiglu_bwd_workspace_bytes", "layernorm_fwd",
    "layernorm_bwd", "sp_partial_sum_dropout_residual", "sp_dropout_bwd", "attn_fwd", "attn_bwd",
    "attn_bwd_workspace_bytes", "attn_fwd_workspace_bytes", "tp_attn_fwd", "tp_attn_fwd_workspace_bytes",
    "tp_attn_bwd", "tp_attn_bwd_workspace_bytes", "profile_enable",
    "profile_collect", "status_string", "version",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtpmlp.so")

F32, BF16 = 0, 1
ACT_NONE, ACT_GELU_TANH = 0, 1
_ACTS = {"none": ACT_NONE, "gelu_tanh": ACT_GELU_TANH, ACT_NONE: ACT_NONE, ACT_GELU_TANH: ACT_GELU_TANH}

_vp, _i64, _int, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
_f32, _u64 = ctypes.c_float, ctypes.c_uint64

_SIGNATURES = {
    "column_parallel_fwd": [_vp, _int, _int, _i64, _i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _vp, _i64, _vp, _i64],
    "row_parallel_fwd": [_vp, _int, _i64, _i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64],
    "shard_partial_sum": [_vp, _int, _i64, _i64, _vp, _i64, _i64, _vp, _i64],
    "tp_mlp_fwd": [_vp, _int, _i64, _i64, _i64, _int, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _vp],
    "tp_mlp_bwd": [_vp, _int, _i64, _i64, _i64, _int, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                   _vp, _sz],
    "tp_mlp_bwd_noalloc": [_vp, _int, _i64, _i64, _i64, _int, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                           _vp],
    "tpmlp_noalloc_scratch_bytes": [],
    "bias_gelu_fwd": [_vp, _int, _i64, _i64, _vp, _i64, _vp, _vp, _i64, _vp, _i64],
    "gelu_bwd": [_vp, _int, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64],
    "column_parallel_bwd": [_vp, _int, _i64, _i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp,
                            _i64, _vp],
    "row_parallel_bwd": [_vp, _int, _i64, _i64, _i64, _int, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64],
    "tpmlp_bwd_workspace_bytes": [_int, _i64, _i64, _i64, _int],
    "swiglu_pack_shard": [_vp, _int, _i64, _i64, _int, _int, _vp, _i64, _vp, _i64, _vp],
    "swiglu_unpack_grad": [_vp, _i64, _i64, _int, _int, _vp, _vp, _i64, _vp, _i64],
    "tp_swiglu_fwd": [_vp, _int, _i64, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp, _vp],
    "tp_swiglu_bwd_workspace_bytes": [_int, _i64, _i64, _i64, _int],
    "tp_swiglu_bwd": [_vp, _int, _i64, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz],
    "layernorm_fwd": [_vp, _i64, _i64, _vp, _i64, _vp, _vp, _f32, _vp, _i64, _vp, _vp],
    "layernorm_bwd": [_vp, _i64, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp],
    "sp_partial_sum_dropout_residual": [_vp, _int, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _f32, _u64, _i64, _vp,
                                        _i64],
    "sp_dropout_bwd": [_vp, _i64, _i64, _vp, _i64, _f32, _u64, _i64, _vp, _i64],
    "attn_fwd": [_vp, _i64, _i64, _int, _int, _int, _f32, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _sz],
    "attn_fwd_workspace_bytes": [_i64, _i64, _int],
    "attn_bwd_workspace_bytes": [_i64, _i64, _int],
    "attn_bwd": [_vp, _i64, _i64, _int, _int, _int, _f32, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp,
                 _vp, _i64, _vp, _i64, _vp, _i64, _vp, _sz],
    "tp_attn_fwd": [_vp, _i64, _i64, _i64, _int, _int, _int, _int, _f32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz],
    "tp_attn_fwd_workspace_bytes": [_i64, _i64, _int, _int, _int],
    "tp_attn_bwd_workspace_bytes": [_i64, _i64, _int, _int, _int],
    "tp_attn_bwd": [_vp, _i64, _i64, _i64, _int, _int, _int, _int, _f32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                    _vp, _vp, _sz],
    "tpmlp_status_string": [_int],
    "tpmlp_last_error": [],
    "tpmlp_version": [],
    "tpmlp_profile_enable": [ctypes.c_char_p],
    "tpmlp_profile_collect": [ctypes.c_char_p, _sz],
}
_RESTYPES = {"tpmlp_bwd_workspace_bytes": _sz, "tpmlp_noalloc_scratch_bytes": _sz, "attn_bwd_workspace_bytes": _sz, "tp_attn_bwd_workspace_bytes": _sz,
             "attn_fwd_workspace_bytes": _sz, "tp_attn_fwd_workspace_bytes": _sz,
             "tp_swiglu_bwd_workspace_bytes": _sz, "tpmlp_status_string": ctypes.c_char_p,
             "tpmlp_last_error": ctypes.c_char_p, "tpmlp_version": ctypes.c_char_p}


class TpmlpError(RuntimeError):
    """A non-OK status from libtpmlp."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status
        self.message = message


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m linear_layers_amd.build`")
    handle = ctypes.CDLL(LIB_PATH)
    for name, args in _SIGNATURES.items():
        fn = getattr(handle, name)
        fn.argtypes = args
        fn.restype = _RESTYPES.get(name, ctypes.c_int)
    return handle


_lib = None


def __getattr__(name):
    # The library is loaded on first use, so the package (and its build
    # module) import without it; any call then fails loudly if it is absent.
    if name == "lib":
        return _get_lib()
    raise AttributeError(name)


def _get_lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = _load()
    return _lib


def status_string(status: int) -> str:
    return _get_lib().tpmlp_status_string(status).decode()


def version() -> str:
    return _get_lib().tpmlp_version().decode()


def _check(status: int) -> None:
    if status != 0:
        raise TpmlpError(status, f"{status_string(status)}: {_get_lib().tpmlp_last_error().decode()}")


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}; libtpmlp takes bfloat16 or float32")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else (t.data_ptr() or None)


def _ld(t: Optional[torch.Tensor], width: int) -> int:
    """Leading dimension of a row-major 2-D tensor (or view)."""
    if t is None:
        return width
    if t.dim() != 2:
        raise ValueError(f"expected a 2-D tensor, got shape {tuple(t.shape)}")
    if t.shape[0] > 1 and t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("rows must be contiguous (stride(1) == 1)")
    return t.stride(0) if t.shape[0] > 1 else width


def _stream(stream, like: torch.Tensor):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    return torch.cuda.current_stream(like.device).cuda_stream


def _require_contiguous(name: str, t: Optional[torch.Tensor]) -> None:
    if t is not None and t.numel() > 0 and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_STORAGE = (torch.bfloat16, torch.float32)
_F32T, _BF16T, _U8T = torch.float32, torch.bfloat16, torch.uint8


def _dims(name: str, t, n: int) -> tuple:
    """Shape of a tensor argument that must have n dimensions."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dim() != n:
        raise ValueError(f"{name} must be {n}-D, got shape {tuple(t.shape)}")
    return tuple(t.shape)


def _args(*specs) -> None:
    """Check tensor arguments before any library call (the library cannot see
    buffer sizes, so a short or mistyped buffer would be read or written past
    its end on the device).

    Each spec is (name, tensor, shape, dtypes, optional): the exact shape, the
    allowed dtype(s), and whether None is allowed.  A non-tensor or a wrong
    dtype raises TypeError; a wrong shape, a tensor not on a CUDA (HIP)
    device, or tensors on different devices raise ValueError.  Shapes and
    dtypes are checked for every argument before devices.
    """
    present = []
    for name, t, shape, dtypes, optional in specs:
        if t is None:
            if optional:
                continue
            raise ValueError(f"{name} is required")
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
        if tuple(t.shape) != tuple(int(x) for x in shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(int(x) for x in shape)}")
        dts = dtypes if isinstance(dtypes, tuple) else (dtypes,)
        if t.dtype not in dts:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {' or '.join(str(d) for d in dts)}")
        present.append((name, t))
    dev = None
    for name, t in present:
        if not t.is_cuda:
            raise ValueError(f"{name} is on {t.device}; libtpmlp takes device tensors")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {dev}")


def _storage(name: str, t) -> torch.dtype:
    """The storage dtype of the call, taken from its first input."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype not in _STORAGE:
        raise TypeError(f"unsupported dtype {t.dtype}; libtpmlp takes bfloat16 or float32")
    return t.dtype


def _ws(name: str, t) -> tuple:
    """Spec of a workspace argument: a 1-D uint8 device buffer of any length."""
    return (name, t, (t.numel(),) if isinstance(t, torch.Tensor) else (0,), _U8T, False)


def column_parallel_fwd(X, W_shard, tp_size: int, Y_shard, bias_shard=None, H_save=None,
                        act="gelu_tanh", stream=None) -> None:
    """Y_shard = Act(X @ W_shard + bias_shard); optionally H_save = X @ W_shard + bias_shard."""
    T, K = _dims("X", X, 2)
    Ns = _dims("W_shard", W_shard, 2)[1]
    dt = _storage("X", X)
    _args(("X", X, (T, K), dt, False), ("W_shard", W_shard, (K, Ns), dt, False), ("Y_shard", Y_shard, (T, Ns), dt, False),
          ("bias_shard", bias_shard, (Ns,), dt, True), ("H_save", H_save, (T, Ns), dt, True))
    _check(_get_lib().column_parallel_fwd(_stream(stream, X), _dtype(X), _ACTS[act], T, K, Ns * tp_size, tp_size,
                                   _ptr(X), _ld(X, K), _ptr(W_shard), _ld(W_shard, Ns), _ptr(bias_shard),
                                   _ptr(Y_shard), _ld(Y_shard, Ns), _ptr(H_save), _ld(H_save, Ns)))


def row_parallel_fwd(X_shard, W_shard, tp_size: int, Z_partial, stream=None) -> None:
    """Z_partial (fp32) = X_shard @ W_shard."""
    T, Ks = _dims("X_shard", X_shard, 2)
    N = _dims("W_shard", W_shard, 2)[1]
    dt = _storage("X_shard", X_shard)
    _args(("X_shard", X_shard, (T, Ks), dt, False), ("W_shard", W_shard, (Ks, N), dt, False),
          ("Z_partial", Z_partial, (T, N), _F32T, False))
    _check(_get_lib().row_parallel_fwd(_stream(stream, X_shard), _dtype(X_shard), T, Ks * tp_size, N, tp_size,
                                _ptr(X_shard), _ld(X_shard, Ks), _ptr(W_shard), _ld(W_shard, N),
                                _ptr(Z_partial), _ld(Z_partial, N)))


def shard_partial_sum(partials, out, tp_size: Optional[int] = None, stream=None) -> None:
    """out = partials[0] + ... + partials[tp-1] (fp32, ascending).

    ``partials`` is a [tp, T, N] tensor (or a view with any shard stride and
    row stride); ``out`` is [T, N].
    """
    P, T, N = _dims("partials", partials, 3)
    tp = P if tp_size is None else tp_size
    if not 1 <= tp <= P:
        raise ValueError(f"tp_size {tp} outside [1, {P}] (partials holds {P} shards)")
    _args(("partials", partials, (P, T, N), _F32T, False), ("out", out, (T, N), _F32T, False))
    if T > 1 and N > 1 and partials.stride(2) != 1:
        raise ValueError("partials must be [tp, T, N] with contiguous rows")
    _check(_get_lib().shard_partial_sum(_stream(stream, out), tp, T, N, _ptr(partials), partials.stride(0),
                                 partials.stride(1) if T > 1 else N, _ptr(out), _ld(out, N)))


def tp_mlp_fwd(X, W1_shard, b1_shard, W2_shard, tp_size: int, A_save, Z_partial, H_save=None,
               stream=None) -> None:
    """One shard of Z = GeLU(X W1 + b1) W2: writes A_save, H_save (optional) and Z_partial."""
    T, h = _dims("X", X, 2)
    Fs = _dims("W1_shard", W1_shard, 2)[1]
    dt = _storage("X", X)
    _args(("X", X, (T, h), dt, False), ("W1_shard", W1_shard, (h, Fs), dt, False), ("b1_shard", b1_shard, (Fs,), dt, True),
          ("W2_shard", W2_shard, (Fs, h), dt, False), ("A_save", A_save, (T, Fs), dt, False),
          ("Z_partial", Z_partial, (T, h), _F32T, False), ("H_save", H_save, (T, Fs), dt, True))
    for n, t in (("X", X), ("W2_shard", W2_shard), ("A_save", A_save), ("Z_partial", Z_partial), ("H_save", H_save)):
        _require_contiguous(n, t)
    _check(_get_lib().tp_mlp_fwd(_stream(stream, X), _dtype(X), T, h, Fs * tp_size, tp_size, _ptr(X), _ptr(W1_shard),
                          _ld(W1_shard, Fs), _ptr(b1_shard), _ptr(W2_shard), _ptr(H_save), _ptr(A_save),
                          _ptr(Z_partial)))


def _mlp_bwd_args(X, W1_shard, W2_shard, H_save, A_save, dZ, dX_partial, dW1_shard, dW2_shard, db1_shard, T, h, Fs,
                  *extra):
    dt = _storage("X", X)
    _args(*extra, ("X", X, (T, h), dt, False), ("W1_shard", W1_shard, (h, Fs), dt, False),
          ("W2_shard", W2_shard, (Fs, h), dt, False), ("H_save", H_save, (T, Fs), dt, False),
          ("A_save", A_save, (T, Fs), dt, False), ("dZ", dZ, (T, h), dt, False),
          ("dX_partial", dX_partial, (T, h), _F32T, False), ("dW1_shard", dW1_shard, (h, Fs), _F32T, False),
          ("dW2_shard", dW2_shard, (Fs, h), _F32T, False), ("db1_shard", db1_shard, (Fs,), _F32T, True))


def tpmlp_bwd_workspace_bytes(dtype: int, T: int, h: int, F: int, tp_size: int) -> int:
    return int(_get_lib().tpmlp_bwd_workspace_bytes(dtype, T, h, F, tp_size))


def tp_mlp_bwd(X, W1_shard, W2_shard, H_save, A_save, dZ, tp_size: int, dX_partial, dW1_shard, dW2_shard,
               db1_shard=None, workspace=None, stream=None) -> None:
    """One shard's backward; workspace is a device uint8 tensor (allocated here if None)."""
    T, h = _dims("X", X, 2)
    Fs = _dims("W1_shard", W1_shard, 2)[1]
    F = Fs * tp_size
    _mlp_bwd_args(X, W1_shard, W2_shard, H_save, A_save, dZ, dX_partial, dW1_shard, dW2_shard, db1_shard, T, h, Fs,
                  *([] if workspace is None else [_ws("workspace", workspace)]))
    for n, t in (("X", X), ("W2_shard", W2_shard), ("H_save", H_save), ("A_save", A_save), ("dZ", dZ),
                 ("dX_partial", dX_partial), ("dW1_shard", dW1_shard), ("dW2_shard", dW2_shard)):
        _require_contiguous(n, t)
    dt = _dtype(X)
    if workspace is None:
        workspace = torch.empty(max(1, tpmlp_bwd_workspace_bytes(dt, T, h, F, tp_size)), dtype=torch.uint8,
                                device=X.device)
    _check(_get_lib().tp_mlp_bwd(_stream(stream, X), dt, T, h, F, tp_size, _ptr(X), _ptr(W1_shard), _ld(W1_shard, Fs),
                          _ptr(W2_shard), _ptr(H_save), _ptr(A_save), _ptr(dZ), _ptr(dX_partial), _ptr(dW1_shard),
                          _ptr(db1_shard), _ptr(dW2_shard), _ptr(workspace), workspace.numel()))


def tp_mlp_bwd_noalloc(X, W1_shard, W2_shard, H_save, A_save, dZ, tp_size: int, dX_partial, dW1_shard, dW2_shard,
                       db1_shard=None, stream=None) -> None:
    """tp_mlp_bwd with its workspace in the library's static device scratch array (no allocation)."""
    T, h = _dims("X", X, 2)
    Fs = _dims("W1_shard", W1_shard, 2)[1]
    F = Fs * tp_size
    _mlp_bwd_args(X, W1_shard, W2_shard, H_save, A_save, dZ, dX_partial, dW1_shard, dW2_shard, db1_shard, T, h, Fs)
    for n, t in (("X", X), ("W2_shard", W2_shard), ("H_save", H_save), ("A_save", A_save), ("dZ", dZ),
                 ("dX_partial", dX_partial), ("dW1_shard", dW1_shard), ("dW2_shard", dW2_shard)):
        _require_contiguous(n, t)
    _check(_get_lib().tp_mlp_bwd_noalloc(_stream(stream, X), _dtype(X), T, h, F, tp_size, _ptr(X), _ptr(W1_shard),
                                         _ld(W1_shard, Fs), _ptr(W2_shard), _ptr(H_save), _ptr(A_save), _ptr(dZ),
                                         _ptr(dX_partial), _ptr(dW1_shard), _ptr(db1_shard), _ptr(dW2_shard)))


def bias_gelu_fwd(Hin, A_out, bias=None, H_out=None, stream=None) -> None:
    """A_out = GeLU(Hin + bias), H_out = Hin + bias (Hin fp32; the rest in A_out's storage dtype)."""
    T, N = _dims("Hin", Hin, 2)
    dt = _storage("A_out", A_out)
    _args(("Hin", Hin, (T, N), _F32T, False), ("A_out", A_out, (T, N), dt, False), ("bias", bias, (N,), dt, True),
          ("H_out", H_out, (T, N), dt, True))
    _check(_get_lib().bias_gelu_fwd(_stream(stream, Hin), _dtype(A_out), T, N, _ptr(Hin), _ld(Hin, N), _ptr(bias),
                                    _ptr(A_out), _ld(A_out, N), _ptr(H_out), _ld(H_out, N)))


def gelu_bwd(dA, H, dH_out, stream=None) -> None:
    """dH_out = dA * GeLU'(H) (dA fp32; H and dH_out in the storage dtype)."""
    T, N = _dims("dA", dA, 2)
    dt = _storage("H", H)
    _args(("dA", dA, (T, N), _F32T, False), ("H", H, (T, N), dt, False), ("dH_out", dH_out, (T, N), dt, False))
    _check(_get_lib().gelu_bwd(_stream(stream, dA), _dtype(H), T, N, _ptr(dA), _ld(dA, N), _ptr(H), _ld(H, N),
                               _ptr(dH_out), _ld(dH_out, N)))


def tpmlp_noalloc_scratch_bytes() -> int:
    return int(_get_lib().tpmlp_noalloc_scratch_bytes())


def column_parallel_bwd(X, W_shard, dY, tp_size: int, dX_partial, dW_shard, db_shard=None, stream=None) -> None:
    """dX_partial = dY W_shard^T, dW_shard = X^T dY, db_shard = column sums of dY (fp32 outputs)."""
    T, K = _dims("X", X, 2)
    Ns = _dims("W_shard", W_shard, 2)[1]
    dt = _storage("X", X)
    _args(("X", X, (T, K), dt, False), ("W_shard", W_shard, (K, Ns), dt, False), ("dY", dY, (T, Ns), dt, False),
          ("dX_partial", dX_partial, (T, K), _F32T, False), ("dW_shard", dW_shard, (K, Ns), _F32T, False),
          ("db_shard", db_shard, (Ns,), _F32T, True))
    _check(_get_lib().column_parallel_bwd(_stream(stream, X), _dtype(X), T, K, Ns * tp_size, tp_size, _ptr(X), _ld(X, K),
                                   _ptr(W_shard), _ld(W_shard, Ns), _ptr(dY), _ld(dY, Ns), _ptr(dX_partial),
                                   _ld(dX_partial, K), _ptr(dW_shard), _ld(dW_shard, Ns), _ptr(db_shard)))


def row_parallel_bwd(X_shard, W_shard, dY, tp_size: int, dX_shard, dW_shard, stream=None) -> None:
    """dX_shard = dY W_shard^T, dW_shard = X_shard^T dY (fp32 outputs)."""
    T, Ks = _dims("X_shard", X_shard, 2)
    N = _dims("W_shard", W_shard, 2)[1]
    dt = _storage("X_shard", X_shard)
    _args(("X_shard", X_shard, (T, Ks), dt, False), ("W_shard", W_shard, (Ks, N), dt, False),
          ("dY", dY, (T, N), dt, False), ("dX_shard", dX_shard, (T, Ks), _F32T, False),
          ("dW_shard", dW_shard, (Ks, N), _F32T, False))
    _check(_get_lib().row_parallel_bwd(_stream(stream, X_shard), _dtype(X_shard), T, Ks * tp_size, N, tp_size,
                                _ptr(X_shard), _ld(X_shard, Ks), _ptr(W_shard), _ld(W_shard, N), _ptr(dY),
                                _ld(dY, N), _ptr(dX_shard), _ld(dX_shard, Ks), _ptr(dW_shard), _ld(dW_shard, N)))


def swiglu_pack_shard(W_gate, W_up, tp_size: int, shard: int, W_gu_shard, stream=None) -> None:
    """W_gu_shard [h, 2F/tp] = shard `shard` of [W_gate | W_up], interleaved in groups of 8 columns."""
    h, F = _dims("W_gate", W_gate, 2)
    dt = _storage("W_gate", W_gate)
    if tp_size < 1 or F % tp_size:
        raise ValueError(f"F = {F} is not divisible by tp_size {tp_size}")
    _args(("W_gate", W_gate, (h, F), dt, False), ("W_up", W_up, (h, F), dt, False),
          ("W_gu_shard", W_gu_shard, (h, 2 * (F // tp_size)), dt, False))
    _require_contiguous("W_gu_shard", W_gu_shard)
    _check(_get_lib().swiglu_pack_shard(_stream(stream, W_gate), _dtype(W_gate), h, F, tp_size, shard,
                                        _ptr(W_gate), _ld(W_gate, F), _ptr(W_up), _ld(W_up, F), _ptr(W_gu_shard)))


def swiglu_unpack_grad(dW_gu_shard, tp_size: int, shard: int, dW_gate, dW_up, stream=None) -> None:
    """Columns of shard `shard` of dW_gate and dW_up [h, F] (fp32) from the packed dW_gu_shard."""
    h, F = _dims("dW_gate", dW_gate, 2)
    if tp_size < 1 or F % tp_size:
        raise ValueError(f"F = {F} is not divisible by tp_size {tp_size}")
    _args(("dW_gu_shard", dW_gu_shard, (h, 2 * (F // tp_size)), _F32T, False), ("dW_gate", dW_gate, (h, F), _F32T, False),
          ("dW_up", dW_up, (h, F), _F32T, False))
    _require_contiguous("dW_gu_shard", dW_gu_shard)
    _check(_get_lib().swiglu_unpack_grad(_stream(stream, dW_gu_shard), h, F, tp_size, shard, _ptr(dW_gu_shard),
                                         _ptr(dW_gate), _ld(dW_gate, F), _ptr(dW_up), _ld(dW_up, F)))


def tp_swiglu_fwd(X, W_gu_shard, W_down_shard, tp_size: int, A_save, Z_partial, GU_save=None, stream=None) -> None:
    """One shard of down = (silu(X W_gate) * (X W_up)) W_down: writes A_save, GU_save (optional), Z_partial."""
    T, h = _dims("X", X, 2)
    Fs = _dims("W_down_shard", W_down_shard, 2)[0]
    dt = _storage("X", X)   # the library itself refuses fp32 storage for the gated MLP
    _args(("X", X, (T, h), dt, False), ("W_gu_shard", W_gu_shard, (h, 2 * Fs), dt, False),
          ("W_down_shard", W_down_shard, (Fs, h), dt, False), ("A_save", A_save, (T, Fs), dt, False),
          ("Z_partial", Z_partial, (T, h), _F32T, False), ("GU_save", GU_save, (T, 2 * Fs), dt, True))
    for n, t in (("X", X), ("W_gu_shard", W_gu_shard), ("W_down_shard", W_down_shard), ("A_save", A_save),
                 ("Z_partial", Z_partial), ("GU_save", GU_save)):
        _require_contiguous(n, t)
    _check(_get_lib().tp_swiglu_fwd(_stream(stream, X), _dtype(X), T, h, Fs * tp_size, tp_size, _ptr(X),
                                    _ptr(W_gu_shard), _ptr(W_down_shard), _ptr(GU_save), _ptr(A_save),
                                    _ptr(Z_partial)))


def tp_swiglu_bwd_workspace_bytes(dtype: int, T: int, h: int, F: int, tp_size: int) -> int:
    return int(_get_lib().tp_swiglu_bwd_workspace_bytes(dtype, T, h, F, tp_size))


def tp_swiglu_bwd(X, W_gu_shard, W_down_shard, GU_save, A_save, dZ, tp_size: int, dX_partial, dW_gu_shard,
                  dW_down_shard, workspace=None, stream=None) -> None:
    """One shard's backward of the gated MLP; workspace is a device uint8 tensor (allocated here if None)."""
    T, h = _dims("X", X, 2)
    Fs = _dims("W_down_shard", W_down_shard, 2)[0]
    F = Fs * tp_size
    dt = _storage("X", X)
    _args(("X", X, (T, h), dt, False), ("W_gu_shard", W_gu_shard, (h, 2 * Fs), dt, False),
          ("W_down_shard", W_down_shard, (Fs, h), dt, False), ("GU_save", GU_save, (T, 2 * Fs), dt, False),
          ("A_save", A_save, (T, Fs), dt, False), ("dZ", dZ, (T, h), dt, False),
          ("dX_partial", dX_partial, (T, h), _F32T, False), ("dW_gu_shard", dW_gu_shard, (h, 2 * Fs), _F32T, False),
          ("dW_down_shard", dW_down_shard, (Fs, h), _F32T, False),
          *([] if workspace is None else [_ws("workspace", workspace)]))
    for n, t in (("X", X), ("W_gu_shard", W_gu_shard), ("W_down_shard", W_down_shard), ("GU_save", GU_save),
                 ("A_save", A_save), ("dZ", dZ), ("dX_partial", dX_partial), ("dW_gu_shard", dW_gu_shard),
                 ("dW_down_shard", dW_down_shard)):
        _require_contiguous(n, t)
    dt = _dtype(X)
    if workspace is None:
        workspace = torch.empty(max(1, tp_swiglu_bwd_workspace_bytes(dt, T, h, F, tp_size)), dtype=torch.uint8,
                                device=X.device)
    _check(_get_lib().tp_swiglu_bwd(_stream(stream, X), dt, T, h, F, tp_size, _ptr(X), _ptr(W_gu_shard),
                                    _ptr(W_down_shard), _ptr(GU_save), _ptr(A_save), _ptr(dZ), _ptr(dX_partial),
                                    _ptr(dW_gu_shard), _ptr(dW_down_shard), _ptr(workspace), workspace.numel()))


def layernorm_fwd(X, gamma, beta, Y, mean, rstd, eps: float = 1e-5, stream=None) -> None:
    """Y = LayerNorm(X) per row (bf16 in/out, fp32 gamma/beta/statistics).  Y may be a row block of a larger buffer."""
    rows, h = _dims("X", X, 2)
    _args(("X", X, (rows, h), _BF16T, False), ("gamma", gamma, (h,), _F32T, False), ("beta", beta, (h,), _F32T, False),
          ("Y", Y, (rows, h), _BF16T, False), ("mean", mean, (rows,), _F32T, False),
          ("rstd", rstd, (rows,), _F32T, False))
    _check(_get_lib().layernorm_fwd(_stream(stream, X), rows, h, _ptr(X), _ld(X, h), _ptr(gamma), _ptr(beta), eps,
                                    _ptr(Y), _ld(Y, h), _ptr(mean), _ptr(rstd)))


def layernorm_bwd(X, gamma, mean, rstd, dY, dX, dgamma=None, dbeta=None, dRes=None, stream=None) -> None:
    """dX (fp32) from dY (fp32), plus dRes (bf16) if given; dgamma/dbeta = this block's sums (fp32)."""
    rows, h = _dims("X", X, 2)
    _args(("X", X, (rows, h), _BF16T, False), ("gamma", gamma, (h,), _F32T, False), ("mean", mean, (rows,), _F32T, False),
          ("rstd", rstd, (rows,), _F32T, False), ("dY", dY, (rows, h), _F32T, False), ("dX", dX, (rows, h), _F32T, False),
          ("dgamma", dgamma, (h,), _F32T, True), ("dbeta", dbeta, (h,), _F32T, True),
          ("dRes", dRes, (rows, h), _BF16T, True))
    _check(_get_lib().layernorm_bwd(_stream(stream, X), rows, h, _ptr(X), _ld(X, h), _ptr(gamma), _ptr(mean),
                                    _ptr(rstd), _ptr(dY), _ld(dY, h), _ptr(dRes), _ld(dRes, h), _ptr(dX), _ld(dX, h),
                                    _ptr(dgamma), _ptr(dbeta)))


def sp_partial_sum_dropout_residual(partials, residual, out, p: float, seed: int, row0: int,
                                    tp_size: Optional[int] = None, stream=None) -> None:
    """out = residual + Dropout(sum of partials[s]) over this GPU's rows (partials: [tp, rows, h] view, fp32)."""
    P, rows, h = _dims("partials", partials, 3)
    tp = P if tp_size is None else tp_size
    if not 1 <= tp <= P:
        raise ValueError(f"tp_size {tp} outside [1, {P}] (partials holds {P} shards)")
    _args(("partials", partials, (P, rows, h), _F32T, False), ("residual", residual, (rows, h), _BF16T, False),
          ("out", out, (rows, h), _BF16T, False))
    if rows > 1 and h > 1 and partials.stride(2) != 1:
        raise ValueError("partials must be [tp, rows, h] with contiguous rows")
    _check(_get_lib().sp_partial_sum_dropout_residual(_stream(stream, out), tp, rows, h, _ptr(partials),
                                                      partials.stride(0), partials.stride(1) if rows > 1 else h,
                                                      _ptr(residual), _ld(residual, h), p, seed, row0, _ptr(out),
                                                      _ld(out, h)))


def sp_dropout_bwd(dOut, dZ, p: float, seed: int, row0: int, stream=None) -> None:
    """dZ = Dropout'(dOut) for this GPU's rows (bf16); dZ may be a row block of the gathered gradient."""
    rows, h = _dims("dOut", dOut, 2)
    _args(("dOut", dOut, (rows, h), _BF16T, False), ("dZ", dZ, (rows, h), _BF16T, False))
    _check(_get_lib().sp_dropout_bwd(_stream(stream, dOut), rows, h, _ptr(dOut), _ld(dOut, h), p, seed, row0,
                                     _ptr(dZ), _ld(dZ, h)))


def attn_fwd_workspace_bytes(batch: int, seq: int, heads: int) -> int:
    return int(_get_lib().attn_fwd_workspace_bytes(batch, seq, heads))


def attn_fwd(Q, K, V, O, batch: int, seq: int, heads: int, causal: bool = True, scale: Optional[float] = None,
             lse=None, workspace=None, head_dim: int = 128, stream=None) -> None:
    """O = softmax(Q K^T * scale) V per head (bf16; head h in columns [128h, 128h+128)); lse [heads, T] fp32;
    workspace a device uint8 tensor (allocated here if None and needed)."""
    w = heads * head_dim
    T = batch * seq
    sc = head_dim ** -0.5 if scale is None else scale
    _args(("Q", Q, (T, w), _BF16T, False), ("K", K, (T, w), _BF16T, False), ("V", V, (T, w), _BF16T, False),
          ("O", O, (T, w), _BF16T, False), ("lse", lse, (heads, T), _F32T, True),
          *([] if workspace is None else [_ws("workspace", workspace)]))
    if workspace is None and causal:
        n = attn_fwd_workspace_bytes(batch, seq, heads)
        if n > 0:
            workspace = torch.empty(n, dtype=torch.uint8, device=Q.device)
    _check(_get_lib().attn_fwd(_stream(stream, O), batch, seq, heads, head_dim, int(bool(causal)), sc, _ptr(Q),
                               _ld(Q, w), _ptr(K), _ld(K, w), _ptr(V), _ld(V, w), _ptr(O), _ld(O, w), _ptr(lse),
                               _ptr(workspace), 0 if workspace is None else workspace.numel()))


def attn_bwd_workspace_bytes(batch: int, seq: int, heads: int) -> int:
    return int(_get_lib().attn_bwd_workspace_bytes(batch, seq, heads))


def attn_bwd(Q, K, V, O, dO, lse, dQ, dK, dV, batch: int, seq: int, heads: int, causal: bool = True,
             scale: Optional[float] = None, workspace=None, head_dim: int = 128, stream=None) -> None:
    """dQ, dK, dV (bf16) of attn_fwd for upstream dO; workspace a device uint8 tensor (allocated here if None)."""
    w = heads * head_dim
    T = batch * seq
    sc = head_dim ** -0.5 if scale is None else scale
    _args(*[(n, t, (T, w), _BF16T, False) for n, t in (("Q", Q), ("K", K), ("V", V), ("O", O), ("dO", dO), ("dQ", dQ),
                                                         ("dK", dK), ("dV", dV))],
          ("lse", lse, (heads, T), _F32T, False), *([] if workspace is None else [_ws("workspace", workspace)]))
    if workspace is None:
        workspace = torch.empty(max(1, attn_bwd_workspace_bytes(batch, seq, heads)), dtype=torch.uint8,
                                device=Q.device)
    _check(_get_lib().attn_bwd(_stream(stream, Q), batch, seq, heads, head_dim, int(bool(causal)), sc, _ptr(Q),
                               _ld(Q, w), _ptr(K), _ld(K, w), _ptr(V), _ld(V, w), _ptr(O), _ld(O, w), _ptr(dO),
                               _ld(dO, w), _ptr(lse), _ptr(dQ), _ld(dQ, w), _ptr(dK), _ld(dK, w), _ptr(dV),
                               _ld(dV, w), _ptr(workspace), workspace.numel()))


def tp_attn_fwd_workspace_bytes(batch: int, seq: int, heads: int, tp_size: int, head_dim: int = 128) -> int:
    return int(_get_lib().tp_attn_fwd_workspace_bytes(batch, seq, heads, head_dim, tp_size))


def tp_attn_fwd(X, Wqkv_shard, Wo_shard, QKV_save, O_save, lse, Z_partial, batch: int, seq: int, heads: int,
                tp_size: int, causal: bool = True, scale: Optional[float] = None, workspace=None,
                head_dim: int = 128, stream=None) -> None:
    """One shard of the head-sharded attention block (contiguous tensors; heads = all heads of the layer);
    workspace a device uint8 tensor (allocated here if None and needed)."""
    T, h = _dims("X", X, 2)
    if tp_size < 1 or heads % tp_size:
        raise ValueError(f"heads = {heads} is not divisible by tp_size {tp_size}")
    hs = heads // tp_size
    w = hs * head_dim
    if T != batch * seq:
        raise ValueError(f"X has {T} rows, expected batch * seq = {batch * seq}")
    _args(("X", X, (T, h), _BF16T, False), ("Wqkv_shard", Wqkv_shard, (h, 3 * w), _BF16T, False),
          ("Wo_shard", Wo_shard, (w, h), _BF16T, False), ("QKV_save", QKV_save, (T, 3 * w), _BF16T, False),
          ("O_save", O_save, (T, w), _BF16T, False), ("lse", lse, (hs, T), _F32T, False),
          ("Z_partial", Z_partial, (T, h), _F32T, False), *([] if workspace is None else [_ws("workspace", workspace)]))
    sc = head_dim ** -0.5 if scale is None else scale
    for n, t in (("X", X), ("Wqkv_shard", Wqkv_shard), ("Wo_shard", Wo_shard), ("QKV_save", QKV_save),
                 ("O_save", O_save), ("lse", lse), ("Z_partial", Z_partial)):
        _require_contiguous(n, t)
    if workspace is None and causal:
        n = tp_attn_fwd_workspace_bytes(batch, seq, heads, tp_size, head_dim)
        if n > 0:
            workspace = torch.empty(n, dtype=torch.uint8, device=X.device)
    _check(_get_lib().tp_attn_fwd(_stream(stream, X), batch, seq, h, heads, head_dim, tp_size, int(bool(causal)), sc,
                                  _ptr(X), _ptr(Wqkv_shard), _ptr(Wo_shard), _ptr(QKV_save), _ptr(O_save), _ptr(lse),
                                  _ptr(Z_partial), _ptr(workspace), 0 if workspace is None else workspace.numel()))


def tp_attn_bwd_workspace_bytes(batch: int, seq: int, heads: int, tp_size: int, head_dim: int = 128) -> int:
    return int(_get_lib().tp_attn_bwd_workspace_bytes(batch, seq, heads, head_dim, tp_size))


def tp_attn_bwd(X, Wqkv_shard, Wo_shard, QKV_save, O_save, lse, dZ, dX_partial, dWqkv_shard, dWo_shard,
                batch: int, seq: int, heads: int, tp_size: int, causal: bool = True, scale: Optional[float] = None,
                workspace=None, head_dim: int = 128, stream=None) -> None:
    """Backward of tp_attn_fwd for dZ; workspace a device uint8 tensor (allocated here if None)."""
    T, h = _dims("X", X, 2)
    if tp_size < 1 or heads % tp_size:
        raise ValueError(f"heads = {heads} is not divisible by tp_size {tp_size}")
    hs = heads // tp_size
    w = hs * head_dim
    if T != batch * seq:
        raise ValueError(f"X has {T} rows, expected batch * seq = {batch * seq}")
    _args(("X", X, (T, h), _BF16T, False), ("Wqkv_shard", Wqkv_shard, (h, 3 * w), _BF16T, False),
          ("Wo_shard", Wo_shard, (w, h), _BF16T, False), ("QKV_save", QKV_save, (T, 3 * w), _BF16T, False),
          ("O_save", O_save, (T, w), _BF16T, False), ("lse", lse, (hs, T), _F32T, False),
          ("dZ", dZ, (T, h), _BF16T, False), ("dX_partial", dX_partial, (T, h), _F32T, False),
          ("dWqkv_shard", dWqkv_shard, (h, 3 * w), _F32T, False), ("dWo_shard", dWo_shard, (w, h), _F32T, False),
          *([] if workspace is None else [_ws("workspace", workspace)]))
    sc = head_dim ** -0.5 if scale is None else scale
    for n, t in (("X", X), ("Wqkv_shard", Wqkv_shard), ("Wo_shard", Wo_shard), ("QKV_save", QKV_save),
                 ("O_save", O_save), ("lse", lse), ("dZ", dZ), ("dX_partial", dX_partial),
                 ("dWqkv_shard", dWqkv_shard), ("dWo_shard", dWo_shard)):
        _require_contiguous(n, t)
    if workspace is None:
        workspace = torch.empty(max(1, tp_attn_bwd_workspace_bytes(batch, seq, heads, tp_size, head_dim)),
                                dtype=torch.uint8, device=X.device)
    _check(_get_lib().tp_attn_bwd(_stream(stream, X), batch, seq, h, heads, head_dim, tp_size, int(bool(causal)), sc,
                                  _ptr(X), _ptr(Wqkv_shard), _ptr(Wo_shard), _ptr(QKV_save), _ptr(O_save), _ptr(lse),
                                  _ptr(dZ), _ptr(dX_partial), _ptr(dWqkv_shard), _ptr(dWo_shard), _ptr(workspace),
                                  workspace.numel()))


def profile_enable(filter: Optional[str] = "") -> None:
    """Bracket matching kernel launches with HIP events (None disables)."""
    _check(_get_lib().tpmlp_profile_enable(None if filter is None else filter.encode()))


def profile_collect(ordered: bool = False):
    """Launches recorded since the last collect.

    ordered=True: [(role, symbol), ...] in launch order.  Otherwise
    {role|symbol: (launches, total_ms, symbol, clocks_ghz)}, where clocks_ghz
    lists the shader clock sampled over workgroup 0's main loop of each
    bf16 GEMM launch (empty for other kernels).
    """
    buf = ctypes.create_string_buffer(1 << 20)
    _check(_get_lib().tpmlp_profile_collect(buf, len(buf)))
    recs = json.loads(buf.value.decode() or "[]")
    if ordered:
        return [(r[0], r[1]) for r in recs]
    agg = {}
    for role, sym, ms, ghz in recs:
        n, tot, _, clocks = agg.get(f"{role}|{sym}", (0, 0.0, sym, []))
        agg[f"{role}|{sym}"] = (n + 1, tot + ms, sym, clocks + ([ghz] if ghz > 0 else []))
    return agg
