"""Host-side checks of the C ABI (no GPU needed).

The library loads, exports every function include/tpmlp.h declares, and
refuses bad arguments on the host before any HIP call, with the documented
status codes.  Only invalid calls are made here, so no kernel is launched.
"""
import ctypes
import os
import re

import pytest

import linear_layers_amd as tl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, E_NULL, E_SHAPE, E_DIV, E_ALIGN, E_DTYPE, E_ACT, E_WS = 0, 1, 2, 3, 4, 5, 6, 7
P = 0x100000  # a 16-byte aligned stand-in address; never dereferenced (validation fails first)


def declared_functions():
    src = open(os.path.join(ROOT, "include", "tpmlp.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char\s*\*|const char\s*\*)\s*\*?\s*(\w+)\s*\(",
                                 src, flags=re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert {"column_parallel_fwd", "row_parallel_fwd", "shard_partial_sum", "tp_mlp_fwd", "tp_mlp_bwd",
            "column_parallel_bwd", "row_parallel_bwd"} <= set(names)
    handle = ctypes.CDLL(tl.LIB_PATH)
    for n in names:
        assert hasattr(handle, n), f"{n} declared but not exported"


def test_status_strings():
    for code, name in [(OK, "TPMLP_OK"), (E_DIV, "TPMLP_E_DIVISIBILITY"), (8, "TPMLP_E_HIP")]:
        assert tl.status_string(code) == name


def call_fwd(dtype=1, T=64, h=64, F=128, tp=2, X=P, W1=P, ldw1=64, b1=None, W2=P, H=None, A=P, Z=P):
    return tl.lib.tp_mlp_fwd(None, dtype, T, h, F, tp, X, W1, ldw1, b1, W2, H, A, Z)


@pytest.mark.parametrize("kw,status", [
    (dict(tp=3), E_DIV), (dict(tp=0), E_DIV), (dict(tp=-1), E_DIV),
    (dict(T=-1), E_SHAPE), (dict(h=0), E_SHAPE), (dict(F=0), E_SHAPE),
    (dict(ldw1=32), E_SHAPE), (dict(T=1 << 31), E_SHAPE),
    (dict(X=None), E_NULL), (dict(W1=None), E_NULL), (dict(A=None), E_NULL), (dict(Z=None), E_NULL),
    (dict(X=P + 2), E_ALIGN), (dict(Z=P + 4), E_ALIGN), (dict(h=60), E_ALIGN), (dict(ldw1=68), E_ALIGN),
    (dict(F=2 * 60), E_ALIGN), (dict(dtype=2), E_DTYPE), (dict(dtype=0, h=62), E_ALIGN),
    # a leading dimension of 2^22 elements or more is refused before the first of the two GEMMs
    (dict(ldw1=1 << 22), E_SHAPE), (dict(h=1 << 22, ldw1=64), E_SHAPE),
])
def test_tp_mlp_fwd_validation(kw, status):
    assert call_fwd(**kw) == status
    assert tl.lib.tpmlp_last_error().decode() != ""


def test_divisibility_message():
    assert call_fwd(F=96, tp=5) == E_DIV
    assert b"not divisible by tp_size 5" in tl.lib.tpmlp_last_error()


def test_column_parallel_fwd_validation():
    f = tl.lib.column_parallel_fwd
    assert f(None, 1, 9, 8, 16, 32, 2, P, 16, P, 16, None, P, 16, None, 16) == E_ACT
    assert f(None, 1, 1, 8, 16, 30, 4, P, 16, P, 8, None, P, 8, None, 8) == E_DIV
    assert f(None, 1, 1, 8, 16, 32, 2, P, 8, P, 16, None, P, 16, None, 16) == E_SHAPE     # ldx < K
    assert f(None, 1, 1, 8, 16, 32, 2, P, 16, P, 16, P + 8, P, 16, None, 16) == E_ALIGN  # bias misaligned
    assert f(None, 1, 1, 8, 16, 32, 2, P, 16, P, 16, None, P, 16, P, 8) == E_SHAPE       # ldh < width


def test_row_parallel_and_partial_sum_validation():
    assert tl.lib.row_parallel_fwd(None, 1, 8, 30, 16, 4, P, 8, P, 16, P, 16) == E_DIV
    assert tl.lib.row_parallel_fwd(None, 1, 8, 32, 16, 2, P, 16, P, 16, P, 12) == E_SHAPE
    s = tl.lib.shard_partial_sum
    assert s(None, 0, 8, 16, P, 128, 16, P + 4096, 16) == E_DIV
    assert s(None, 2, 8, 18, P, 144, 18, P + 4096, 18) == E_ALIGN
    assert s(None, 2, 8, 16, P, 130, 16, P + 4096, 16) == E_ALIGN
    assert s(None, 2, 8, 16, P, 128, 16, P + 256, 16) == E_SHAPE     # out overlaps partial 0 (not exactly)
    assert s(None, 2, 8, 16, P, 128, 16, P, 20) == E_SHAPE           # in place needs ldo == ldp
    assert s(None, 2, 8, 16, None, 128, 16, P, 16) == E_NULL


def test_bwd_validation_and_workspace_size():
    ws = tl.tpmlp_bwd_workspace_bytes(1, 4096, 1024, 4096, 2)
    assert ws >= 4096 * 2048 * 2 and ws % 256 == 0
    assert tl.tpmlp_bwd_workspace_bytes(1, 8, 8, 30, 4) == 0
    f = tl.lib.tp_mlp_bwd
    args = [None, 1, 64, 64, 128, 2, P, P, 64, P, P, P, P, P, P, None, P]
    assert f(*args, P, 16) == E_WS
    assert f(*args, None, ws) == E_NULL
    assert f(*args, P + 16, 1 << 30) == E_ALIGN
    assert tl.lib.column_parallel_bwd(None, 1, 8, 16, 30, 4, P, 16, P, 8, P, 8, P, 16, P, 8, None) == E_DIV
    assert tl.lib.row_parallel_bwd(None, 1, 8, 32, 16, 2, P, 16, P, 16, P, 16, P, 16, P, 8) == E_SHAPE
    # two GEMMs each: every leading dimension is checked before the first launch
    assert tl.lib.column_parallel_bwd(None, 1, 8, 16, 32, 2, P, 1 << 22, P, 16, P, 16, P, 16, P, 16, None) == E_SHAPE
    assert tl.lib.row_parallel_bwd(None, 1, 8, 32, 16, 2, P, 16, P, 16, P, 1 << 22, P, 16, P, 16) == E_SHAPE
    big = [None, 1, 64, 64, 128, 2, P, P, 1 << 22, P, P, P, P, P, P, None, P]
    assert f(*big, P, 1 << 30) == E_SHAPE


def test_swiglu_validation():
    fwd = tl.lib.tp_swiglu_fwd
    # (stream, dtype, T, h, F, tp, X, W_gu, W_down, GU, A, Z); every call here is refused on the host
    assert fwd(None, 0, 64, 64, 256, 2, P, P, P, None, P, P) == E_DTYPE   # fp32 is not implemented
    assert fwd(None, 1, 64, 64, 40, 2, P, P, P, None, P, P) == E_DIV     # F/tp = 20, not a multiple of 8
    assert fwd(None, 1, 64, 64, 256, 3, P, P, P, None, P, P) == E_DIV    # 256 % 3
    assert fwd(None, 1, 64, 64, 256, 2, None, P, P, None, P, P) == E_NULL
    assert fwd(None, 1, 64, 64, 256, 2, P, P, P, P + 8, P, P) == E_ALIGN
    bwd = tl.lib.tp_swiglu_bwd
    ws = tl.tp_swiglu_bwd_workspace_bytes(1, 64, 64, 256, 2)
    assert ws >= 64 * 256 * 2 and ws % 256 == 0
    assert tl.tp_swiglu_bwd_workspace_bytes(0, 64, 64, 256, 2) == 0
    assert tl.tp_swiglu_bwd_workspace_bytes(1, 64, 64, 40, 2) == 0
    args = [None, 1, 64, 64, 256, 2, P, P, P, P, P, P, P, P, P]
    assert bwd(*args, P, 16) == E_WS
    assert bwd(*args, None, ws) == E_NULL
    assert bwd(*args, P + 16, ws) == E_ALIGN
    pack = tl.lib.swiglu_pack_shard
    assert pack(None, 1, 64, 256, 2, 2, P, 256, P, 256, P) == E_SHAPE    # shard out of range
    assert pack(None, 1, 64, 256, 2, -1, P, 256, P, 256, P) == E_SHAPE
    assert pack(None, 1, 64, 40, 2, 0, P, 40, P, 40, P) == E_DIV
    assert pack(None, 1, 64, 256, 2, 0, P, 128, P, 256, P) == E_SHAPE    # ldg < F
    unpack = tl.lib.swiglu_unpack_grad
    assert unpack(None, 64, 256, 2, 0, P, P, 256, P, 250) == E_SHAPE     # ldu < F
    assert unpack(None, 64, 256, 2, 0, P, P, 258, P, 256) == E_ALIGN


E_VALUE = 9


def test_sp_validation():
    lib = tl.lib
    assert tl.status_string(E_VALUE) == "TPMLP_E_VALUE"
    # layernorm_fwd(stream, rows, h, X, ldx, gamma, beta, eps, Y, ldy, mean, rstd): refused on the host
    assert lib.layernorm_fwd(None, 8, 64, P, 64, P, P, 0.0, P, 64, P, P) == E_VALUE
    assert lib.layernorm_fwd(None, 8, 60, P, 64, P, P, 1e-5, P, 64, P, P) == E_ALIGN
    assert lib.layernorm_fwd(None, 8, 16392, P, 16392, P, P, 1e-5, P, 16392, P, P) == E_SHAPE
    assert lib.layernorm_fwd(None, 8, 64, P, 64, None, P, 1e-5, P, 64, P, P) == E_NULL
    assert lib.layernorm_fwd(None, 8, 64, P, 32, P, P, 1e-5, P, 64, P, P) == E_SHAPE
    assert lib.layernorm_bwd(None, 8, 64, P, 64, P, P, P, P, 64, P + 8, 64, P, 64, None, None) == E_ALIGN
    assert lib.layernorm_bwd(None, 8, 64, P, 64, P, P, P, None, 64, None, 64, P, 64, None, None) == E_NULL
    s = lib.sp_partial_sum_dropout_residual
    assert s(None, 2, 8, 64, P, 512, 64, P, 64, 1.0, 1, 0, P, 64) == E_VALUE
    assert s(None, 2, 8, 64, P, 512, 64, P, 64, -0.1, 1, 0, P, 64) == E_VALUE
    assert s(None, 2, 8, 64, P, 512, 64, P, 64, float("nan"), 1, 0, P, 64) == E_VALUE
    assert s(None, 0, 8, 64, P, 512, 64, P, 64, 0.1, 1, 0, P, 64) == E_DIV
    assert s(None, 2, 8, 64, P, 514, 64, P, 64, 0.1, 1, 0, P, 64) == E_ALIGN
    assert s(None, 2, 8, 64, P, 512, 64, P, 64, 0.1, 1, -1, P, 64) == E_SHAPE
    d = lib.sp_dropout_bwd
    assert d(None, 8, 64, P, 64, 1.5, 1, 0, P, 64) == E_VALUE
    assert d(None, 8, 64, P, 64, 0.1, 1, 0, None, 64) == E_NULL
    assert d(None, 8, 64, P, 60, 0.1, 1, 0, P, 64) == E_SHAPE


def test_attn_validation():
    f = tl.lib.attn_fwd
    # (stream, batch, seq, heads, head_dim, causal, scale, Q, ldq, K, ldk, V, ldv, O, ldo, lse, workspace, bytes):
    # refused on the host
    assert f(None, 1, 8, 1, 64, 1, 0.1, P, 64, P, 64, P, 64, P, 64, None, None, 0) == E_SHAPE
    assert f(None, 1, 8, 1, 128, 2, 0.1, P, 128, P, 128, P, 128, P, 128, None, None, 0) == E_VALUE
    for bad in (float("inf"), 0.0, -0.1):   # the scale must be finite and positive
        assert f(None, 1, 8, 1, 128, 1, bad, P, 128, P, 128, P, 128, P, 128, None, None, 0) == E_VALUE
    assert f(None, 1, 8, 0, 128, 1, 0.1, P, 128, P, 128, P, 128, P, 128, None, None, 0) == E_SHAPE
    assert f(None, 1, 8, 2, 128, 1, 0.1, P, 128, P, 256, P, 256, P, 256, None, None, 0) == E_SHAPE   # ldq < heads*128
    assert f(None, 1, 8, 1, 128, 1, 0.1, None, 128, P, 128, P, 128, P, 128, None, None, 0) == E_NULL
    assert f(None, 1, 8, 1, 128, 1, 0.1, P, 128, P, 128, P, 128, P + 8, 128, None, None, 0) == E_ALIGN
    # causal, 4096 tokens: key chunks need the workspace (checked after the shapes); up to 1664
    # tokens (26 key blocks of 64, one chunk) every query block is whole and none is needed
    need = tl.attn_fwd_workspace_bytes(1, 4096, 1)
    assert need >= 2 * 16 * 128 * 128 * 4
    assert tl.attn_fwd_workspace_bytes(1, 1664, 1) == 0 and tl.attn_fwd_workspace_bytes(1, 1728, 1) > 0
    fw = [None, 1, 4096, 1, 128, 1, 0.1, P, 128, P, 128, P, 128, P, 128, None]
    assert f(*fw, None, 0) == E_NULL
    assert f(*fw, P, need - 1) == E_WS
    assert f(*fw, P + 16, need) == E_ALIGN
    b = tl.lib.attn_bwd
    args = [None, 1, 8, 1, 128, 1, 0.1, P, 128, P, 128, P, 128, P, 128, P, 128, P, P, 128, P, 128, P, 128]
    assert b(*args, P, 16) == E_WS
    assert b(*args, None, 1 << 20) == E_NULL
    assert b(*args, P + 16, 1 << 20) == E_ALIGN
    args[15] = None   # lse is required by the backward
    assert b(*args, P, 1 << 20) == E_NULL


def test_attn_block_validation():
    f = tl.lib.tp_attn_fwd
    # (stream, batch, seq, h, heads, head_dim, tp, causal, scale, X, Wqkv, Wo, QKV, O, lse, Z, workspace, bytes):
    # refused on the host
    assert f(None, 1, 8, 512, 4, 128, 3, 1, 0.1, P, P, P, P, P, P, P, None, 0) == E_DIV       # 4 heads over 3 shards
    assert f(None, 1, 8, 512, 4, 64, 2, 1, 0.1, P, P, P, P, P, P, P, None, 0) == E_SHAPE      # head_dim 64
    assert f(None, 1, 8, 512, 4, 128, 2, 3, 0.1, P, P, P, P, P, P, P, None, 0) == E_VALUE     # causal not 0/1
    assert f(None, 1, 8, 512, 4, 128, 2, 1, 0.1, P, P, P, P, P, None, P, None, 0) == E_NULL   # lse required
    assert f(None, 1, 8, 512, 4, 128, 2, 1, 0.1, P, P, P + 8, P, P, P, P, None, 0) == E_ALIGN
    # the attention core's workspace is checked before the QKV projection is launched
    need = tl.tp_attn_fwd_workspace_bytes(1, 4096, 4, 2)
    assert need == tl.attn_fwd_workspace_bytes(1, 4096, 2) > 0
    fw = [None, 1, 4096, 512, 4, 128, 2, 1, 0.1, P, P, P, P, P, P, P]
    assert f(*fw, None, 0) == E_NULL
    assert f(*fw, P, need - 1) == E_WS
    # causal dQ partials: none up to 1664 tokens (one chunk of 26 key blocks); at 32K tokens at most
    # 8 key chunks per query block
    assert tl.attn_bwd_workspace_bytes(1, 1664, 10) == 2 * 1664 * 10 * 4
    assert tl.attn_bwd_workspace_bytes(1, 1728, 10) > 2 * 1728 * 10 * 4
    assert tl.attn_bwd_workspace_bytes(1, 32768, 10) <= 2 * 32768 * 10 * 4 + 256 * 10 * 4.5 * 65536
    assert tl.lib.tp_attn_bwd_workspace_bytes(1, 8, 4, 128, 3) == 0
    assert tl.lib.tp_attn_bwd_workspace_bytes(1, 8, 4, 128, 2) >= 8 * 256 * 2 * 4
    b = tl.lib.tp_attn_bwd
    args = [None, 1, 8, 512, 4, 128, 2, 1, 0.1, P, P, P, P, P, P, P, P, P, P]
    assert b(*args, P, 16) == E_WS
    assert b(*args, None, 1 << 20) == E_NULL
    assert b(*args, P + 16, 1 << 20) == E_ALIGN
