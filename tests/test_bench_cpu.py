"""bench.py's host-side accounting, on the CPU: every workload's flop and byte
counts are defined for every kernel role the library reports, and the
multi-GPU request is refused with a message."""
import subprocess
import sys

import pytest

import bench
import synth

ROLES = ["gemm.mlp_fwd1", "gemm.mlp_fwd2", "gemm.mlp_dgrad_act", "gemm.mlp_wgrad2", "gemm.mlp_wgrad1",
         "gemm.mlp_wgrad2+gemm.mlp_wgrad1", "gemm.mlp_wgrad2+gemm.mlp_wgrad1+gemm.mlp_dgrad1", "gemm.mlp_dgrad1", "gemm.swiglu_fwd1", "gemm.swiglu_fwd2", "gemm.swiglu_dgrad_act", "gemm.swiglu_wgrad2",
         "gemm.swiglu_wgrad1", "gemm.swiglu_dgrad1", "gemm.swiglu_wgrad2+gemm.swiglu_dgrad_act", "partial_sum", "colsum", "layernorm_fwd", "layernorm_bwd",
         "layernorm_param_grad", "sp_sum_dropout_residual", "sp_dropout_bwd", "gemm.attn_qkv", "attn_fwd",
         "gemm.attn_out", "gemm.attn_out_dgrad", "gemm.attn_out_wgrad", "attn_bwd_dot", "attn_bwd_dkdv",
         "attn_bwd_dq", "gemm.attn_qkv_wgrad", "gemm.attn_qkv_dgrad"]
BENCH_WORKLOADS = ["llama7b_bf16", "qwen3_swiglu_bf16", "llama7b_sp_bf16", "attn_proj_bf16"]


@pytest.mark.parametrize("name", BENCH_WORKLOADS)
def test_accounting_defined_for_every_role(name):
    wl = synth.WORKLOADS[name]
    total = bench.step_flops(wl)
    assert total > 0
    gemm_sum = 0.0
    for role in ROLES:
        f = bench.role_flops(wl, role)
        assert f >= 0.0
        if role.startswith("gemm.") and "+" not in role:   # joined launches repeat their parts
            gemm_sum += f
        b = bench.algorithmic_bytes(wl, role)
        assert b is None or b > 0
    assert gemm_sum <= total + 1.0
    assert isinstance(bench.workload_text(wl), str) and name in bench.workload_text(wl)


def test_mlp_step_is_six_equal_gemms():
    wl = synth.WORKLOADS["llama7b_bf16"]
    u = 2.0 * wl.T * wl.h * wl.Fs
    assert bench.step_flops(wl) == 6 * u
    assert bench.role_flops(wl, "gemm.mlp_wgrad2+gemm.mlp_wgrad1") == 2 * u   # the paired weight gradients
    assert bench.role_flops(wl, "gemm.mlp_wgrad2+gemm.mlp_wgrad1+gemm.mlp_dgrad1") == 3 * u   # joined by dX


def test_attention_block_counts():
    wl = synth.WORKLOADS["attn_proj_bf16"]
    T, d, hs = wl.T, wl.head_dim, wl.heads // wl.tp
    pm = 2.0 * T * (T + 1) / 2 * d * hs
    w = hs * d
    assert bench.step_flops(wl) == pytest.approx(12 * 2.0 * T * wl.h * w + 7 * pm)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr) or "1 GPU" in (r.stdout + r.stderr)


def test_joined_roles_sum_their_parts():
    wl = synth.WORKLOADS["qwen3_swiglu_bf16"]
    j = "gemm.swiglu_wgrad2+gemm.swiglu_dgrad_act"
    assert bench.role_flops(wl, j) == bench.role_flops(wl, "gemm.swiglu_wgrad2") + \
        bench.role_flops(wl, "gemm.swiglu_dgrad_act")
    assert bench.algorithmic_bytes(wl, j) == bench.algorithmic_bytes(wl, "gemm.swiglu_wgrad2") + \
        bench.algorithmic_bytes(wl, "gemm.swiglu_dgrad_act")
