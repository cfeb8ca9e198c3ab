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


def test_cpu_baseline_reports_its_split_and_host():
    """The oracle's CPU time on a small MLP shard: the forward and backward
    seconds of the measured calls add up to the reported time, and the BLAS
    library and host memory are named."""
    wl = synth.Workload("t", 3, "bf16", T=64, h=64, F=256, tp=2, x_std=1.0, w_std=0.05, b_std=0.1, dz_std=1.0)
    out = bench.cpu_baseline(wl, synth.mlp_inputs(wl), 0.3)
    assert out["kind"] == "oracle" and out["value"] > 0
    assert abs(out["fwd_seconds"] + out["bwd_seconds"] - out["seconds"]) <= 0.01 + 0.05 * out["seconds"]
    assert out["fwd_seconds"] > 0 and out["bwd_seconds"] > 0
    assert out["host_ram_gb"] is None or out["host_ram_gb"] > 0
    assert "blas" in out


def test_memory_bound_role_bytes():
    """The partial sum of this GPU's T/tp rows reads tp partials and writes one
    sum (all T rows in the forward-only step); the db1 reduction reads one row
    of column sums per tile row of the dH product."""
    wl = synth.WORKLOADS["llama7b_bf16"]
    assert bench.hbm_role_bytes(wl, "partial_sum") == (8 + 1) * (8192 // 8) * 4096 * 4
    tiny = synth.WORKLOADS["tiny_f32"]
    assert bench.hbm_role_bytes(tiny, "partial_sum") == 3 * 128 * 256 * 4
    g = synth.WORKLOADS["gpt2m_bf16"]
    assert bench.hbm_role_bytes(g, "colsum", 128) == (4096 // 128 * 2048 + 2048) * 4
    assert bench.hbm_role_bytes(g, "gemm.mlp_fwd1") is None
    assert bench.tile_rows("gemm_w4_kernel<128,128,1,1,2>") == 128 and bench.tile_rows("partial_sum_kernel<4>") is None
