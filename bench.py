#!/usr/bin/env python3
"""Benchmark of one GPU's share of the tensor-parallel MLP block.

One step = the whole per-GPU hot path for shard 0 of the Llama-7B-scale MLP
(T=8192 tokens, h=4096, F=16384, tp=8, bf16 storage, fp32 accumulate):
  tp_mlp_fwd        GEMM1 + bias/GeLU epilogue, GEMM2 -> fp32 partial Z_0
  shard_partial_sum this GPU's 1/tp share of the Z all-reduce arithmetic
                    (rows [0, T/tp) of all tp partials; the other shards'
                    partials were computed once during set-up)
  tp_mlp_bwd        dH (GEMM + GeLU'), dW2, dW1, dX_0 partial
  shard_partial_sum the same share of the dX all-reduce
Inputs sit in HBM before the timed region starts.  `value` is the GEMM work
(6 products of 2*T*h*F/tp flops) per second over the timed steps.

Prints ONE JSON line.  `--gpus N` with N > 1 is refused: the library runs
one GPU's shard, and the shards of the other GPUs are simulated in turn on
that GPU.

Profiling helpers (used with rocprofv3, see the profiles/ summaries):
  --profile-pass OUT.json   a plain copy of known size, then one step; writes
                            the step's kernel roles and symbols in launch order
  --summarize-profile DIR   turn rocprofv3 output under DIR into the text
                            summaries and traffic table under profiles/
Machine probes (libtpmlp_probe.so, no MLP work):
  --probe                   per-CU load-path rate for the GEMM tiles' operand
                            patterns and LDS fragment-read rates, the bounds
                            the GEMM design is measured against
  --power                   board power (hwmon) against its cap while the
                            workload's step runs back to back for 3 s
"""
from __future__ import annotations

import argparse
import csv
import gc
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CUs x 4096 flop/clk x 2.4 GHz)
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 (matrix and vector)
PEAK_SCLK_GHZ = 2.4         # the engine clock that peak assumes
PEAK_HBM_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")


def traffic_path(workload: str) -> str:
    return os.path.join(PROFILES, f"{workload}_traffic.json")


def mfma_path(workload: str) -> str:
    return os.path.join(PROFILES, f"{workload}_mfma.json")

XCDS = 8                    # MI355X: 8 accelerator dies, GRBM_GUI_ACTIVE sums their busy cycles
COLD_FLUSH_BYTES = 512 << 20   # written between steps by the cold-cache timing

CALIB_BYTES = 256 << 20     # the plain copy used to scale the HBM byte counters

# Default warm-up.  After the GPU has idled, the first tens of milliseconds of
# steps run slower while its clocks ramp up: measured on the Llama-7B shard,
# 50 steps timed after 10 warm-up steps took 0.676 ms each, after 50 to 400
# warm-up steps 0.651-0.657 ms.  So by default the warm-up runs at least this
# many steps and this long; `--warmup W` runs exactly W steps instead.
WARMUP_MIN_STEPS = 100
WARMUP_MIN_S = 0.15
WARMUP_PROFILED = 10        # the last warm-up steps, timed per kernel to find the dominant one


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default: at least %d steps and %.0f ms, until the clocks settle)"
                    % (WARMUP_MIN_STEPS, WARMUP_MIN_S * 1e3))
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache timing")
    ap.add_argument("--workload", default="llama7b_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle CPU time for the baseline")
    ap.add_argument("--breakdown", action="store_true", help="also print per-kernel timings to stderr")
    ap.add_argument("--vendor", action="store_true",
                    help="also time the step's six products through torch.matmul (hipBLASLt) as a yardstick")
    ap.add_argument("--profile-pass", metavar="OUT_JSON", default=None)
    ap.add_argument("--summarize-profile", metavar="DIR", default=None)
    ap.add_argument("--probe", action="store_true", help="run the machine probes and exit")
    ap.add_argument("--power", action="store_true",
                    help="sample the board power (hwmon) while the workload's step runs back to back, and exit")
    return ap.parse_args()


# Kernel sources that cannot affect a workload's kernels (they hold other
# kernels only), left out of its fingerprint.  probes.hip builds a library of
# its own and never affects any.
_UNRELATED_SOURCES = {"mlp": {"attn.hpp", "sp.hpp", "swiglu.hpp", "epilogue.hpp"},
                      "swiglu": {"attn.hpp", "sp.hpp", "epilogue.hpp"},
                      "sp_mlp": {"attn.hpp", "swiglu.hpp", "epilogue.hpp"},
                      "proj": {"sp.hpp", "swiglu.hpp", "epilogue.hpp"}}
_NEVER_IN_FINGERPRINT = {"probes.hip"}


def kernel_fingerprint(kind: str) -> str:
    """Hash of the kernel sources a workload's kernels are built from: counters
    taken on other sources are stale."""
    h = hashlib.sha256()
    skip = _UNRELATED_SOURCES.get(kind, set()) | _NEVER_IN_FINGERPRINT
    for f in sorted(glob.glob(os.path.join(ROOT, "linear_layers_amd", "csrc", "*"))):
        if os.path.basename(f) in skip:
            continue
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode() + fh.read())
    return h.hexdigest()[:16]


def canon(name: str) -> str:
    """Kernel name as the library reports it, from a demangled rocprofv3 name."""
    n = name.replace("void tpmlp::", "").replace("tpmlp::", "")
    n = re.sub(r"\(.*\)$", "", n).replace(" ", "").replace("true", "1").replace("false", "0")
    return re.sub(r"\bfloat\b", "f32", n)


# GEMMs of one shard's step, in units of 2*T*h*(F/tp) flops: the plain MLP
# has six equal ones; in the gated MLP the joined gate/up layer is twice as
# wide, so its forward product, its weight gradient and the input gradient
# through it count twice.  A launch that runs several products reports their
# role names joined by '+' (e.g. gemm.mlp_wgrad2+gemm.mlp_wgrad1+gemm.mlp_dgrad1)
# and counts as the sum of its parts.
ROLE_UNITS = {
    "sp_mlp": {"gemm.mlp_fwd1": 1, "gemm.mlp_fwd2": 1, "gemm.mlp_dgrad_act": 1, "gemm.mlp_wgrad2": 1,
               "gemm.mlp_wgrad1": 1, "gemm.mlp_dgrad1": 1},
    "mlp": {"gemm.mlp_fwd1": 1, "gemm.mlp_fwd2": 1, "gemm.mlp_dgrad_act": 1, "gemm.mlp_wgrad2": 1,
            "gemm.mlp_wgrad1": 1, "gemm.mlp_dgrad1": 1},
    "swiglu": {"gemm.swiglu_fwd1": 2, "gemm.swiglu_fwd2": 1, "gemm.swiglu_dgrad_act": 1, "gemm.swiglu_wgrad2": 1,
               "gemm.swiglu_wgrad1": 2, "gemm.swiglu_dgrad1": 2},
}


def attn_product_flops(wl, T=None):
    """Flops of one score-sized product (Q K^T, P V, ...) over the shard's heads:
    2 * d per unmasked (query, key) pair, causal, one sequence of T tokens."""
    T = wl.T if T is None else T
    return 2.0 * (T * (T + 1) / 2) * wl.head_dim * (wl.heads // wl.tp)


def proj_role_flops(wl, T=None):
    """The head-sharded attention block's kernels.  Each attention kernel counts
    the products its own outputs need: the forward 2 (S, PV); the dK/dV kernel
    4 (S and dP recomputed, dV, dK); the dQ kernel 3 (S, dP, dQ)."""
    T = wl.T if T is None else T
    w = wl.heads // wl.tp * wl.head_dim
    pm = attn_product_flops(wl, T)
    g = 2.0 * T * wl.h * w
    return {"gemm.attn_qkv": 3 * g, "attn_fwd": 2 * pm, "gemm.attn_out": g, "gemm.attn_out_dgrad": g,
            "gemm.attn_out_wgrad": g, "attn_bwd_dkdv": 4 * pm, "attn_bwd_dq": 3 * pm, "gemm.attn_qkv_wgrad": 3 * g,
            "gemm.attn_qkv_dgrad": 3 * g}


# Launches that run several of a step's products together (each part also has
# a role of its own).
def role_flops(wl, role):
    if "+" in role:      # products joined in one launch: the sum of their parts
        return sum(role_flops(wl, r) for r in role.split("+"))
    if wl.kind == "proj":
        return proj_role_flops(wl).get(role, 0.0)
    return ROLE_UNITS[wl.kind].get(role, 0) * 2.0 * wl.T * wl.h * wl.Fs


def step_flops(wl, T=None):
    """Algorithmic flops of one step.  The attention backward counts 5 products
    (S, dP, dV, dK, dQ), whatever the kernels recompute."""
    if wl.kind == "proj":
        r = proj_role_flops(wl, T)
        return sum(v for k, v in r.items() if k.startswith("gemm.")) + 7 * attn_product_flops(wl, T)
    T = wl.T if T is None else T
    if wl.kind == "mlp" and wl.dz_std is None:      # forward only, every shard on this GPU
        return wl.tp * 2 * 2.0 * T * wl.h * wl.Fs
    units = sum(ROLE_UNITS[wl.kind].values())
    return units * 2.0 * T * wl.h * wl.Fs


def algorithmic_bytes(wl, role):
    """The GEMM's operands and outputs, each read or written once (for products
    joined in one launch, role names joined by '+', the sum of their parts)."""
    if "+" in role:
        parts = [algorithmic_bytes(wl, r) for r in role.split("+")]
        return None if any(p is None for p in parts) else sum(parts)
    T, h, Fs = wl.T, wl.h, wl.Fs
    return {"gemm.mlp_fwd1": T * h * 2 + h * Fs * 2 + 2 * T * Fs * 2,
            "gemm.mlp_fwd2": T * Fs * 2 + Fs * h * 2 + T * h * 4,
            "gemm.mlp_dgrad_act": T * h * 2 + Fs * h * 2 + T * Fs * 2 + T * Fs * 2,
            "gemm.mlp_wgrad2": T * Fs * 2 + T * h * 2 + Fs * h * 4,
            "gemm.mlp_wgrad1": T * h * 2 + T * Fs * 2 + h * Fs * 4,
            "gemm.mlp_dgrad1": T * Fs * 2 + h * Fs * 2 + T * h * 4,
            "gemm.swiglu_fwd1": T * h * 2 + h * 2 * Fs * 2 + T * Fs * 2 + T * 2 * Fs * 2,
            "gemm.swiglu_fwd2": T * Fs * 2 + Fs * h * 2 + T * h * 4,
            "gemm.swiglu_dgrad_act": T * h * 2 + Fs * h * 2 + T * 2 * Fs * 2 + T * 2 * Fs * 2,
            "gemm.swiglu_wgrad2": T * Fs * 2 + T * h * 2 + Fs * h * 4,
            "gemm.swiglu_wgrad1": T * h * 2 + T * 2 * Fs * 2 + h * 2 * Fs * 4,
            "gemm.swiglu_dgrad1": T * 2 * Fs * 2 + h * 2 * Fs * 2 + T * h * 4}.get(role) if wl.kind != "proj" \
        else _proj_bytes(wl, role)


def hbm_role_bytes(wl, role, colsum_bm=256):
    """Algorithmic HBM bytes of one launch of a memory-bound role of the step:
    the partial sum reads the tp partials of its rows and writes their sum
    (rows [0, T/tp): this GPU's share, or all T rows in the forward-only
    step); the db1 reduction reads one fp32 row of column sums per tile row of
    the dH product (colsum_bm rows a tile) and writes db1.  None for others."""
    T, h, Fs, tp = wl.T, wl.h, wl.Fs, wl.tp
    if role == "partial_sum":
        rows = T if (wl.kind == "mlp" and wl.dz_std is None) else T // tp
        return (tp + 1) * rows * h * 4
    if role == "colsum":
        return (((T + colsum_bm - 1) // colsum_bm) * Fs + Fs) * 4
    return None


def tile_rows(sym):
    """BM of a GEMM kernel symbol such as gemm_w4_kernel<128,128,1,1,2> (None if not one)."""
    m = re.search(r"<(\d+),", sym or "")
    return int(m.group(1)) if m else None


def _proj_bytes(wl, role):
    T, h = wl.T, wl.h
    hs = wl.heads // wl.tp
    w = hs * wl.head_dim
    return {"gemm.attn_qkv": T * h * 2 + h * 3 * w * 2 + T * 3 * w * 2,
            "gemm.attn_out": T * w * 2 + w * h * 2 + T * h * 4,
            "gemm.attn_out_dgrad": T * h * 2 + w * h * 2 + T * w * 2,
            "gemm.attn_out_wgrad": T * w * 2 + T * h * 2 + w * h * 4,
            "gemm.attn_qkv_wgrad": T * h * 2 + T * 3 * w * 2 + h * 3 * w * 4,
            "gemm.attn_qkv_dgrad": T * 3 * w * 2 + h * 3 * w * 2 + T * h * 4,
            # Q, K, V in, O out, lse out
            "attn_fwd": T * 3 * w * 2 + T * w * 2 + T * hs * 4,
            # Q, K, V, dO, lse, D in; dK, dV out
            "attn_bwd_dkdv": T * 4 * w * 2 + 2 * T * hs * 4 + T * 2 * w * 2,
            # Q, K, V, dO, lse, D in; dQ out
            "attn_bwd_dq": T * 4 * w * 2 + 2 * T * hs * 4 + T * w * 2}.get(role)


def _time_sample(run, probe, T, target_s):
    """Rows of the sample and its oracle time: grow the row count toward
    target_s; when the whole workload takes less than that, repeat it."""
    dt = run(probe)
    rows = int(min(T, max(probe, probe * target_s / max(dt, 1e-3))))
    rows = max(probe, rows - rows % 8) if rows < T else T
    dt, reps = run(rows), 1
    if rows == T and dt < target_s:
        more = min(100000, int(target_s / max(dt, 1e-6)))
        for _ in range(more - 1):
            dt += run(rows)
        reps = max(more, 1)
    return rows, reps, dt


def _blas_info():
    """(BLAS threads, 'library version') of numpy's BLAS as threadpoolctl sees it."""
    try:
        from threadpoolctl import threadpool_info
        libs = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        threads = max([p.get("num_threads", 1) for p in libs] or [1])
        blas = ", ".join(f"{p.get('internal_api')} {p.get('version')}" for p in libs) or None
        return threads, blas
    except Exception:  # noqa: BLE001
        return os.cpu_count() or 1, None


def _host_ram_gb():
    try:
        with open("/proc/meminfo") as f:
            kib = int(next(ln for ln in f if ln.startswith("MemTotal")).split()[1])
        return round(kib / 2**20, 1)
    except (OSError, StopIteration, ValueError):
        return None


def cpu_baseline(wl, raw, target_s: float):
    """Time the float64 oracle (fwd + bwd of shard 0) on a sample of rows."""
    import synth
    from oracle import ref
    from oracle import swiglu as sw
    from oracle import sp as osp
    threads, blas = _blas_info()
    Fs = wl.Fs
    if wl.kind == "proj":
        return _cpu_baseline_proj(wl, raw, target_s, threads, blas)
    if wl.kind == "swiglu":
        W_gu = sw.pack_shard(synth.to_f64(raw["W_gate"], wl.dtype), synth.to_f64(raw["W_up"], wl.dtype), wl.tp, 0)
        Wd = synth.to_f64(raw["W_down"][:Fs], wl.dtype)
    else:
        W1 = synth.to_f64(raw["W1"][:, :Fs], wl.dtype)
        W2 = synth.to_f64(raw["W2"][:Fs], wl.dtype)
        b1 = synth.to_f64(raw["b1"][:Fs], wl.dtype) if "b1" in raw else None

    fwd_only = "dZ" not in raw
    calls = []   # (forward seconds, backward seconds) of every run() call

    def run_fwd(rows):
        # every shard's forward, then the sum of the partials (the forward-only workload's step)
        X = synth.to_f64(raw["X"][:rows], wl.dtype)
        t0 = time.perf_counter()
        parts = []
        for i in range(wl.tp):
            W1i = synth.to_f64(raw["W1"][:, i * Fs:(i + 1) * Fs], wl.dtype)
            W2i = synth.to_f64(raw["W2"][i * Fs:(i + 1) * Fs], wl.dtype)
            H = ref.matmul(X, W1i)
            if "b1" in raw:
                H = H + synth.to_f64(raw["b1"][i * Fs:(i + 1) * Fs], wl.dtype)[None, :]
            parts.append(ref.matmul(ref.gelu_tanh(H), W2i))
        ref.shard_partial_sum(parts)
        dt = time.perf_counter() - t0
        calls.append((dt, 0.0))
        return dt

    def run(rows):
        if fwd_only:
            return run_fwd(rows)
        X = synth.to_f64(raw["X"][:rows], wl.dtype)
        dZ = synth.to_f64(raw["dZ"][:rows], wl.dtype)
        t0 = time.perf_counter()
        if wl.kind == "sp_mlp":
            ln = osp.layernorm_fwd(X, raw["ln_gamma"], raw["ln_beta"])
            X = ln["Y"]
        if wl.kind == "swiglu":
            G, U = sw.deinterleave(ref.matmul(X, W_gu))
            A = sw.silu(G) * U
            out = [ref.matmul(A, Wd)]
            t_fwd = time.perf_counter()
            dA = ref.matmul(dZ, Wd.T)
            dGU = sw.interleave(dA * U * sw.silu_grad(G), dA * sw.silu(G))
            out += [ref.matmul(A.T, dZ), ref.matmul(X.T, dGU), ref.matmul(dGU, W_gu.T)]
        else:
            H = ref.matmul(X, W1) + (b1[None, :] if b1 is not None else 0.0)
            A = ref.gelu_tanh(H)
            out = [ref.matmul(A, W2)]
            t_fwd = time.perf_counter()
            dA = ref.matmul(dZ, W2.T)
            dH = dA * ref.gelu_tanh_grad(H)
            out += [ref.matmul(A.T, dZ), ref.matmul(X.T, dH), ref.matmul(dH, W1.T)]
        if wl.kind == "sp_mlp":
            Xr = synth.to_f64(raw["X"][:rows], wl.dtype)
            out.append(osp.partial_sum_dropout_residual([out[0]], Xr, synth.SP_DROPOUT_P, wl.seed, 0))
            out.append(osp.dropout_bwd(dZ, synth.SP_DROPOUT_P, wl.seed, 0))
            out.append(osp.layernorm_bwd(Xr, raw["ln_gamma"], out[3])["dX"])
        del out
        t1 = time.perf_counter()
        calls.append((t_fwd - t0, t1 - t_fwd))
        return t1 - t0

    rows, reps, dt = _time_sample(run, min(wl.T, 256), wl.T, target_s)
    flops = step_flops(wl) * rows / wl.T * reps
    measured = calls[-reps:]   # the calls dt covers (the probe call comes first)
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "fwd_seconds": round(sum(c[0] for c in measured), 6), "bwd_seconds": round(sum(c[1] for c in measured), 6),
            "blas": blas, "host_ram_gb": _host_ram_gb(),
            "sample": (f"float64 numpy oracle, all {wl.tp} shards' forward and their partial sum" if fwd_only else
                       "float64 numpy oracle, shard 0 fwd+bwd") +
                      f" on the first {rows} of {wl.T} token rows (h={wl.h}, F/tp={Fs})" +
                      (f", {reps} repetitions" if reps > 1 else "") +
                      f"; {dt:.2f} s for {flops / 1e9:.1f} GFLOP",
            "seconds": round(dt, 3), "host_cpus": os.cpu_count(),
            "affinity": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


def _cpu_baseline_proj(wl, raw, target_s, threads, blas=None):
    """The attention block oracle (shard 0 fwd+bwd) on a causal sequence made of
    the first rows tokens; the flops use the same count at that length."""
    import synth
    from oracle import attn as oat
    W = {n: synth.to_f64(raw[n], wl.dtype) for n in ("Wq", "Wk", "Wv", "Wo")}

    def run(rows):
        X = synth.to_f64(raw["X"][:rows], wl.dtype)
        dZ = synth.to_f64(raw["dOut"][:rows], wl.dtype)
        t0 = time.perf_counter()
        oat.tp_attn_block_bwd_shard(X, W["Wq"], W["Wk"], W["Wv"], W["Wo"], dZ, 1, rows, wl.heads, wl.head_dim,
                                    wl.tp, 0, True, wl.head_dim ** -0.5)
        return time.perf_counter() - t0

    rows, reps, dt = _time_sample(run, min(wl.T, 128), wl.T, target_s)
    flops = step_flops(wl, rows) * reps
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"float64 numpy oracle, shard 0 fwd+bwd of the attention block on a causal sequence of the "
                      f"first {rows} of {wl.T} tokens (h={wl.h}, {wl.heads // wl.tp} heads)" +
                      (f", {reps} repetitions" if reps > 1 else "") + f"; {dt:.2f} s for "
                      f"{flops / 1e9:.1f} GFLOP",
            "fwd_seconds": None, "bwd_seconds": None, "blas": blas, "host_ram_gb": _host_ram_gb(),
            "seconds": round(dt, 3), "host_cpus": os.cpu_count(),
            "affinity": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


class Step:
    """Device buffers of the workload and the step's library calls."""

    def __init__(self, wl, raw, tl, torch):
        self.wl, self.tl = wl, tl
        T, h, F, tp, Fs = wl.T, wl.h, wl.F, wl.tp, wl.Fs
        dev = torch.device("cuda:0")

        f32 = wl.dtype == "f32"

        def up(a):
            if f32:
                return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

        self.X, self.dZ = up(raw["X"]), up(raw["dZ"])
        # Each shard's weights packed as its own rank would hold them.
        self.W1s = [up(np.ascontiguousarray(raw["W1"][:, i * Fs:(i + 1) * Fs])) for i in range(tp)]
        self.W2s = [up(raw["W2"][i * Fs:(i + 1) * Fs]) for i in range(tp)]
        self.b1s = [None if "b1" not in raw else up(raw["b1"][i * Fs:(i + 1) * Fs]) for i in range(tp)]
        bf = torch.float32 if f32 else torch.bfloat16
        self.A = torch.empty((T, Fs), dtype=bf, device=dev)
        self.H = torch.empty((T, Fs), dtype=bf, device=dev)
        self.Zp = torch.empty((tp, T, h), dtype=torch.float32, device=dev)
        self.dXp = torch.empty((tp, T, h), dtype=torch.float32, device=dev)
        self.rows = T // tp
        self.Zsum = torch.empty((self.rows, h), dtype=torch.float32, device=dev)
        self.dXsum = torch.empty((self.rows, h), dtype=torch.float32, device=dev)
        self.dW1 = torch.empty((h, Fs), dtype=torch.float32, device=dev)
        self.dW2 = torch.empty((Fs, h), dtype=torch.float32, device=dev)
        self.db1 = torch.empty((Fs,), dtype=torch.float32, device=dev) if "b1" in raw else None
        self.ws = torch.empty(max(1, tl.tpmlp_bwd_workspace_bytes(tl.F32 if f32 else tl.BF16, T, h, F, tp)),
                              dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.current_stream(dev)
        for i in range(1, tp):  # the other shards' partials, computed once
            self.shard(i)

    def shard(self, i):
        tl, s = self.tl, self
        tl.tp_mlp_fwd(s.X, s.W1s[i], s.b1s[i], s.W2s[i], s.wl.tp, s.A, s.Zp[i], H_save=s.H, stream=s.stream)
        tl.tp_mlp_bwd(s.X, s.W1s[i], s.W2s[i], s.H, s.A, s.dZ, s.wl.tp, s.dXp[i], s.dW1, s.dW2, db1_shard=s.db1,
                      workspace=s.ws, stream=s.stream)

    def parts(self):
        """Shard 0's forward call and backward call alone, with their GEMM flops."""
        tl, s, u = self.tl, self, 2.0 * self.wl.T * self.wl.h * self.wl.Fs

        def fwd():
            tl.tp_mlp_fwd(s.X, s.W1s[0], s.b1s[0], s.W2s[0], s.wl.tp, s.A, s.Zp[0], H_save=s.H, stream=s.stream)

        def bwd():
            tl.tp_mlp_bwd(s.X, s.W1s[0], s.W2s[0], s.H, s.A, s.dZ, s.wl.tp, s.dXp[0], s.dW1, s.dW2, db1_shard=s.db1,
                          workspace=s.ws, stream=s.stream)
        return {"tp_mlp_fwd": (fwd, 2 * u), "tp_mlp_bwd": (bwd, 4 * u)}

    def __call__(self):
        tl, s = self.tl, self
        tl.tp_mlp_fwd(s.X, s.W1s[0], s.b1s[0], s.W2s[0], s.wl.tp, s.A, s.Zp[0], H_save=s.H, stream=s.stream)
        tl.shard_partial_sum(s.Zp[:, :s.rows], s.Zsum, stream=s.stream)
        tl.tp_mlp_bwd(s.X, s.W1s[0], s.W2s[0], s.H, s.A, s.dZ, s.wl.tp, s.dXp[0], s.dW1, s.dW2, db1_shard=s.db1,
                      workspace=s.ws, stream=s.stream)
        tl.shard_partial_sum(s.dXp[:, :s.rows], s.dXsum, stream=s.stream)


class FwdStep:
    """A forward-only MLP workload (the tiny fp32 one): every shard's forward
    on this GPU in turn, then the sum of all their partials."""

    def __init__(self, wl, raw, tl, torch):
        self.wl, self.tl = wl, tl
        T, h, tp, Fs = wl.T, wl.h, wl.tp, wl.Fs
        dev = torch.device("cuda:0")
        f32 = wl.dtype == "f32"
        dt = torch.float32 if f32 else torch.bfloat16

        def up(a):
            if f32:
                return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

        self.X = up(raw["X"])
        self.W1s = [up(np.ascontiguousarray(raw["W1"][:, i * Fs:(i + 1) * Fs])) for i in range(tp)]
        self.W2s = [up(raw["W2"][i * Fs:(i + 1) * Fs]) for i in range(tp)]
        self.b1s = [None if "b1" not in raw else up(raw["b1"][i * Fs:(i + 1) * Fs]) for i in range(tp)]
        self.A = torch.empty((T, Fs), dtype=dt, device=dev)
        self.Zp = torch.empty((tp, T, h), dtype=torch.float32, device=dev)
        self.Z = torch.empty((T, h), dtype=torch.float32, device=dev)
        self.rows = T
        self.stream = torch.cuda.current_stream(dev)

    def __call__(self):
        tl, s = self.tl, self
        for i in range(s.wl.tp):
            tl.tp_mlp_fwd(s.X, s.W1s[i], s.b1s[i], s.W2s[i], s.wl.tp, s.A, s.Zp[i], stream=s.stream)
        tl.shard_partial_sum(s.Zp, s.Z, stream=s.stream)


class SwiGLUStep:
    """The gated MLP's device buffers and step: shard 0 fwd, its share of the
    partial sum of down, shard 0 bwd, its share of the partial sum of dX."""

    def __init__(self, wl, raw, tl, torch):
        self.wl, self.tl = wl, tl
        T, h, F, tp, Fs = wl.T, wl.h, wl.F, wl.tp, wl.Fs
        dev = torch.device("cuda:0")
        bf = torch.bfloat16

        def up(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(bf).to(dev)

        self.stream = torch.cuda.current_stream(dev)
        self.X, self.dZ = up(raw["X"]), up(raw["dZ"])
        Wg, Wu = up(raw["W_gate"]), up(raw["W_up"])
        self.Wgus = []
        for i in range(tp):  # each shard's joined weight as its own rank would hold it
            w = torch.empty((h, 2 * Fs), dtype=bf, device=dev)
            tl.swiglu_pack_shard(Wg, Wu, tp, i, w, stream=self.stream)
            self.Wgus.append(w)
        del Wg, Wu
        self.Wds = [up(raw["W_down"][i * Fs:(i + 1) * Fs]) for i in range(tp)]
        self.A = torch.empty((T, Fs), dtype=bf, device=dev)
        self.GU = torch.empty((T, 2 * Fs), dtype=bf, device=dev)
        self.Zp = torch.empty((tp, T, h), dtype=torch.float32, device=dev)
        self.dXp = torch.empty((tp, T, h), dtype=torch.float32, device=dev)
        self.rows = T // tp
        self.Zsum = torch.empty((self.rows, h), dtype=torch.float32, device=dev)
        self.dXsum = torch.empty((self.rows, h), dtype=torch.float32, device=dev)
        self.dWgu = torch.empty((h, 2 * Fs), dtype=torch.float32, device=dev)
        self.dWd = torch.empty((Fs, h), dtype=torch.float32, device=dev)
        self.ws = torch.empty(tl.tp_swiglu_bwd_workspace_bytes(tl.BF16, T, h, F, tp), dtype=torch.uint8, device=dev)
        for i in range(1, tp):
            self.fwd(i)
            self.bwd(i)

    def fwd(self, i):
        s = self
        s.tl.tp_swiglu_fwd(s.X, s.Wgus[i], s.Wds[i], s.wl.tp, s.A, s.Zp[i], GU_save=s.GU, stream=s.stream)

    def bwd(self, i):
        s = self
        s.tl.tp_swiglu_bwd(s.X, s.Wgus[i], s.Wds[i], s.GU, s.A, s.dZ, s.wl.tp, s.dXp[i], s.dWgu, s.dWd,
                           workspace=s.ws, stream=s.stream)

    def parts(self):
        u = 2.0 * self.wl.T * self.wl.h * self.wl.Fs
        return {"tp_swiglu_fwd": (lambda: self.fwd(0), 3 * u), "tp_swiglu_bwd": (lambda: self.bwd(0), 6 * u)}

    def __call__(self):
        s = self
        s.fwd(0)
        s.tl.shard_partial_sum(s.Zp[:, :s.rows], s.Zsum, stream=s.stream)
        s.bwd(0)
        s.tl.shard_partial_sum(s.dXp[:, :s.rows], s.dXsum, stream=s.stream)


class SPStep:
    """The MLP inside the sequence-parallel region, rank 0's step: LayerNorm of
    its T/tp rows into its block of the gathered input (the other ranks' blocks
    are filled once in set-up), the shard's MLP forward, its reduce-scatter
    rows fused with dropout and the residual; backward: dropout' of its rows
    into its block of the gathered gradient, the shard's MLP backward, the
    reduce-scatter rows of dX, LayerNorm backward plus the residual path."""

    def __init__(self, wl, raw, tl, torch):
        import synth
        self.wl, self.tl = wl, tl
        T, h, F, tp, Fs = wl.T, wl.h, wl.F, wl.tp, wl.Fs
        dev = torch.device("cuda:0")
        bf = torch.bfloat16

        def up(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(bf).to(dev)

        self.stream = torch.cuda.current_stream(dev)
        self.p, self.seed = synth.SP_DROPOUT_P, wl.seed
        self.rows = T // tp
        self.X, self.dOut = up(raw["X"]), up(raw["dZ"])
        self.gamma = torch.from_numpy(raw["ln_gamma"]).to(dev)
        self.beta = torch.from_numpy(raw["ln_beta"]).to(dev)
        self.W1s = [up(np.ascontiguousarray(raw["W1"][:, i * Fs:(i + 1) * Fs])) for i in range(tp)]
        self.W2s = [up(raw["W2"][i * Fs:(i + 1) * Fs]) for i in range(tp)]
        self.Y = torch.empty((T, h), dtype=bf, device=dev)          # gathered LayerNorm output
        self.dZ = torch.empty((T, h), dtype=bf, device=dev)         # gathered upstream gradient
        self.mean = torch.empty((T,), dtype=torch.float32, device=dev)
        self.rstd = torch.empty((T,), dtype=torch.float32, device=dev)
        self.A = torch.empty((T, Fs), dtype=bf, device=dev)
        self.H = torch.empty((T, Fs), dtype=bf, device=dev)
        self.Zp = torch.empty((tp, T, h), dtype=torch.float32, device=dev)
        self.dXp = torch.empty((tp, T, h), dtype=torch.float32, device=dev)
        self.out = torch.empty((self.rows, h), dtype=bf, device=dev)
        self.dYln = torch.empty((self.rows, h), dtype=torch.float32, device=dev)
        self.dXseq = torch.empty((self.rows, h), dtype=torch.float32, device=dev)
        self.dgamma = torch.empty((h,), dtype=torch.float32, device=dev)
        self.dbeta = torch.empty((h,), dtype=torch.float32, device=dev)
        self.dW1 = torch.empty((h, Fs), dtype=torch.float32, device=dev)
        self.dW2 = torch.empty((Fs, h), dtype=torch.float32, device=dev)
        self.ws = torch.empty(tl.tpmlp_bwd_workspace_bytes(tl.BF16, T, h, F, tp), dtype=torch.uint8, device=dev)
        for i in range(1, tp):  # the other ranks' gathered blocks
            self.ln(i)
            self.drop_bwd(i)
        for j in range(1, tp):  # and the other shards' partials
            self.mlp(j)

    def blk(self, i):
        return slice(i * self.rows, (i + 1) * self.rows)

    def ln(self, i):
        s, b = self, self.blk(i)
        s.tl.layernorm_fwd(s.X[b], s.gamma, s.beta, s.Y[b], s.mean[b], s.rstd[b], stream=s.stream)

    def drop_bwd(self, i):
        s, b = self, self.blk(i)
        s.tl.sp_dropout_bwd(s.dOut[b], s.dZ[b], s.p, s.seed, i * s.rows, stream=s.stream)

    def mlp(self, j):
        s, tl = self, self.tl
        tl.tp_mlp_fwd(s.Y, s.W1s[j], None, s.W2s[j], s.wl.tp, s.A, s.Zp[j], H_save=s.H, stream=s.stream)
        tl.tp_mlp_bwd(s.Y, s.W1s[j], s.W2s[j], s.H, s.A, s.dZ, s.wl.tp, s.dXp[j], s.dW1, s.dW2, workspace=s.ws,
                      stream=s.stream)

    def __call__(self):
        s, tl, b = self, self.tl, self.blk(0)
        s.ln(0)
        tl.tp_mlp_fwd(s.Y, s.W1s[0], None, s.W2s[0], s.wl.tp, s.A, s.Zp[0], H_save=s.H, stream=s.stream)
        tl.sp_partial_sum_dropout_residual(s.Zp[:, b], s.X[b], s.out, s.p, s.seed, 0, stream=s.stream)
        s.drop_bwd(0)
        tl.tp_mlp_bwd(s.Y, s.W1s[0], s.W2s[0], s.H, s.A, s.dZ, s.wl.tp, s.dXp[0], s.dW1, s.dW2, workspace=s.ws,
                      stream=s.stream)
        tl.shard_partial_sum(s.dXp[:, b], s.dYln, stream=s.stream)
        tl.layernorm_bwd(s.X[b], s.gamma, s.mean[b], s.rstd[b], s.dYln, s.dXseq, dgamma=s.dgamma, dbeta=s.dbeta,
                         dRes=s.dOut[b], stream=s.stream)


class AttnBlockStep:
    """The head-sharded attention block, shard 0's step: tp_attn_fwd (QKV
    projection, causal attention over its heads, O-projection partial), its
    share of the partial sum of the output, tp_attn_bwd, its share of the
    partial sum of dX.  The other shards' partials are computed once."""

    def __init__(self, wl, raw, tl, torch):
        self.wl, self.tl = wl, tl
        T, h, tp = wl.T, wl.h, wl.tp
        hs = wl.heads // tp
        w = hs * wl.head_dim
        dev = torch.device("cuda:0")
        bf = torch.bfloat16

        def up(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(bf).to(dev)

        self.stream = torch.cuda.current_stream(dev)
        self.X, self.dZ = up(raw["X"]), up(raw["dOut"])
        self.Wqkv = [up(np.concatenate([raw[n][:, i * w:(i + 1) * w] for n in ("Wq", "Wk", "Wv")], axis=1))
                     for i in range(tp)]
        self.Wo = [up(raw["Wo"][i * w:(i + 1) * w]) for i in range(tp)]
        self.QKV = torch.empty((T, 3 * w), dtype=bf, device=dev)
        self.O = torch.empty((T, w), dtype=bf, device=dev)
        self.lse = torch.empty((hs, T), dtype=torch.float32, device=dev)
        self.Zp = torch.empty((tp, T, h), dtype=torch.float32, device=dev)
        self.dXp = torch.empty((tp, T, h), dtype=torch.float32, device=dev)
        self.rows = T // tp
        self.Zsum = torch.empty((self.rows, h), dtype=torch.float32, device=dev)
        self.dXsum = torch.empty((self.rows, h), dtype=torch.float32, device=dev)
        self.dWqkv = torch.empty((h, 3 * w), dtype=torch.float32, device=dev)
        self.dWo = torch.empty((w, h), dtype=torch.float32, device=dev)
        self.ws = torch.empty(tl.tp_attn_bwd_workspace_bytes(1, T, wl.heads, tp), dtype=torch.uint8, device=dev)
        self.fws = torch.empty(max(1, tl.tp_attn_fwd_workspace_bytes(1, T, wl.heads, tp)), dtype=torch.uint8,
                               device=dev)
        for i in range(1, tp):
            self.fwd(i)
            self.bwd(i)

    def fwd(self, i):
        s = self
        s.tl.tp_attn_fwd(s.X, s.Wqkv[i], s.Wo[i], s.QKV, s.O, s.lse, s.Zp[i], 1, s.wl.T, s.wl.heads, s.wl.tp,
                         causal=True, workspace=s.fws, stream=s.stream)

    def bwd(self, i):
        s = self
        s.tl.tp_attn_bwd(s.X, s.Wqkv[i], s.Wo[i], s.QKV, s.O, s.lse, s.dZ, s.dXp[i], s.dWqkv, s.dWo, 1, s.wl.T,
                         s.wl.heads, s.wl.tp, causal=True, workspace=s.ws, stream=s.stream)

    def parts(self):
        r = proj_role_flops(self.wl)
        f = r["gemm.attn_qkv"] + r["attn_fwd"] + r["gemm.attn_out"]
        return {"tp_attn_fwd": (lambda: self.fwd(0), f), "tp_attn_bwd": (lambda: self.bwd(0), step_flops(self.wl) - f)}

    def __call__(self):
        s = self
        s.fwd(0)
        s.tl.shard_partial_sum(s.Zp[:, :s.rows], s.Zsum, stream=s.stream)
        s.bwd(0)
        s.tl.shard_partial_sum(s.dXp[:, :s.rows], s.dXsum, stream=s.stream)


def make_step(wl, tl, torch):
    import synth
    if wl.kind == "proj":
        raw = synth.proj_inputs(wl, which=("X", "Wq", "Wk", "Wv", "Wo", "dOut"))
        return raw, AttnBlockStep(wl, raw, tl, torch)
    if wl.kind == "sp_mlp":
        raw = synth.sp_inputs(wl)
        return raw, SPStep(wl, raw, tl, torch)
    if wl.kind == "swiglu":
        raw = synth.swiglu_inputs(wl)
        return raw, SwiGLUStep(wl, raw, tl, torch)
    if wl.kind == "mlp":
        raw = synth.mlp_inputs(wl)
        return raw, (Step(wl, raw, tl, torch) if wl.dz_std is not None else FwdStep(wl, raw, tl, torch))
    raise SystemExit(f"workload {wl.name}: no benchmark step")


def step_roles(tl, step, torch):
    """Kernel roles and symbols of one step, in launch order."""
    tl.profile_enable("")
    step()
    torch.cuda.synchronize()
    order = tl.profile_collect(ordered=True)
    tl.profile_enable(None)
    return order


def synth_kind(workload: str) -> str:
    import synth
    return synth.WORKLOADS[workload].kind


def load_traffic(workload: str, symbol: str, role: str):
    """Calibrated HBM bytes per launch of (role, symbol), if measured on these sources."""
    try:
        with open(traffic_path(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None, "no traffic table"
    if t.get("fingerprint") != kernel_fingerprint(synth_kind(workload)):
        return None, "kernel sources changed since the counters were taken"
    e = t.get("launches", {}).get(role)
    if not e or e.get("kernel") != symbol:
        return None, "no counters for this kernel"
    return e["fetch_bytes"] + e["write_bytes"], "FETCH_SIZE + WRITE_SIZE, scaled by a plain copy"


def load_mfma(workload: str, symbol: str, role: str):
    """MFMA-busy fraction of (role, symbol) from the committed counter summary, if taken on these sources."""
    try:
        with open(mfma_path(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None, "no MFMA counter table"
    if t.get("fingerprint") != kernel_fingerprint(synth_kind(workload)):
        return None, "kernel sources changed since the counters were taken"
    e = t.get("launches", {}).get(role)
    if not e or e.get("kernel") != symbol:
        return None, "no counters for this kernel"
    return e["mfma_busy"], ("SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x GRBM_GUI_ACTIVE / 8 XCDs): the fraction of the "
                            "kernel's cycles the matrix cores were busy, at whatever clock it ran")


def epilogue_ablation(wl, step, tl, torch, n):
    """The fused bias+GeLU epilogue of the first product against the same
    product with an fp32 output followed by the standalone epilogue pass, and
    the standalone GeLU' pass, on shard 0 of the workload (same stream)."""
    T, Fs = wl.T, wl.Fs
    stream = step.stream
    X, W1, b1, A, H = step.X, step.W1s[0], step.b1s[0], step.A, step.H
    P = torch.empty((T, Fs), dtype=torch.float32, device=X.device)
    dH = torch.empty_like(A)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3

    fused = timed(lambda: tl.column_parallel_fwd(X, W1, wl.tp, A, bias_shard=b1, H_save=H, stream=stream))
    gemm = timed(lambda: tl.row_parallel_fwd(X, W1, 1, P, stream=stream))
    bgf = timed(lambda: tl.bias_gelu_fwd(P, A, bias=b1, H_out=H, stream=stream))
    gb = timed(lambda: tl.gelu_bwd(P, H, dH, stream=stream))
    esz = A.element_size()
    bgf_bytes = T * Fs * (4 + 2 * esz) + (Fs * esz if b1 is not None else 0)
    gb_bytes = T * Fs * (4 + 2 * esz)
    return {"what": f"X W1_0 ({T}x{Fs}, K={wl.h}) with the bias+GeLU epilogue fused vs an fp32 product then "
                    "bias_gelu_fwd; gelu_bwd over the same [T, F/tp]",
            "fused_us": round(fused, 2), "unfused_gemm_fp32_us": round(gemm, 2),
            "bias_gelu_fwd_us": round(bgf, 2), "unfused_total_us": round(gemm + bgf, 2),
            "fusion_saves_us": round(gemm + bgf - fused, 2),
            "bias_gelu_fwd_gbs": round(bgf_bytes / (bgf * 1e-6) / 1e9, 1),
            "gelu_bwd_us": round(gb, 2), "gelu_bwd_gbs": round(gb_bytes / (gb * 1e-6) / 1e9, 1),
            "hbm_peak_gbs": PEAK_HBM_GBS,
            "bytes": {"bias_gelu_fwd": bgf_bytes, "gelu_bwd": gb_bytes}}


def vendor_yardstick(wl, step, torch, n):
    """The six products of shard 0's MLP step through torch.matmul (hipBLASLt),
    bf16 in and out, timed one by one on the step's stream: a yardstick for
    the library's GEMMs, never on its path.  Transposed operands are made
    contiguous beforehand (outside the timing), so every product runs NN."""
    X, W1, W2, A, dZ = step.X, step.W1s[0], step.W2s[0], step.A, step.dZ
    W1T, W2T, XT, AT = (W1.t().contiguous(), W2.t().contiguous(), X.t().contiguous(), A.t().contiguous())
    stream = step.stream
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    prods = {"fwd1 X W1": (X, W1), "fwd2 A W2": (A, W2), "dgrad_act dZ W2^T": (dZ, W2T),
             "wgrad2 A^T dZ": (AT, dZ), "wgrad1 X^T dH": (XT, A), "dgrad1 dH W1^T": (A, W1T)}
    out, total = {}, 0.0
    with torch.cuda.stream(stream):
        for name, (a, b) in prods.items():
            torch.matmul(a, b)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(n):
                torch.matmul(a, b)
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / n * 1e3
            fl = 2.0 * a.shape[0] * a.shape[1] * b.shape[1]
            out[name] = {"us": round(us, 2), "tflops": round(fl / (us * 1e-6) / 1e12, 1)}
            total += us
    return {"what": "torch.matmul (hipBLASLt), bf16 in and out, every product NN with transposes made "
                    "contiguous beforehand; a yardstick, not the library's path",
            "products": out, "sum_us": round(total, 2)}


def workload_text(wl):
    T, h, F, tp, Fs = wl.T, wl.h, wl.F, wl.tp, wl.Fs
    what = {"llama7b_bf16": "the Llama-7B-scale MLP", "gpt2m_bf16": "the GPT-2-medium-scale MLP",
            "gpt3_bf16": "the GPT-3-175B-scale MLP",
            "qwen3_swiglu_bf16": "the Qwen3-8B-scale gated MLP (SwiGLU)",
            "llama7b_sp_bf16": "the Llama-7B-scale MLP inside the sequence-parallel region (LayerNorm before it, "
                               "dropout p=0.1 and the residual after it, T/tp rows of the residual stream per GPU)",
            }.get(wl.name, "the MLP")
    if wl.kind == "proj":
        hs = wl.heads // tp
        return (f"{wl.name}: one shard of the head-sharded attention block, T={T} tokens (one causal sequence), "
                f"h={h}, {wl.heads} heads of {wl.head_dim}, tp={tp} ({hs} heads per shard): fused QKV projection "
                f"{h}x{3 * hs * wl.head_dim}, flash attention, O projection {hs * wl.head_dim}x{h} into an fp32 "
                f"partial; fwd+bwd plus this GPU's 1/tp share of the output and dX partial sums; bf16 storage, "
                f"fp32 accumulate")
    if wl.dz_std is None:
        return (f"{wl.name}: all {tp} shards of the MLP in turn on this GPU, T={T} tokens, h={h}, F={F}, tp={tp} "
                f"(F/tp={Fs}), {'fp32' if wl.dtype == 'f32' else 'bf16'} storage, fp32 accumulate; forward only "
                f"(column-parallel GEMM with bias+GeLU, row-parallel GEMM into an fp32 partial per shard), then "
                f"the on-device sum of the {tp} partials")
    return (f"{wl.name}: one shard of {what}, T={T} tokens, h={h}, F={F}, tp={tp} (F/tp={Fs}), bf16 storage, "
            f"fp32 accumulate; fwd+bwd plus this GPU's 1/tp share of the output and dX partial sums")


def smi_sclk_mhz():
    """GPU 0's shader clock as rocm-smi reports it at this moment, in MHz
    (None when rocm-smi is missing or prints no sclk line)."""
    import shutil
    import subprocess
    exe = shutil.which("rocm-smi") or "/opt/rocm/bin/rocm-smi"
    if not os.path.exists(exe):
        return None
    try:
        r = subprocess.run([exe, "--showclocks"], capture_output=True, text=True, timeout=20)
    except (OSError, subprocess.SubprocessError):
        return None
    m = re.search(r"sclk clock level:\s*\d+:\s*\((\d+)\s*Mhz\)", r.stdout, re.I)
    return int(m.group(1)) if m else None


def run_bench(args):
    import torch
    import synth
    import linear_layers_amd as tl

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    wl = synth.WORKLOADS[args.workload]
    T, h, F, tp, Fs = wl.T, wl.h, wl.F, wl.tp, wl.Fs
    t_setup = time.perf_counter()
    raw, step = make_step(wl, tl, torch)
    stream = step.stream
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    # Python's cyclic garbage collector is kept out of the measured loops: a
    # full pass over the interpreter's heap (torch alone holds ~170k tracked
    # objects) stops the host for tens of ms, and a step's launches queue
    # behind it, so one pass landing inside a timed region stretched that
    # step by 20-30 ms.  Everything alive now is frozen out of later passes
    # and collection stays off until the measurements are taken.
    gc.collect()
    gc.freeze()
    gc.disable()
    smi_before = smi_sclk_mhz()   # before the warm-up, so that the query's idle time precedes it

    # Warm-up: plain steps until the clocks settle, then the last few with
    # every kernel timed to find the dominant one.
    profiled = WARMUP_PROFILED if args.warmup is None else max(1, min(args.warmup, WARMUP_PROFILED))
    plain = 0
    t_w = time.perf_counter()
    if args.warmup is None:
        while plain < WARMUP_MIN_STEPS - profiled or time.perf_counter() - t_w < WARMUP_MIN_S:
            step()
            plain += 1
            if plain % 10 == 0:
                torch.cuda.synchronize()   # count GPU time, not launch time
    else:
        for _ in range(max(0, args.warmup - profiled)):
            step()
            plain += 1
    torch.cuda.synchronize()
    warmup_steps = plain + profiled
    tl.profile_enable("")
    for _ in range(profiled):
        step()
    torch.cuda.synchronize()
    warm = tl.profile_collect()
    tl.profile_enable(None)
    by_role = {}
    for k, (n, ms, sym, clocks) in warm.items():
        role = k.split("|")[0]
        r = by_role.setdefault(role, [0, 0.0, sym, []])
        r[0] += n
        r[1] += ms
        r[3] += clocks
    dominant = max(by_role, key=lambda r: by_role[r][1])

    # Timed region: K steps between two synchronisations; the dominant
    # kernel's launches are bracketed by events on the launch stream.
    tl.profile_enable(dominant)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    smi_after = smi_sclk_mhz()
    timed = tl.profile_collect()
    tl.profile_enable(None)
    ms_step = e0.elapsed_time(e1) / args.steps

    flops_step = step_flops(wl)
    value = flops_step / (ms_step * 1e-3) / 1e12
    peak = PEAK_F32_TFLOPS if wl.dtype == "f32" else PEAK_BF16_TFLOPS

    # Per-step durations over as many steps again, warm and then cold: the cold
    # pass writes a 512 MB buffer between steps (off the clock), which evicts
    # the operands from L2 and the 256 MB Infinity Cache.
    def per_step(n, flush=None):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in ev:
            if flush is not None:
                flush.fill_(1.0)
            a.record(stream)
            step()
            b.record(stream)
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in ev)

    warm_t = per_step(args.steps)
    step_ms = {"mean": round(ms_step, 4), "median": round(warm_t[len(warm_t) // 2], 4), "min": round(warm_t[0], 4),
               "steps": len(warm_t)}
    cold = None
    if not args.no_cold:
        flush = torch.empty(COLD_FLUSH_BYTES // 4, dtype=torch.float32, device="cuda:0")
        cold_t = per_step(args.steps, flush)
        del flush
        med = cold_t[len(cold_t) // 2]
        cold = {"median_ms": round(med, 4), "min_ms": round(cold_t[0], 4), "steps": len(cold_t),
                "value_at_median": round(flops_step / (med * 1e-3) / 1e12, 2),
                "flush_bytes_between_steps": COLD_FLUSH_BYTES}

    # The step's forward and backward calls, each timed alone (after the timed
    # region, so they do not change it): same launches, same stream.
    parts = {}
    if hasattr(step, "parts"):
        for name, (fn, pflops) in step.parts().items():
            fn()
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(args.steps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            pms = e0.elapsed_time(e1) / args.steps
            ptf = pflops / (pms * 1e-3) / 1e12
            parts[name] = {"us": round(pms * 1e3, 2), "tflops": round(ptf, 2),
                           "pct_of_peak": round(100 * ptf / peak, 2)}

    ablation = epilogue_ablation(wl, step, tl, torch, args.steps) if isinstance(step, Step) else None
    vendor = vendor_yardstick(wl, step, torch, args.steps) if args.vendor and isinstance(step, Step) else None
    gc.enable()

    # Dominant kernel: algorithmic flops per launch / mean launch duration.
    dom_key = max((k for k in timed if k.startswith(dominant + "|")), key=lambda k: timed[k][1])
    n_launch, dom_ms, dom_sym, dom_clocks = timed[dom_key]
    per_launch_ms = dom_ms / n_launch
    achieved = role_flops(wl, dominant) / (per_launch_ms * 1e-3) / 1e12
    # The peak assumes the 2.4 GHz peak engine clock; the clock the GEMM
    # actually ran at (sampled in-kernel over workgroup 0's main loop) is
    # reported beside it, with the peak scaled to that clock.
    sclk = sum(dom_clocks) / len(dom_clocks) if dom_clocks else None
    traffic, traffic_note = load_traffic(wl.name, dom_sym, dominant)
    mfma_busy, mfma_note = load_mfma(wl.name, dom_sym, dominant)
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic,
                "traffic_note": traffic_note, "mfma_busy": mfma_busy, "mfma_busy_note": mfma_note,
                "algorithmic_bytes": None, "kernel": dom_sym, "role": dominant, "launches": n_launch,
                "mean_launch_us": round(per_launch_ms * 1e3, 2), "flop_per_launch": role_flops(wl, dominant),
                "sclk_ghz": round(sclk, 3) if sclk else None,
                "peak_at_sclk": round(peak * sclk / PEAK_SCLK_GHZ, 1) if sclk else None,
                "frac_at_sclk": round(achieved / (peak * sclk / PEAK_SCLK_GHZ), 4) if sclk else None}
    roofline["algorithmic_bytes"] = algorithmic_bytes(wl, dominant)

    kernels = {}
    for role, (n, ms, sym, clocks) in sorted(by_role.items(), key=lambda kv: -kv[1][1]):
        us = ms / n * 1e3
        entry = {"kernel": sym, "mean_us": round(us, 2)}
        if clocks:
            entry["sclk_ghz"] = round(sum(clocks) / len(clocks), 3)
        if role.startswith("gemm") or role_flops(wl, role):
            entry["tflops"] = round(role_flops(wl, role) / (us * 1e-6) / 1e12, 1)
        elif role in ("partial_sum", "colsum"):
            bm = tile_rows(by_role.get("gemm.mlp_dgrad_act", (0, 0, "", []))[2]) or 256
            nbytes = hbm_role_bytes(wl, role, bm)
            entry["gbs"] = round(nbytes / (us * 1e-6) / 1e9, 1)
        kernels[role] = entry

    out = {
        "metric": {"mlp": "TFLOP/s and % of bf16 MFMA peak for TP-sharded MLP fwd+bwd",
                   "swiglu": "TFLOP/s and % of bf16 MFMA peak for TP-sharded gated MLP (SwiGLU) fwd+bwd",
                   "sp_mlp": "TFLOP/s and % of bf16 MFMA peak for the TP+SP MLP block fwd+bwd",
                   "proj": "TFLOP/s and % of bf16 MFMA peak for the head-sharded attention block fwd+bwd"}[wl.kind],
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warmup_steps,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if wl.dtype == "f32" else "bf16",
        "data": "synthetic (seeded normal inputs and random-init weights of the workload's shapes)",
        "config": {"workload": workload_text(wl),
                   "global_batch": T, "seq_len": None, "parallelism": f"tp{tp} shard simulated on 1 GPU"},
        "pct_of_peak": round(100 * value / peak, 2),
        "step_ms": step_ms,
        "sclk_rocm_smi_mhz": {"before_warmup": smi_before, "after_timed": smi_after,
                              "note": "instantaneous readings outside the timed steps; the clock the dominant "
                                      "kernel ran at is roofline.sclk_ghz (sampled in-kernel)"},
        "cold": cold,
        "roofline": roofline,
        "parts": parts,
        "epilogue_ablation": ablation,
        "vendor_yardstick": vendor,
        "kernels_warmup": kernels,
        "wall_s_timed": round(wall, 4),
        "setup_s": round(setup_s, 2),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, raw, args.cpu_seconds)
        out["cpu_baseline"]["gpu_over_cpu"] = round(value / out["cpu_baseline"]["value"], 1)
    if args.breakdown:
        print(json.dumps(timed), file=sys.stderr)
    print(json.dumps(out), flush=True)


def run_profile_pass(args):
    """A plain copy of CALIB_BYTES, then set-up and one step (for rocprofv3 --pmc)."""
    import torch
    import synth
    import linear_layers_amd as tl

    src = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)            # the first kernel of the process: the calibration copy
    torch.cuda.synchronize()
    wl = synth.WORKLOADS[args.workload]
    raw, step = make_step(wl, tl, torch)
    step()                    # warm
    torch.cuda.synchronize()
    order = step_roles(tl, step, torch)   # the last step: its launches in order
    with open(args.profile_pass, "w") as f:
        json.dump({"workload": wl.name, "order": order, "fingerprint": kernel_fingerprint(wl.kind),
                   "cus": torch.cuda.get_device_properties(0).multi_processor_count}, f)
    print(json.dumps({"profile_pass": args.profile_pass, "launches": len(order)}), flush=True)


def _read_pmc(csv_path, counter):
    """(dispatch id, kernel name, value) of one counter, in dispatch order."""
    rows = []
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    rows.sort()
    return rows


def summarize_mfma(d, roles, cmds):
    """profiles/<workload>_mfma.{txt,json}: MFMA-busy fraction of each kernel role of one step."""
    csvs = glob.glob(os.path.join(d, "mfma", "**", "*counter_collection.csv"), recursive=True)
    busy = _read_pmc(csvs[0], "SQ_VALU_MFMA_BUSY_CYCLES")
    gui = _read_pmc(csvs[0], "GRBM_GUI_ACTIVE")
    simds = 4 * int(roles.get("cus", 256))
    n = len(roles["order"])
    lib_b = [r for r in busy if "tpmlp::" in r[1]][-n:]
    lib_g = [r for r in gui if "tpmlp::" in r[1]][-n:]
    launches = {}
    lines = [f"# MFMA utilisation per launch, {roles['workload']} step (one launch of each kernel role)", "",
             f"command: {cmds.get('mfma', 'rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE -- python3 bench.py --profile-pass OUT')}",
             "", f"mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / ({simds} SIMDs x GRBM_GUI_ACTIVE / {XCDS} XCDs): the share of",
             "the kernel's cycles in which the matrix cores were busy, at whatever clock the kernel ran",
             "(against the 2.4 GHz peak, frac = mfma_busy x clock / 2.4 GHz).", "",
             f"{'role':24s} {'kernel':44s} {'cycles':>9s} {'mfma_busy':>9s}"]
    for (role, sym), (_, name, b), (_, _, g) in zip(roles["order"], lib_b, lib_g):
        assert canon(name) == sym, f"launch order mismatch: {canon(name)} != {sym}"
        cyc = g / XCDS
        frac = b / (simds * cyc) if cyc > 0 else 0.0
        if role in launches:   # a role launched twice in the step keeps its first launch
            continue
        launches[role] = {"kernel": sym, "mfma_busy": round(frac, 4), "cycles": round(cyc)}
        lines.append(f"{role:24s} {sym:44s} {cyc:9.0f} {frac:9.3f}")
    with open(os.path.join(PROFILES, f"{roles['workload']}_mfma.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(mfma_path(roles["workload"]), "w") as f:
        json.dump({"fingerprint": roles["fingerprint"], "workload": roles["workload"], "simds": simds,
                   "launches": launches}, f, indent=1)


def summarize_profile(d):
    """Write profiles/*.txt and profiles/traffic.json from rocprofv3 output under d."""
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(d, "roles.json")) as f:
        roles = json.load(f)
    cmds = {}
    if os.path.exists(os.path.join(d, "commands.json")):
        with open(os.path.join(d, "commands.json")) as f:
            cmds = json.load(f)
    if os.path.isdir(os.path.join(d, "mfma")):
        summarize_mfma(d, roles, cmds)
    if not os.path.isdir(os.path.join(d, "fetch_size")):
        return
    scaled = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        csvs = glob.glob(os.path.join(d, counter.lower(), "**", "*counter_collection.csv"), recursive=True)
        rows = _read_pmc(csvs[0], counter)
        calib = next(r for r in rows if "copy" in r[1].lower())
        factor = CALIB_BYTES / (calib[2] * 1024.0)
        lib = [r for r in rows if "tpmlp::" in r[1]]
        last = lib[-len(roles["order"]):]
        for (role, sym), (_, name, kib) in zip(roles["order"], last):
            assert canon(name) == sym, f"launch order mismatch: {canon(name)} != {sym}"
            scaled.setdefault(role, {"kernel": sym})[counter] = (kib, kib * 1024.0 * factor)
        scaled.setdefault("_calibration", {})[counter] = {"counter_kib": calib[2], "factor": factor}
    launches = {}
    lines = [f"# HBM traffic per launch, {roles['workload']} step (one launch of each kernel role)",
             "", f"fetch: {cmds.get('fetch', 'rocprofv3 --pmc FETCH_SIZE -- python3 bench.py --profile-pass OUT')}",
             f"write: {cmds.get('write', 'rocprofv3 --pmc WRITE_SIZE -- python3 bench.py --profile-pass OUT')}",
             "", "Counters are KiB per dispatch, scaled by the factor that maps a plain "
             f"{CALIB_BYTES >> 20} MiB copy (torch copy_, first kernel of the process) to its known bytes:",
             f"  FETCH_SIZE factor {scaled['_calibration']['FETCH_SIZE']['factor']:.4f} "
             f"(copy read {scaled['_calibration']['FETCH_SIZE']['counter_kib']:.0f} KiB)",
             f"  WRITE_SIZE factor {scaled['_calibration']['WRITE_SIZE']['factor']:.4f} "
             f"(copy wrote {scaled['_calibration']['WRITE_SIZE']['counter_kib']:.0f} KiB)", "",
             "alg MB: the algorithmic bytes of the launch (operands and outputs once each); "
             "ratio: (fetch + write) / alg MB.", "",
             f"{'role':22s} {'kernel':44s} {'fetch MB':>9s} {'write MB':>9s} {'alg MB':>9s} {'ratio':>6s}"]
    import synth
    wl = synth.WORKLOADS[roles["workload"]]
    bm = tile_rows(scaled.get("gemm.mlp_dgrad_act", {}).get("kernel")) or 256
    for role, e in scaled.items():
        if role.startswith("_"):
            continue
        fb, wb = e["FETCH_SIZE"][1], e["WRITE_SIZE"][1]
        alg = algorithmic_bytes(wl, role) if role.startswith("gemm") else hbm_role_bytes(wl, role, bm)
        launches[role] = {"kernel": e["kernel"], "fetch_bytes": fb, "write_bytes": wb, "algorithmic_bytes": alg}
        tail = f" {alg / 1e6:9.1f} {(fb + wb) / alg:6.2f}" if alg else f" {'-':>9s} {'-':>6s}"
        lines.append(f"{role:22s} {e['kernel']:44s} {fb / 1e6:9.1f} {wb / 1e6:9.1f}" + tail)
    with open(os.path.join(PROFILES, f"{roles['workload']}_step_hbm_traffic.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(traffic_path(roles["workload"]), "w") as f:
        json.dump({"fingerprint": roles["fingerprint"], "workload": roles["workload"], "launches": launches,
                   "calibration": scaled["_calibration"]}, f, indent=1)
    # kernel-trace statistics
    stats = glob.glob(os.path.join(d, "stats", "**", "*kernel_stats.csv"), recursive=True)
    if stats:
        with open(stats[0]) as f:
            st = list(csv.DictReader(f))
        out = [f"# Kernel durations, {roles['workload']} bench run",
               "", f"command: {cmds.get('stats', 'rocprofv3 --kernel-trace --stats -- python3 bench.py')}", "",
               f"{'kernel':60s} {'calls':>6s} {'avg us':>9s} {'min us':>9s} {'max us':>9s} {'%':>6s}"]
        for r in st:
            name = canon(r["Name"])
            if len(name) > 60:
                name = name[:57] + "..."
            out.append(f"{name:60s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} "
                       f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} {float(r['Percentage']):6.2f}")
        with open(os.path.join(PROFILES, f"{roles['workload']}_kernel_stats.txt"), "w") as f:
            f.write("\n".join(out) + "\n")
    print(f"wrote profiles for {roles['workload']}")


# (mode, pattern, label) of the load-path probe, run at two pairs of leading
# dimensions: powers of two, and padded by 64 elements.
PROBE_LOADS = [
    (0, 0, "LDS DMA, A and B as in the GEMM tiles"),
    (0, 1, "LDS DMA, A only (8 rows x 128 B a load)"),
    (0, 3, "LDS DMA, A only, a load's rows 32 apart"),
    (0, 2, "LDS DMA, B only (2 K-rows x 512 B a load)"),
    (1, 0, "register loads, A and B"),
    (1, 1, "register loads, A only"),
    (1, 2, "register loads, B only"),
    (2, 0, "register loads + ds_write_b128, A and B"),
]
PROBE_LDS = [(0, w, "ds_read_b128") for w in (4, 8, 16)] + [(1, w, "ds_read_b64_tr_b16") for w in (4, 8, 16)]


def run_probes():
    """Run libtpmlp_probe.so's probes on the current GPU: one text line per
    case, then one JSON line with every figure."""
    import ctypes
    path = os.path.join(ROOT, "linear_layers_amd", "libtpmlp_probe.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    lib.tpmlp_probe_last_error.restype = ctypes.c_char_p
    out = (ctypes.c_double * 4)()
    res = {"load_path": [], "lds_read": []}
    for lda, ldb in ((4096, 8192), (4160, 8256)):
        print(f"load path, lda {lda}, ldb {ldb} (bf16 elements; 64 KB per CU per step, 64 steps)", flush=True)
        for mode, pat, label in PROBE_LOADS:
            rc = lib.tpmlp_probe_load_path(mode, pat, lda, ldb, 20, out)
            if rc != 0:
                raise SystemExit(f"load probe {mode}/{pat}: {lib.tpmlp_probe_last_error().decode()}")
            us, ghz, gbs, bpc = out[0], out[1], out[2], out[3]
            print(f"  {label:44s} {us:7.1f} us {gbs:7.0f} GB/s  clk {ghz:.2f} GHz  {bpc:5.1f} B/clk/CU", flush=True)
            res["load_path"].append({"mode": mode, "pattern": pat, "lda": lda, "ldb": ldb, "label": label,
                                     "us": round(us, 2), "sclk_ghz": round(ghz, 3), "gb_s": round(gbs, 1),
                                     "bytes_per_clk_cu": round(bpc, 2)})
    print("LDS reads (8 independent reads per wave, then a wait)", flush=True)
    for tr, waves, label in PROBE_LDS:
        rc = lib.tpmlp_probe_lds_read(tr, waves, 4096, out)
        if rc != 0:
            raise SystemExit(f"LDS probe {label}/{waves}: {lib.tpmlp_probe_last_error().decode()}")
        print(f"  {label:20s} {waves:2d} waves: {out[1]:6.1f} B/clk/CU", flush=True)
        res["lds_read"].append({"instruction": label, "waves": waves, "bytes_per_clk_cu": round(out[1], 1)})
    print(json.dumps(res))


POWER_SECONDS = 3.0      # back-to-back steps timed by --power
POWER_SAMPLE_S = 0.02


def run_power(args):
    """Board power while the workload's step runs back to back: the GPU's
    hwmon power1_input (instantaneous, microwatts) and power1_cap, read from
    sysfs by a host thread every 20 ms; the first 0.5 s is left out.  Prints
    one text line and one JSON line."""
    import threading
    import torch
    import synth
    import linear_layers_amd as tl
    mons = sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*/power1_input"))
    if not mons or not torch.cuda.is_available():
        raise SystemExit("no GPU power sensor (hwmon power1_input) or no GPU visible")
    hw = os.path.dirname(mons[0])

    def read(name):
        try:
            with open(os.path.join(hw, name)) as f:
                return int(f.read())
        except (OSError, ValueError):
            return None

    wl = synth.WORKLOADS[args.workload]
    _, step = make_step(wl, tl, torch)
    gc.collect()
    gc.freeze()
    gc.disable()
    idle = read("power1_input")
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            samples.append((time.perf_counter(), read("power1_input"), read("temp2_input")))
            time.sleep(POWER_SAMPLE_S)

    th = threading.Thread(target=sampler)
    th.start()
    t0, n = time.perf_counter(), 0
    while time.perf_counter() - t0 < POWER_SECONDS:
        step()
        n += 1
        if n % 20 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stop.set()
    th.join()
    gc.enable()
    watts = sorted(p / 1e6 for t, p, _ in samples if t - t0 > 0.5 and p is not None)
    temps = [c / 1e3 for t, _, c in samples if t - t0 > 0.5 and c is not None]
    cap = read("power1_cap")
    res = {"workload": wl.name, "steps": n, "ms_per_step": round(wall / n * 1e3, 4),
           "power_cap_w": cap / 1e6 if cap else None, "idle_w": idle / 1e6 if idle else None,
           "samples": len(watts), "median_w": watts[len(watts) // 2], "p10_w": watts[len(watts) // 10],
           "p90_w": watts[9 * len(watts) // 10], "max_w": watts[-1],
           "junction_c": [min(temps), max(temps)] if temps else None}
    print(f"{wl.name}: {n} steps in {wall:.2f} s; power cap {res['power_cap_w']} W, idle {res['idle_w']} W; "
          f"under load median {res['median_w']:.0f} W (p10 {res['p10_w']:.0f}, p90 {res['p90_w']:.0f}, "
          f"max {res['max_w']:.0f}); junction {res['junction_c']} C", flush=True)
    print(json.dumps(res))


def main():
    args = parse()
    if args.probe:
        run_probes()
        return
    if args.power:
        run_power(args)
        return
    if args.summarize_profile:
        summarize_profile(args.summarize_profile)
        return
    if args.gpus != 1:
        print(json.dumps({"error": f"--gpus {args.gpus}: the benchmark runs on one GPU only; "
                                   "other tensor-parallel ranks are simulated on it in turn, "
                                   "and the multi-GPU path is a design, not code"}))
        sys.exit(2)
    if args.profile_pass:
        run_profile_pass(args)
        return
    run_bench(args)


if __name__ == "__main__":
    main()
