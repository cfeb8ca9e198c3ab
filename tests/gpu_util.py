"""Host-side helpers of the GPU tests: uploads, downloads and error ratios.

Only data movement happens here (torch allocations and copies); every value
compared comes from the library's kernels or from the float64 oracle.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth

TOL = {"bf16": 2e-2, "f32": 1e-5}


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Upload a drawn tensor (float32 values or bf16 bit patterns)."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Download a device tensor to float64 (bf16 decoded bit-exactly)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return synth.bf16_bits_to_f32(t.view(torch.int16).numpy().view(np.uint16)).astype(np.float64)
    return t.numpy().astype(np.float64)


def empty(shape, dtype: str, fill=float("nan")) -> torch.Tensor:
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return torch.full(shape, fill, dtype=tdt, device="cuda")


def empty_f32(shape, fill=float("nan")) -> torch.Tensor:
    return torch.full(shape, fill, dtype=torch.float32, device="cuda")


def err_ratio(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref| (NaN anywhere counts as failure)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"shape {got.shape} != {ref.shape}"
    if got.size == 0:
        return 0.0
    if not np.all(np.isfinite(got)):
        return float("inf")
    scale = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got - ref))) / (scale if scale > 0 else 1.0)


def assert_close(got, ref, dtype: str, what: str, tol: float = None):
    tol = TOL[dtype] if tol is None else tol
    r = err_ratio(got, ref)
    assert r <= tol, f"{what}: max|err|/max|ref| = {r:.3e} > {tol:.0e}"
    return r


def sync():
    torch.cuda.synchronize()
