"""Helpers shared by the GPU parity tests (device upload, comparisons)."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import long_context_exact_ring_amd as ra

# Tolerances for the comparison with the fp64 oracle: bf16 inputs -> max-abs
# 1e-2 and mean-abs 1e-3; fp32 inputs -> max-abs 1e-5.  Applied to out, lse
# and every gradient.
TOL = {"bf16": (1e-2, 1e-3), "f32": (1e-5, 1e-5)}


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    ra.lib()  # fails loudly when the HIP library is missing


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.cuda()


def compare(name: str, got, ref: np.ndarray, dtype: str, mask: np.ndarray | None = None):
    """Assert max/mean abs error against the oracle; returns (max, mean)."""
    g = got.detach().float().cpu().numpy() if isinstance(got, torch.Tensor) else np.asarray(got)
    g = g.astype(np.float64)
    if mask is not None:
        g, ref = g[mask], ref[mask]
    both_inf = np.isneginf(g) & np.isneginf(ref)
    assert np.array_equal(np.isneginf(g), np.isneginf(ref)), f"{name}: -inf pattern differs"
    assert not np.any(np.isnan(g)), f"{name}: NaN in GPU result"
    err = np.abs(np.where(both_inf, 0.0, g - np.where(both_inf, 0.0, ref)))
    mx, mean = float(err.max(initial=0.0)), float(err.mean()) if err.size else 0.0
    tmax, tmean = TOL[dtype]
    log(f"  {name}: max_abs={mx:.3e} mean_abs={mean:.3e} (tol {tmax:g}/{tmean:g})")
    assert mx <= tmax, f"{name}: max abs error {mx:.3e} > {tmax}"
    assert mean <= tmean, f"{name}: mean abs error {mean:.3e} > {tmean}"
    return mx, mean
