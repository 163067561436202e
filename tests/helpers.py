"""Shared test helpers (no method arithmetic)."""
from __future__ import annotations

import numpy as np
import torch

# Tolerances (absolute) for floating-point parity with the fp64 oracle.
TOL_F32 = 1e-4          # fp32 inputs: out, lse, lazy ratio
TOL_BF16_OUT = 2e-2     # bf16 inputs: attention output
TOL_BF16_LSE = 1e-3     # bf16 inputs: log-sum-exp
TOL_BF16_RATIO = 1e-3   # bf16 inputs: lazy ratio


def np64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a device/host tensor to float64 numpy."""
    return t.detach().to("cpu", torch.float64).numpy()


def maxerr(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b)))


def assert_close(name: str, got, want, tol: float) -> None:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, f"{name}: shape {got.shape} != {want.shape}"
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    e = maxerr(got, want)
    assert e <= tol, f"{name}: max abs err {e:.3e} > {tol:.1e}"
