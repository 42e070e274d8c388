"""Shared helpers for the GPU parity tests (inputs come from the seeded input
module; expected values from the fp64 oracle)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

BF16_TOL = 2e-2   # max-abs, bf16 inputs with fp32 accumulation
F32_TOL = 1e-4    # max-abs, fp32 inputs
# relative RMS error bound of the full-size bf16 checks: the RNE rounding of a
# bf16 output alone is ~1.6e-3 relative RMS; the bf16 states and softmax
# weights add about as much again in quadrature (~2.3e-3)
RMS_TOL = 3e-3


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import recurrence_augmented_dilated_amd as R
    R.lib()  # raises loudly if librat.so is missing
    return R


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def max_abs(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def rel_rms(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.sqrt(np.mean((got - ref) ** 2) / max(np.mean(ref ** 2), 1e-30))) if ref.size else 0.0


def report(name, got, ref, rms_max=None):
    """Print max-abs and relative RMS errors; assert rel_rms <= rms_max if
    given.  Returns the max-abs error."""
    err = max_abs(got, ref)
    rms = rel_rms(got, ref)
    print(f"[parity] {name}: max_abs={err:.3e} rel_rms={rms:.3e}", flush=True)
    if rms_max is not None:
        assert rms <= rms_max, (name, rms, rms_max)
    return err
