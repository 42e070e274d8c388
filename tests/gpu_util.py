"""Shared helpers for the GPU parity tests (inputs come from the seeded input
module; expected values from the fp64 oracle)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

BF16_TOL = 2e-2   # max-abs, bf16 inputs with fp32 accumulation
F32_TOL = 1e-4    # max-abs, fp32 inputs


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


def report(name, got, ref):
    err = max_abs(got, ref)
    rms = float(np.sqrt(np.mean((np.asarray(got) - np.asarray(ref)) ** 2) / max(np.mean(np.asarray(ref) ** 2), 1e-30)))
    print(f"[parity] {name}: max_abs={err:.3e} rel_rms={rms:.3e}", flush=True)
    return err
