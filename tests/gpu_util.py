"""Helpers shared by the GPU parity tests (no method arithmetic here)."""

from __future__ import annotations

import numpy as np
import torch

# Tolerances: max relative (normwise) error of fp32 outputs and gradients, and
# of outputs computed from bf16 operands.
TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def device():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm device")
    return torch.device("cuda:0")


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device())


def sigma32(s: float) -> float:
    """The fp32 value of sigma that the C ABI receives."""
    return float(np.float32(s))


def normwise_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max |gpu - ref| / max |ref| over all elements."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    denom = np.max(np.abs(ref)) if ref.size else 1.0
    if denom == 0:
        denom = 1.0
    return float(np.max(np.abs(gpu - ref)) / denom) if ref.size else 0.0


def assert_close(gpu, ref, tol, what=""):
    err = normwise_err(gpu, ref)
    assert np.all(np.isfinite(np.asarray(gpu))), f"{what}: non-finite output"
    assert err <= tol, f"{what}: normwise error {err:.3e} > {tol:.1e}"
    return err


def u32(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def bf16_round_cpu(a: np.ndarray) -> np.ndarray:
    """Nearest bf16 (ties to even) via torch on the CPU, back as float64."""
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
