"""Shared helpers of the GPU parity tests: device inputs from the seeded
workload generator, host copies for the oracle, and the comparison rules."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import workloads as W

DEV = torch.device("cuda")


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def say(msg: str) -> None:
    """Name the case on stdout before a GPU step (flushed)."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact host float64 copy of a bf16 / fp32 tensor (or int copy)."""
    t = t.detach().cpu()
    if t.is_floating_point():
        return t.to(torch.float64).numpy()
    if t.dtype == torch.bool:
        return t.numpy()
    return t.numpy()


def conv_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max_i |got - ref| / max(|ref_i|, RMS(ref)) (the conv's error measure)."""
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    denom = np.maximum(np.abs(ref), rms if rms > 0 else 1.0)
    return float(np.max(np.abs(got - ref) / denom)) if ref.size else 0.0


CONV_TOL = {"bf16": 1e-2, "f32": 1e-5}


def device_inputs(w: W.Workload, parts=("conv", "logits", "selector", "sampling"), seed=None):
    require_gpu()
    return W.make_inputs(w, device=DEV, seed=seed, parts=parts)


def sample_indices(n: int, k: int, seed: int = 0) -> np.ndarray:
    """First, last and k-2 seeded random indices of range(n), sorted."""
    if n <= k:
        return np.arange(n)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, n - 1), size=k - 2, replace=False)
    return np.sort(np.concatenate([[0, n - 1], mid]))
