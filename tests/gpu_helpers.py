"""Shared helpers of the GPU parity tests (no method arithmetic here)."""
import sys

import numpy as np
import torch

DEV = "cuda"
TOL = {"f32": 1e-5, "bf16": 2e-2}


def say(*a):
    """Print and flush, so the last case is known if a GPU step dies."""
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def maxerr(gpu: torch.Tensor, ref: np.ndarray) -> float:
    g = f64(gpu)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.isfinite(g).all()
    return float(np.abs(g - ref).max()) if g.size else 0.0


def random_selection(rng, n_cand: int, k: int) -> list:
    """A valid kept set for stage-wise attention tests: min(k, n_cand)
    distinct candidates in ascending order, then -1."""
    n = min(k, n_cand)
    sel = sorted(rng.choice(n_cand, size=n, replace=False).tolist()) if n else []
    return sel + [-1] * (k - n)
