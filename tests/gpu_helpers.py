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


def check_fp8(got, ref):
    """FP8 attention output against the oracle's attend_fp8 (o, amean, rms):
    every element within 2^-4 amean + 2^-8 |o| + 3e-3 (the kernel rounds each
    probability times its value row's exponent to E4M3: relative error at most
    2^-4 per weight; the rest covers bf16 outputs and split records), and the
    mean of ((o_gpu - o) / rms)^2 below (0.6 * 2^-4)^2."""
    o, am, rm = ref
    g = f64(got)
    assert g.shape == o.shape and np.isfinite(g).all()
    err = np.abs(g - o)
    tol = 2.0 ** -4 * am + 2.0 ** -8 * np.abs(o) + 3e-3
    worst = float((err / tol).max())
    ms = float(np.mean((err / np.maximum(rm, 1e-3)) ** 2))
    say(f"  max err {err.max():.3g}, worst err/tol {worst:.3f}, mean (err/rms)^2 {ms:.3g}")
    assert worst <= 1.0
    assert ms <= (0.6 * 2.0 ** -4) ** 2


def fp8_host_rows(codes, words):
    """FP8 rows as the library stores them (codes, one scale word per row with
    the exponent byte in bits 23..30) in the oracle's layout: codes and the
    exponent byte repeated per 32 values."""
    c = codes.cpu().numpy()
    e = (words.cpu().numpy() >> 23).astype(np.uint8)
    return c, np.repeat(e[..., None], c.shape[-1] // 32, axis=-1)
