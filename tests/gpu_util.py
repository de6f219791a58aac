"""Helpers for the GPU parity tests (tolerances, sampling, device setup)."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

# Acceptance tolerances (max abs error against the float64 oracle).
TOL_F32 = 1e-5
TOL_BF16 = 2e-2
TOL_GATE = 1e-6


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_routed_query_amd  # noqa: F401  (fails loudly if libgqa.so is missing)

    return torch.device("cuda:0")


def say(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a failing run shows it."""
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def max_abs(a, b) -> float:
    a = np64(a) if isinstance(a, torch.Tensor) else np.asarray(a, dtype=np.float64)
    b = np64(b) if isinstance(b, torch.Tensor) else np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    return float(np.abs(a - b).max()) if a.size else 0.0


def sample_tokens(T: int, n: int, seed: int, tile: int = 64) -> list[int]:
    """Edge tokens (first, last, tile boundaries) plus seeded random ones."""
    rng = np.random.default_rng(seed)
    edge = {0, 1, T - 1, T - 2}
    for b in range(tile, T, tile * 7):
        edge |= {b - 1, b}
    pts = sorted(t for t in edge if 0 <= t < T)
    pts += sorted(rng.integers(0, T, size=max(n - len(pts), 0)).tolist())
    return pts
