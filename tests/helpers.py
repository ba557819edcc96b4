"""Shared helpers of the GPU parity tests (test infrastructure only)."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

TOL = {"f32": 1e-4, "bf16": 2e-2}   # relative L2 bars for float32 / bfloat16 inputs


def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but no GPU is visible")
    return torch.device("cuda:0")


def say(*a):
    """Name the case before the GPU runs it (flushed, so it survives a crash)."""
    print(*a, file=sys.stderr, flush=True)


def to_cpu(x: dict) -> dict:
    return {k: v.detach().cpu() for k, v in x.items()}


def heads(x: dict, idx) -> dict:
    """Select (b, h) pairs (a list of tuples) as a [1, n, ...] batch."""
    out = {}
    for k, v in x.items():
        out[k] = torch.stack([v[b, h] for b, h in idx])[None]
    return out


def rel_l2(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-300))
