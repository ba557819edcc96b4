"""Error metric (oracle; test infrastructure only).

rel_l2(x, ref) = ||x - ref||_2 / ||ref||_2 over the whole tensor, accumulated
in float64.  The tolerances the tests apply to it (1e-4 for float32 inputs,
2e-2 for bfloat16 inputs) are stated in the tests themselves.
"""

from __future__ import annotations

import numpy as np

from .forms import _f64


def rel_l2(x, ref) -> float:
    x, ref = _f64(x), _f64(ref)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((x - ref).ravel())
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


def rel_l2_per_head(x, ref) -> np.ndarray:
    """Relative L2 per leading (B, H) index; [B, H]."""
    x, ref = _f64(x), _f64(ref)
    d = (x - ref).reshape(x.shape[0], x.shape[1], -1)
    r = ref.reshape(ref.shape[0], ref.shape[1], -1)
    den = np.linalg.norm(r, axis=-1)
    return np.linalg.norm(d, axis=-1) / np.where(den == 0, 1.0, den)
