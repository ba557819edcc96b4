"""Special-case references and a brute force (oracle; test infrastructure only).

None of these uses the closed-form level function or the Fenwick recurrence,
so each is an independent check of ``forms``:

* ``mamba2`` -- the scalar-gated linear recurrence S_t = a_t S_{t-1} +
  k_t v_t^T, o_t = S_t^T q_t.  With every lambda equal to c the log-linear
  operator is c times this: the hierarchical mask collapses to the causal
  mask, leaving Mamba-2's semiseparable mask ([LLA-it] Sommario tecnico
  section 2, item 2; [LLA-es] Resumen tecnico section 2, "Variantes", item 1).
* ``causal_linear_attention`` -- (Q K^T . tril) V: the lower-triangular
  all-ones mask that the hierarchical matrix replaces ([LLA-es] section 2,
  "Conceptos clave", H-matrices).  Equals the operator when log_a = 0 and
  lambda = 1.
* ``diagonal_only`` -- o_t = (q_t . k_t) v_t: only the level-0 bucket (the
  token itself).
* ``brute_force`` -- pure-Python loops over (t, s) with the gate as the
  explicit product prod_{s<r<=t} a_r and the bucket of every key found by the
  Fenwick walk of ``levels.walk_buckets``.  For tiny inputs only.
"""

from __future__ import annotations

import numpy as np

from .forms import _f64
from .levels import walk_buckets


def mamba2(q, k, v, log_a):
    """Scalar-gated linear attention by its recurrence; [B,H,T,dv]."""
    q, k, v, log_a = (_f64(x) for x in (q, k, v, log_a))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    out = np.zeros((B, H, T, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv))
            for t in range(T):
                S = np.exp(log_a[b, h, t]) * S + np.outer(k[b, h, t], v[b, h, t])
                out[b, h, t] = S.T @ q[b, h, t]
    return out


def causal_linear_attention(q, k, v):
    """(Q K^T masked to s <= t) V; [B,H,T,dv]."""
    q, k, v = (_f64(x) for x in (q, k, v))
    T = q.shape[2]
    tril = np.tril(np.ones((T, T)))
    return np.einsum("bhts,bhsd->bhtd", np.einsum("bhtd,bhsd->bhts", q, k) * tril, v)


def diagonal_only(q, k, v, lam0):
    """o_t = lam0_t (q_t . k_t) v_t; lam0: [B,H,T]."""
    q, k, v, lam0 = (_f64(x) for x in (q, k, v, lam0))
    return (lam0 * np.einsum("bhtd,bhtd->bht", q, k))[..., None] * v


def brute_force(q, k, v, a, lam):
    """Pure-Python evaluation of the definition for tiny inputs.

    q, k: [T, dk]; v: [T, dv]; a: [T] gates; lam: [T, L].  Returns [T, dv].
    """
    q, k, v, a, lam = (_f64(x) for x in (q, k, v, a, lam))
    T, dv = v.shape
    out = np.zeros((T, dv))
    for t in range(T):
        for lev, lo, hi in walk_buckets(t):
            for s in range(lo, hi):
                gate = 1.0
                for r in range(s + 1, t + 1):
                    gate *= a[r]
                dot = 0.0
                for i in range(q.shape[1]):
                    dot += q[t, i] * k[s, i]
                for j in range(dv):
                    out[t, j] += lam[t, lev] * gate * dot * v[s, j]
    return out
