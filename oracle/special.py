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
* ``mamba2_backward`` -- the gradients of ``mamba2`` by its adjoint
  recurrence, run backwards in time: the state gradient dS_t = q_t dout_t^T
  + a_{t+1} dS_{t+1}.  With every lambda equal to c, c times these are the
  log-linear operator's gradients (checks ``backward`` without the level
  machinery).
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


def mamba2_backward(q, k, v, log_a, dout):
    """Gradients (dq, dk, dv, dlog_a) of sum(dout * mamba2(...)).

    Forward states S_t = a_t S_{t-1} + k_t v_t^T (S_{-1} = 0) are kept; the
    state gradient runs backwards, dS_t = q_t dout_t^T + a_{t+1} dS_{t+1}, and
    dq_t = S_t dout_t, dk_t = dS_t v_t, dv_t = dS_t^T k_t,
    dlog_a_t = a_t <dS_t, S_{t-1}> (Frobenius product).
    """
    q, k, v, log_a, dout = (_f64(x) for x in (q, k, v, log_a, dout))
    B, H, T, dk_ = q.shape
    dv_ = v.shape[-1]
    grads = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros_like(log_a)]
    for b in range(B):
        for h in range(H):
            a = np.exp(log_a[b, h])
            states = np.zeros((T + 1, dk_, dv_))              # states[t + 1] = S_t
            for t in range(T):
                states[t + 1] = a[t] * states[t] + np.outer(k[b, h, t], v[b, h, t])
            dS = np.zeros((dk_, dv_))
            for t in range(T - 1, -1, -1):
                dS = np.outer(q[b, h, t], dout[b, h, t]) + (a[t + 1] * dS if t + 1 < T else 0.0)
                grads[0][b, h, t] = states[t + 1] @ dout[b, h, t]
                grads[1][b, h, t] = dS @ v[b, h, t]
                grads[2][b, h, t] = dS.T @ k[b, h, t]
                grads[3][b, h, t] = a[t] * np.sum(dS * states[t])
    return tuple(grads)


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
