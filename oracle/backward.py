"""Gradients of the operator (oracle; test infrastructure only).

The pages define the forward operator only; the training kernels they speak of
need its gradients, those of the level weights lambda included ("Log-Linear
Attention", Spanish summary, section 5 "Limitaciones", first item).  These are
the exact gradients of the plain definition

    o_t = sum_{s<=t} A[t,s] (q_t . k_s) v_s,   A[t,s] = lambda_t^{(l(t,s))} M^S[t,s]

for a scalar loss whose gradient with respect to O is ``dout``, written out by
the chain rule on the masked quadratic form, in float64:

    dP[t,s] = dout_t . v_s            S[t,s] = q_t . k_s
    dq_t  = sum_{s<=t} A[t,s] dP[t,s] k_s
    dk_s  = sum_{t>=s} A[t,s] dP[t,s] q_t
    dv_s  = sum_{t>=s} A[t,s] S[t,s] dout_t
    dlambda_t^{(l)} = sum_{s<=t, l(t,s)=l} M^S[t,s] S[t,s] dP[t,s]
    dLambda_u = sum_s A[u,s] S[u,s] dP[u,s] - sum_t A[t,u] S[t,u] dP[t,u]
    dlog_a_r  = sum_{u>=r} dLambda_u

where Lambda is the inclusive cumulative sum of log_a, so that
M^S[t,s] = exp(Lambda_t - Lambda_s) moves with Lambda_t (+) and Lambda_s (-).
Levels with no key (empty buckets) get a zero lambda gradient.

``backward_sampled`` evaluates the same sums at chosen query and key rows only
(long sequences); it is pinned to ``backward_quadratic``.  ``dlog_a_rows``
gives the gate gradient at chosen positions of long sequences through the
forward recurrence (see its docstring); it is pinned to ``backward_quadratic``
too.

Pins (tests/test_oracle_backward.py): every entry of every gradient against
central finite differences of the forward oracle (both of its forms) on tiny
inputs; homogeneity identities (o_t is linear in q_t and in the lambda row of
t; the loss is linear in k and in v); the gate of token 0 never enters the
operator, so its gradient is zero; empty levels get zero; lambda on level 0
only, and constant lambda (the Mamba-2 recurrence, differentiated backwards in
time) as closed forms; planted mistakes fail these pins
(tests/test_oracle_mutants.py).
"""

from __future__ import annotations

import numpy as np

from . import levels as _levels
from .forms import _f64, decay_matrix


def backward_quadratic(q, k, v, log_a, lam, dout, block=1024):
    """Gradients (dq, dk, dv, dlog_a, dlam) of sum(dout * O), per (batch, head).

    Shapes as in ``forms.forward_quadratic``; dout is [B, H, T, dv].  The query
    rows are processed ``block`` at a time; the key-side sums (dk, dv and the
    column term of dLambda) accumulate over the row blocks.
    """
    q, k, v, log_a, lam, dout = (_f64(x) for x in (q, k, v, log_a, lam, dout))
    B, H, T, dk_ = q.shape
    L = lam.shape[-1]
    if L < _levels.num_levels(T):
        raise ValueError("lambda has too few levels for this T")
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dlam = np.zeros_like(lam)
    dlog_a = np.zeros_like(log_a)
    for b in range(B):
        for h in range(H):
            row_term = np.zeros(T)
            col_term = np.zeros(T)
            for lo in range(0, T, block):
                tq = np.arange(lo, min(lo + block, T))
                S = q[b, h, tq] @ k[b, h].T                            # [R, T]
                dP = dout[b, h, tq] @ v[b, h].T                        # [R, T]
                ms = decay_matrix(log_a[b, h], rows=tq)                # 0 above the diagonal
                lev = _levels.level_table(T, rows=tq).astype(np.int64)
                causal = lev >= 0
                mh = np.take_along_axis(lam[b, h, tq], np.where(causal, lev, 0), axis=1)
                A = np.where(causal, ms * mh, 0.0)
                dq[b, h, tq] = (A * dP) @ k[b, h]
                dk[b, h] += (A * dP).T @ q[b, h, tq]
                dv[b, h] += (A * S).T @ dout[b, h, tq]
                E = np.where(causal, ms * S * dP, 0.0)                 # per pair, without lambda
                for lv in range(L):
                    dlam[b, h, tq, lv] = np.where(lev == lv, E, 0.0).sum(axis=1)
                G = A * S * dP
                row_term[tq] += G.sum(axis=1)
                col_term += G.sum(axis=0)
            dlam_u = row_term - col_term
            dlog_a[b, h] = np.cumsum(dlam_u[::-1])[::-1]
    return dq, dk, dv, dlog_a, dlam


def backward_sampled(q, k, v, log_a, lam, dout, rows):
    """The same gradients at sampled positions, for long sequences: dq and
    dlam at query rows ``rows`` (their row of the pair matrix) and dk and dv
    at key rows ``rows`` (their column: every query t >= s).  Returns a dict
    of [B, H, len(rows), ...] arrays.  The gate of a pair is
    exp(Lambda_t - Lambda_s) with Lambda the inclusive float64 cumulative sum
    of log_a, as in ``forms.decay_matrix``; the level is ``levels.level``.
    """
    q, k, v, log_a, lam, dout = (_f64(x) for x in (q, k, v, log_a, lam, dout))
    B, H, T, _ = q.shape
    L = lam.shape[-1]
    rows = np.asarray(rows, dtype=np.int64)
    R = len(rows)
    res = {"dq": np.zeros((B, H, R, q.shape[-1])), "dlam": np.zeros((B, H, R, L)),
           "dk": np.zeros((B, H, R, k.shape[-1])), "dv": np.zeros((B, H, R, v.shape[-1]))}
    for b in range(B):
        for h in range(H):
            S = q[b, h, rows] @ k[b, h].T
            dP = dout[b, h, rows] @ v[b, h].T
            ms = decay_matrix(log_a[b, h], rows=rows)
            lev = _levels.level_table(T, rows=rows).astype(np.int64)
            causal = lev >= 0
            mh = np.take_along_axis(lam[b, h, rows], np.where(causal, lev, 0), axis=1)
            A = np.where(causal, ms * mh, 0.0)
            res["dq"][b, h] = (A * dP) @ k[b, h]
            E = np.where(causal, ms * S * dP, 0.0)
            for lv in range(L):
                res["dlam"][b, h, :, lv] = np.where(lev == lv, E, 0.0).sum(axis=1)
            cum = np.cumsum(log_a[b, h])
            for i, s in enumerate(rows):
                t = np.arange(s, T)
                lv = np.array([_levels.level(int(u), int(s)) for u in t], dtype=np.int64)
                a_ts = lam[b, h, t, lv] * np.exp(cum[t] - cum[s])
                res["dk"][b, h, i] = (a_ts * (dout[b, h, t] @ v[b, h, s])) @ q[b, h, t]
                res["dv"][b, h, i] = (a_ts * (q[b, h, t] @ k[b, h, s])) @ dout[b, h, t]
    return res


def dlog_a_rows(q, k, v, log_a, lam, dout, rows):
    """The gate gradient at positions ``rows`` of long sequences; [B, H, len(rows)].

    Summing dLambda_u = sum_s G[u,s] - sum_t G[t,u] (G = A . S . dP on the
    pairs s <= t) over u >= r leaves exactly the pairs that straddle r:

        dlog_a_r = sum_{t >= r} sum_{s < r} G[t,s]
                 = sum_{t >= r} dout_t . o_t^{(<r)},

    where o^{(<r)} is the operator's output with the keys s >= r removed
    (k_s = 0 there, which zeroes their scores).  That output comes from the
    token-by-token recurrence (``forms.forward_recurrent``), so a position
    costs one O(T log T) pass instead of the O(T^2) pair matrix."""
    from .forms import forward_recurrent
    q, k, v, log_a, lam, dout = (_f64(x) for x in (q, k, v, log_a, lam, dout))
    B, H, T, _ = q.shape
    rows = np.asarray(rows, dtype=np.int64)
    res = np.zeros((B, H, len(rows)))
    for i, r in enumerate(rows):
        kr = k.copy()
        kr[:, :, r:] = 0.0
        o, _ = forward_recurrent(q, kr, v, lam, log_a=log_a)
        res[:, :, i] = np.einsum("bhtd,bhtd->bh", dout[:, :, r:], o[:, :, r:])
    return res


def loss(out, dout) -> float:
    """sum(dout * out) in float64: the scalar whose gradients are above."""
    return float(np.sum(_f64(out) * _f64(dout)))
