"""Log-linear Gated DeltaNet, forward (oracle; test infrastructure only).

The pages name two instances of the log-linear framework: Log-Linear Mamba-2
and Log-Linear Gated DeltaNet, the latter being the Fenwick-bucket structure
laid over the gated delta rule ([LLA-it] Sommario tecnico section 2, item 4;
[LLA-es] Resumen tecnico section 2, "Variantes", item 2).  They print no
formula for it.  The reading used here is the plainest one the rest of the
pages support: every bucket state is a linear-attention state, the states
all follow the same per-token transition, and the output is the
lambda-weighted combination of the buckets.  For the gated delta rule that
transition is

    A_r = alpha_r (I - beta_r k_r k_r^T),   alpha_r = exp(log_a_r),

and a key enters its bucket as beta_s k_s v_s^T.  With 0-based query t and
key s:

    o_t = sum_{s<=t} lambda_t^{(l(t,s))} beta_s (q_t^T Phi(t,s) k_s) v_s,
    Phi(t,s) = A_t A_{t-1} ... A_{s+1}   (the identity when s = t),

with l(t,s) the same Fenwick level as in the Mamba-2 form.  Replacing A_r by
the scalar a_r and beta by 1 gives that form back.

Two independent evaluations:

* ``gdn_forward_quadratic`` -- the definition: each query vector is carried
  backwards through the transitions (y <- A_s y, A_s symmetric) and dotted
  with every key in turn; O(T^2 d) per head.
* ``gdn_forward_recurrent`` -- one state per Fenwick level, every stored state
  multiplied by A_t on each token, the binary-counter carry of the Mamba-2
  recurrence for the merges; O(T log T d^2) per head.

Special-case references that use neither:

* ``gated_deltanet`` -- the textbook gated delta rule S_t = A_t S_{t-1} +
  beta_t k_t v_t^T, o_t = S_t^T q_t; with every lambda equal to c the
  log-linear operator is c times it.
* ``gdn_brute_force`` -- pure-Python loops with Phi(t,s) built as an explicit
  matrix product and buckets from the Fenwick walk (tiny T).

Pins (tests/test_oracle_deltanet.py): quadratic == recurrence (1e-12); both ==
brute force (T <= 12); lambda = c -> c * gated_deltanet; beta = 0 -> 0;
mutually orthogonal keys -> the log-linear Mamba-2 oracle with values
beta v (the delta term then never touches another key); every key the same
unit vector u -> the log-linear Mamba-2 oracle with gates a_r (1 - beta_r)
and values beta v; lambda on level 0 only -> beta_t (q_t . k_t) v_t; a split
recurrence equals one run; planted mistakes fail.
"""

from __future__ import annotations

import numpy as np

from . import levels as _levels
from .forms import _f64
from .levels import walk_buckets


def gdn_forward_quadratic(q, k, v, log_a, beta, lam, rows=None):
    """The definition, per (batch, head); [B, H, R, dv].

    q, k: [B, H, T, dk]; v: [B, H, T, dv]; log_a, beta: [B, H, T];
    lam: [B, H, T, L] with L >= ceil(log2 T) + 1.  ``rows`` (optional) lists
    the query indices to evaluate, the same for every head.

    For every query t the vector y = Phi(t,s)^T q_t is kept while s runs from
    t down to 0: y starts at q_t, key s contributes
    lambda_t^{(l(t,s))} beta_s (y . k_s) v_s, and then y <- A_s y before the
    next older key.
    """
    q, k, v, log_a, beta, lam = (_f64(x) for x in (q, k, v, log_a, beta, lam))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    if lam.shape[-1] < _levels.num_levels(T):
        raise ValueError("lambda has too few levels for this T")
    tq = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    R = len(tq)
    BH = B * H
    q = q.reshape(BH, T, dk)
    k = k.reshape(BH, T, dk)
    v = v.reshape(BH, T, dv)
    alpha = np.exp(log_a.reshape(BH, T))
    beta = beta.reshape(BH, T)
    lam = lam.reshape(BH, T, lam.shape[-1])
    lev = _levels.level_table(T, rows=tq).astype(np.int64) if R else np.zeros((0, T), np.int64)
    out = np.zeros((BH, R, dv))
    y = np.zeros((BH, R, dk))
    for s in range(T - 1, -1, -1):
        start = tq == s
        if start.any():
            y[:, start] = q[:, s][:, None, :]
        live = tq >= s
        if not live.any():
            continue
        yl = y[:, live]                                          # [BH, R', dk]
        dots = np.einsum("brd,bd->br", yl, k[:, s])              # y . k_s
        lv = lev[live, s]                                        # levels of key s
        w = lam[:, tq[live], lv] * beta[:, s][:, None] * dots    # [BH, R']
        out[:, live] += w[..., None] * v[:, s][:, None, :]
        # carry the query vectors past key s: y <- alpha_s (y - beta_s (y . k_s) k_s)
        y[:, live] = alpha[:, s][:, None, None] * (
            yl - (beta[:, s][:, None] * dots)[..., None] * k[:, s][:, None, :])
    return out.reshape(B, H, R, dv)


class GdnState:
    """One d_k x d_v state per Fenwick level for a batch of heads.

    ``slots[:, l]`` is the bucket of level l (l >= 1) as seen by the next
    query ``t``: sum over its keys s of Phi(t-1, s) beta_s k_s v_s^T.  Slot 0
    is unused; empty buckets are zero.
    """

    def __init__(self, BH: int, dk: int, dv: int, nlev: int, t: int = 0):
        self.t = t
        self.slots = np.zeros((BH, nlev + 1, dk, dv))


def gdn_recurrent_step(st: GdnState, q_t, k_t, v_t, a_t, beta_t, lam_t) -> np.ndarray:
    """One token for every head: q_t, k_t [BH, dk]; v_t [BH, dv];
    a_t, beta_t [BH]; lam_t [BH, >= levels used].  Returns o_t [BH, dv].

    1. every stored bucket S becomes A_t S = a_t (S - beta_t k_t (k_t^T S));
    2. o_t = lam^0 beta_t (q_t . k_t) v_t + sum over stored levels l of
       lam^l S_l^T q_t;
    3. the binary-counter carry: with k* the trailing ones of t, the token's
       beta_t k_t v_t^T and levels 1..k* merge into level k* + 1.
    """
    t = st.t
    act = [lv for lv in _levels.active_levels(t) if lv >= 1]
    if act and max(act) >= st.slots.shape[1]:
        raise ValueError("state has too few levels")
    for lv in act:
        S = st.slots[:, lv]
        kS = np.einsum("bi,bij->bj", k_t, S)
        st.slots[:, lv] = a_t[:, None, None] * (S - beta_t[:, None, None] * np.einsum("bi,bj->bij", k_t, kS))
    o = (lam_t[:, 0] * beta_t * np.einsum("bi,bi->b", q_t, k_t))[:, None] * v_t
    for lv in act:
        o += lam_t[:, lv][:, None] * np.einsum("bij,bi->bj", st.slots[:, lv], q_t)
    kstar = ((t + 1) & -(t + 1)).bit_length() - 1
    if kstar + 1 >= st.slots.shape[1]:
        raise ValueError("state has too few levels for the merge")
    merged = beta_t[:, None, None] * np.einsum("bi,bj->bij", k_t, v_t)
    for lv in range(1, kstar + 1):
        merged += st.slots[:, lv]
        st.slots[:, lv] = 0.0
    st.slots[:, kstar + 1] = merged
    st.t = t + 1
    return o


def gdn_forward_recurrent(q, k, v, log_a, beta, lam, state: GdnState | None = None,
                          nlev: int | None = None):
    """Token-by-token recurrence over [B, H, T, ...] inputs.

    Returns (O [B, H, T, dv], final GdnState over B*H heads).
    """
    q, k, v, log_a, beta, lam = (_f64(x) for x in (q, k, v, log_a, beta, lam))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    BH = B * H
    q, k, v = q.reshape(BH, T, dk), k.reshape(BH, T, dk), v.reshape(BH, T, dv)
    a = np.exp(log_a.reshape(BH, T))
    beta = beta.reshape(BH, T)
    lam = lam.reshape(BH, T, lam.shape[-1])
    if state is None:
        state = GdnState(BH, dk, dv, nlev if nlev is not None else T.bit_length() + 1)
    out = np.zeros((BH, T, dv))
    for i in range(T):
        out[:, i] = gdn_recurrent_step(state, q[:, i], k[:, i], v[:, i], a[:, i], beta[:, i], lam[:, i])
    return out.reshape(B, H, T, dv), state


def gated_deltanet(q, k, v, log_a, beta):
    """The gated delta rule without buckets: S_t = a_t (I - beta_t k_t k_t^T)
    S_{t-1} + beta_t k_t v_t^T, o_t = S_t^T q_t; [B, H, T, dv]."""
    q, k, v, log_a, beta = (_f64(x) for x in (q, k, v, log_a, beta))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    out = np.zeros((B, H, T, dv))
    eye = np.eye(dk)
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv))
            for t in range(T):
                kt = k[b, h, t]
                A = np.exp(log_a[b, h, t]) * (eye - beta[b, h, t] * np.outer(kt, kt))
                S = A @ S + beta[b, h, t] * np.outer(kt, v[b, h, t])
                out[b, h, t] = S.T @ q[b, h, t]
    return out


def gdn_brute_force(q, k, v, a, beta, lam):
    """Pure-Python evaluation for tiny inputs: q, k [T, dk]; v [T, dv];
    a, beta [T]; lam [T, L].  Phi(t,s) is formed as a matrix product."""
    q, k, v, a, beta, lam = (_f64(x) for x in (q, k, v, a, beta, lam))
    T, dk = q.shape
    dv = v.shape[1]
    out = np.zeros((T, dv))
    for t in range(T):
        for lev, lo, hi in walk_buckets(t):
            for s in range(lo, hi):
                phi = np.eye(dk)
                for r in range(s + 1, t + 1):       # Phi = A_t ... A_{s+1}
                    A = a[r] * (np.eye(dk) - beta[r] * np.outer(k[r], k[r]))
                    phi = A @ phi
                coeff = 0.0
                pk = phi @ k[s]
                for i in range(dk):
                    coeff += q[t, i] * pk[i]
                for j in range(dv):
                    out[t, j] += lam[t, lev] * beta[s] * coeff * v[s, j]
    return out
