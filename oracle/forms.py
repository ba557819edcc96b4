"""The two independent forms of the operator (oracle; test infrastructure only).

Both consume float64 copies of exactly the values the GPU receives.

* ``forward_quadratic`` -- the masked quadratic form O = (Q K^T . M^S . M^H) V,
  evaluated row block by row block.  It is the plain definition: the parallel
  form of [LLA-it] Sommario tecnico section 2, item 3 ("Training") and
  [LLA-es] Resumen tecnico section 2, "Forma paralela", without any chunking.
* ``forward_recurrent`` -- the token-by-token recurrence over one state per
  Fenwick level ([LLA-it] section 2, item 3, "Decoding": O(log T) separate
  recurrent states, the output a weighted combination of them; the lay part
  "L'essenziale", box metaphor: on each token only the smallest box is
  updated and, when needed, merged into the bigger boxes).  The state that
  comes out of it is the decode reference.

Pins (tests/test_oracle_forms.py): the two forms agree to 1e-12; both agree
with ``special.brute_force`` (pure-Python loops, explicit product of the
gates, buckets from the Fenwick walk) for T <= 16; lambda constant reduces to
the Mamba-2 recurrence; log_a = 0 and lambda = 1 reduce to causal linear
attention; lambda on level 0 only gives the diagonal term; closed forms for
scalar inputs (geometric series, 1 + popcount(t)/2).
"""

from __future__ import annotations

import numpy as np

from . import levels as _levels


def _f64(x) -> np.ndarray:
    """float64 numpy copy of a numpy array or (CPU) torch tensor."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        if str(x.dtype) not in ("torch.float64",):
            x = x.double()
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


def decay_matrix(log_a: np.ndarray, rows: np.ndarray | None = None) -> np.ndarray:
    """M^S for one sequence: exp(Lambda_t - Lambda_s) for s <= t, else 0.

    Lambda is the inclusive cumulative sum of log_a in float64, so
    Lambda_t - Lambda_s = sum_{s<r<=t} log_a_r and M^S[t, t] = 1.
    ``rows`` restricts the query indices.
    """
    la = _f64(log_a)
    T = la.shape[-1]
    lam_cum = np.cumsum(la)
    t = np.arange(T) if rows is None else np.asarray(rows)
    s = np.arange(T)
    causal = s[None, :] <= t[:, None]
    diff = np.where(causal, lam_cum[t][:, None] - lam_cum[None, :], -np.inf)
    return np.exp(diff)


def decay_matrix_product(a: np.ndarray) -> np.ndarray:
    """M^S for one sequence as the explicit product prod_{s<r<=t} a_r
    (third derivation, for tiny T)."""
    a = _f64(a)
    T = a.shape[-1]
    m = np.zeros((T, T))
    for t in range(T):
        for s in range(t + 1):
            p = 1.0
            for r in range(s + 1, t + 1):
                p *= a[r]
            m[t, s] = p
    return m


def forward_quadratic(q, k, v, log_a, lam, rows=None, chunk=None, pair=None, block=1024):
    """Masked quadratic form, per (batch, head).

    q, k: [B, H, T, dk]; v: [B, H, T, dv]; log_a: [B, H, T];
    lam: [B, H, T, L] with L >= ceil(log2 T) + 1.
    ``rows``: optional 1-D array of query indices (same for every head);
    the result then has shape [B, H, len(rows), dv].
    ``pair``: None, "intra" or "inter" keeps only key/query pairs in the same
    (different) chunk of size ``chunk``; used to isolate parts of the GPU path.
    """
    q, k, v, log_a, lam = (_f64(x) for x in (q, k, v, log_a, lam))
    B, H, T, _ = q.shape
    dv = v.shape[-1]
    L = lam.shape[-1]
    if L < _levels.num_levels(T):
        raise ValueError("lambda has too few levels for this T")
    r_all = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((B, H, len(r_all), dv))
    s_idx = np.arange(T)
    for b in range(B):
        for h in range(H):
            for lo in range(0, len(r_all), block):
                tq = r_all[lo:lo + block]
                scores = q[b, h, tq] @ k[b, h].T                      # [R, T]
                ms = decay_matrix(log_a[b, h], rows=tq)               # [R, T]
                lev = _levels.level_table(T, rows=tq).astype(np.int64)
                causal = lev >= 0
                mh = np.take_along_axis(lam[b, h, tq], np.where(causal, lev, 0), axis=1)
                mh = np.where(causal, mh, 0.0)
                if pair is not None:
                    same = (tq[:, None] // chunk) == (s_idx[None, :] // chunk)
                    mh = mh * (same if pair == "intra" else ~same)
                out[b, h, lo:lo + len(tq)] = (scores * ms * mh) @ v[b, h]
    return out


class FenwickState:
    """Recurrent state of one batch of heads: one d_k x d_v matrix per level.

    ``slots[:, l]`` holds the bucket at level l (l >= 1) as seen by the next
    query ``t``, already decayed up to token t-1; slot 0 is unused (level 0 is
    the query token itself and is never stored).  Empty buckets are zero.
    """

    def __init__(self, BH: int, dk: int, dv: int, nlev: int, t: int = 0):
        self.t = t
        self.slots = np.zeros((BH, nlev + 1, dk, dv))

    def copy(self) -> "FenwickState":
        c = FenwickState(1, 1, 1, 0)
        c.t = self.t
        c.slots = self.slots.copy()
        return c


def recurrent_step(st: FenwickState, q_t, k_t, v_t, a_t, lam_t) -> np.ndarray:
    """One token of the recurrence for every head at once.

    q_t, k_t: [BH, dk]; v_t: [BH, dv]; a_t: [BH] gate a_t = exp(log_a_t);
    lam_t: [BH, >= levels used].  Returns o_t [BH, dv] and advances ``st``.

    1. every stored bucket is decayed by a_t (the gate of the new token
       applies to all older keys, never to the token itself);
    2. o_t = lam^0 (q_t . k_t) v_t + sum over stored levels l of
       lam^l * S_l^T q_t;
    3. binary-counter carry: with k* the number of trailing ones of t, the
       token and the buckets of levels 1..k* merge into the bucket of level
       k* + 1 and levels 1..k* become empty.
    """
    t = st.t
    act = [lv for lv in _levels.active_levels(t) if lv >= 1]
    if act and max(act) >= st.slots.shape[1]:
        raise ValueError("state has too few levels")
    for lv in act:
        st.slots[:, lv] *= a_t[:, None, None]
    o = (lam_t[:, 0] * np.einsum("bi,bi->b", q_t, k_t))[:, None] * v_t
    for lv in act:
        o += lam_t[:, lv][:, None] * np.einsum("bij,bi->bj", st.slots[:, lv], q_t)
    kstar = ((t + 1) & -(t + 1)).bit_length() - 1       # trailing ones of t
    if kstar + 1 >= st.slots.shape[1]:
        raise ValueError("state has too few levels for the merge")
    merged = np.einsum("bi,bj->bij", k_t, v_t)
    for lv in range(1, kstar + 1):
        merged += st.slots[:, lv]
        st.slots[:, lv] = 0.0
    st.slots[:, kstar + 1] = merged
    st.t = t + 1
    return o


def forward_recurrent(q, k, v, lam, log_a=None, a=None, state: FenwickState | None = None,
                      nlev: int | None = None):
    """Token-by-token recurrence over [B, H, T, ...] inputs.

    Gates come from ``log_a`` (a = exp(log_a) in float64) or directly from
    ``a``.  Starts from ``state`` (positions continue at state.t) or from the
    empty state.  Returns (O [B, H, T, dv], final FenwickState over B*H heads).
    """
    q, k, v, lam = (_f64(x) for x in (q, k, v, lam))
    if a is None:
        a = np.exp(_f64(log_a))
    else:
        a = _f64(a)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    BH = B * H
    q, k, v = q.reshape(BH, T, dk), k.reshape(BH, T, dk), v.reshape(BH, T, dv)
    a, lam = a.reshape(BH, T), lam.reshape(BH, T, lam.shape[-1])
    if state is None:
        t_end = T
        state = FenwickState(BH, dk, dv, nlev if nlev is not None else t_end.bit_length() + 1)
    out = np.zeros((BH, T, dv))
    for i in range(T):
        out[:, i] = recurrent_step(state, q[:, i], k[:, i], v[:, i], a[:, i], lam[:, i])
    return out.reshape(B, H, T, dv), state
