"""Pins of the log-linear Gated DeltaNet oracle (CPU only).

Every check ties ``oracle.deltanet`` to something other than itself: the two
forms against each other and against a pure-Python brute force with explicit
matrix products, reductions to the textbook gated delta rule and to the
(separately pinned) log-linear Mamba-2 oracle, and closed forms.
"""

import numpy as np
import pytest
import torch

from oracle import deltanet as dn
from oracle import forms, levels
from oracle.metrics import rel_l2
from fenwick_tree_hierarchical_amd.workloads import WORKLOADS, make_beta, make_inputs


def _inputs(T, d=8, B=1, H=2, seed=0, variant=None):
    w = WORKLOADS["tiny_f32"]
    x = make_inputs(w, B=B, H=H, T=T, d=d, seed=seed, variant=variant)
    beta = make_beta(w, B=B, H=H, T=T, seed=seed)
    return {k: v.double().numpy() for k, v in x.items()}, beta.double().numpy()


@pytest.mark.parametrize("T", [1, 2, 7, 16, 37, 64])
def test_quadratic_equals_recurrence(T):
    x, beta = _inputs(T, variant="weak_decay")
    oq = dn.gdn_forward_quadratic(x["q"], x["k"], x["v"], x["log_a"], beta, x["lam"])
    orr, _ = dn.gdn_forward_recurrent(x["q"], x["k"], x["v"], x["log_a"], beta, x["lam"])
    assert rel_l2(oq, orr) < 1e-12


@pytest.mark.parametrize("T", [1, 3, 5, 12])
def test_brute_force(T):
    x, beta = _inputs(T, d=4, H=1, seed=3)
    ob = dn.gdn_brute_force(x["q"][0, 0], x["k"][0, 0], x["v"][0, 0], np.exp(x["log_a"][0, 0]),
                            beta[0, 0], x["lam"][0, 0])
    oq = dn.gdn_forward_quadratic(x["q"], x["k"], x["v"], x["log_a"], beta, x["lam"])[0, 0]
    orr = dn.gdn_forward_recurrent(x["q"], x["k"], x["v"], x["log_a"], beta, x["lam"])[0][0, 0]
    assert rel_l2(oq, ob) < 1e-12
    assert rel_l2(orr, ob) < 1e-12


def test_constant_lambda_is_gated_deltanet():
    x, beta = _inputs(50, variant="weak_decay+const:1.7")
    o = dn.gdn_forward_quadratic(x["q"], x["k"], x["v"], x["log_a"], beta, x["lam"])
    ref = dn.gated_deltanet(x["q"], x["k"], x["v"], x["log_a"], beta)
    c = x["lam"].flat[0]            # 1.7 rounded to float32
    assert rel_l2(o, c * ref) < 1e-12


def test_gated_deltanet_textbook_values():
    """Two tokens, hand-computed: S_1 = a_1 (I - b_1 k_1 k_1^T) b_0 k_0 v_0^T + b_1 k_1 v_1^T."""
    k = np.array([[1.0, 0.0], [np.sqrt(0.5), np.sqrt(0.5)]])
    q = np.array([[0.0, 1.0], [1.0, 2.0]])
    v = np.array([[3.0], [5.0]])
    a = np.array([1.0, 0.5])
    b = np.array([0.5, 0.25])
    ref = np.zeros((2, 1))
    ref[0] = b[0] * (q[0] @ k[0]) * v[0]                   # = 0
    # (I - b1 k1 k1^T) k0 = (1 - 0.125, -0.125); a1 * b0 * q1 . that = 0.5*0.5*(0.875 - 0.25)
    ref[1] = a[1] * b[0] * (q[1] @ (k[0] - b[1] * (k[1] @ k[0]) * k[1])) * v[0] + b[1] * (q[1] @ k[1]) * v[1]
    assert abs(ref[1, 0] - (0.25 * 0.625 * 3.0 + 0.25 * 3 * np.sqrt(0.5) * 5.0)) < 1e-12
    t = lambda z: z[None, None]  # noqa: E731
    got = dn.gated_deltanet(t(q), t(k), t(v), t(np.log(a)), t(b))[0, 0]
    assert np.allclose(got, ref, atol=1e-14)


def test_beta_zero_is_zero():
    x, beta = _inputs(40)
    o = dn.gdn_forward_quadratic(x["q"], x["k"], x["v"], x["log_a"], 0 * beta, x["lam"])
    assert np.abs(o).max() == 0.0


def test_level_zero_only():
    x, beta = _inputs(33, variant="onehot:0")
    o = dn.gdn_forward_recurrent(x["q"], x["k"], x["v"], x["log_a"], beta, x["lam"])[0]
    ref = (beta * np.einsum("bhtd,bhtd->bht", x["q"], x["k"]))[..., None] * x["v"]
    assert rel_l2(o, ref) < 1e-13


def test_orthogonal_keys_reduce_to_mamba2_form():
    """Keys from one orthonormal basis: (I - b k_r k_r^T) k_s = k_s for r != s,
    so the operator is the log-linear Mamba-2 form with values beta v."""
    T = d = 16
    x, beta = _inputs(T, d=d, H=2, seed=5, variant="weak_decay")
    rng = np.random.default_rng(0)
    for h in range(2):
        Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
        x["k"][0, h] = Qm[rng.permutation(d)]
    o = dn.gdn_forward_quadratic(x["q"], x["k"], x["v"], x["log_a"], beta, x["lam"])
    ref = forms.forward_quadratic(x["q"], x["k"], beta[..., None] * x["v"], x["log_a"], x["lam"])
    assert rel_l2(o, ref) < 1e-12


def test_one_key_direction_reduces_to_mamba2_form():
    """Every key the same unit vector u: A_r u = a_r (1 - beta_r) u, so the
    gates become a_r (1 - beta_r) and the values beta v."""
    x, beta = _inputs(45, d=8, seed=6, variant="weak_decay")
    u = np.random.default_rng(1).standard_normal(8)
    u /= np.linalg.norm(u)
    x["k"][:] = u
    o = dn.gdn_forward_recurrent(x["q"], x["k"], x["v"], x["log_a"], beta, x["lam"])[0]
    ref = forms.forward_quadratic(x["q"], x["k"], beta[..., None] * x["v"],
                                  x["log_a"] + np.log1p(-beta), x["lam"])
    assert rel_l2(o, ref) < 1e-12


def test_sampled_rows_match_full():
    x, beta = _inputs(70, seed=2)
    rows = np.array([0, 5, 31, 32, 69])
    full = dn.gdn_forward_quadratic(x["q"], x["k"], x["v"], x["log_a"], beta, x["lam"])
    part = dn.gdn_forward_quadratic(x["q"], x["k"], x["v"], x["log_a"], beta, x["lam"], rows=rows)
    assert np.array_equal(part, full[:, :, rows])


def test_split_recurrence_equals_one_run():
    x, beta = _inputs(48, seed=4)
    full, st = dn.gdn_forward_recurrent(x["q"], x["k"], x["v"], x["log_a"], beta, x["lam"], nlev=7)
    cut = 29
    sl = lambda z: z[:, :, :cut]   # noqa: E731
    sr = lambda z: z[:, :, cut:]   # noqa: E731
    o1, st1 = dn.gdn_forward_recurrent(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["log_a"]), sl(beta),
                                       sl(x["lam"]), nlev=7)
    o2, st2 = dn.gdn_forward_recurrent(sr(x["q"]), sr(x["k"]), sr(x["v"]), sr(x["log_a"]), sr(beta),
                                       sr(x["lam"]), state=st1)
    assert np.allclose(np.concatenate([o1, o2], axis=2), full, rtol=0, atol=1e-13)
    assert np.allclose(st2.slots, st.slots, rtol=0, atol=1e-13)


def test_bucket_state_is_its_definition():
    """Each recurrent slot equals sum over its bucket of Phi(t-1, s) beta_s k_s v_s^T."""
    T, d = 23, 4
    x, beta = _inputs(T, d=d, H=1, seed=8, variant="weak_decay")
    _, st = dn.gdn_forward_recurrent(x["q"], x["k"], x["v"], x["log_a"], beta, x["lam"], nlev=6)
    k, v, a, b = x["k"][0, 0], x["v"][0, 0], np.exp(x["log_a"][0, 0]), beta[0, 0]
    t = T   # next query
    for lev, lo, hi in levels.walk_buckets(t):
        if lev == 0:
            continue
        ref = np.zeros((d, d))
        for s in range(lo, hi):
            phi = np.eye(d)
            for r in range(s + 1, t):
                phi = a[r] * (np.eye(d) - b[r] * np.outer(k[r], k[r])) @ phi
            ref += b[s] * np.outer(phi @ k[s], v[s])
        assert np.allclose(st.slots[0, lev], ref, rtol=0, atol=1e-13)


# Planted mistakes: each variant of the quadratic form must fail a pin above.
def _mutant_quadratic(q, k, v, log_a, beta, lam, mistake):
    T = q.shape[0]
    out = np.zeros_like(v)
    a = np.exp(log_a)
    for t in range(T):
        for lev, lo, hi in levels.walk_buckets(t):
            for s in range(lo, hi):
                phi = np.eye(q.shape[1])
                rng = range(s + 1, t + 1) if mistake != "own_transition" else range(s, t + 1)
                for r in rng:
                    sign = -1.0 if mistake != "delta_sign" else 1.0
                    A = a[r] * (np.eye(q.shape[1]) + sign * beta[r] * np.outer(k[r], k[r]))
                    phi = (phi @ A) if mistake == "reversed_order" else (A @ phi)
                bs = beta[t] if mistake == "beta_of_query" else beta[s]
                out[t] += lam[t, lev] * bs * (q[t] @ phi @ k[s]) * v[s]
    return out


@pytest.mark.parametrize("mistake", ["own_transition", "delta_sign", "reversed_order", "beta_of_query"])
def test_planted_mistakes_fail(mistake):
    """A mistake in the definition fails the textbook gated delta rule pin
    (lambda constant), which is written without buckets or Phi products."""
    T, d = 9, 4
    x, beta = _inputs(T, d=d, H=1, seed=11, variant="weak_decay+const:1.0")
    args = (x["q"][0, 0], x["k"][0, 0], x["v"][0, 0], x["log_a"][0, 0], beta[0, 0], x["lam"][0, 0])
    ref = dn.gated_deltanet(x["q"], x["k"], x["v"], x["log_a"], beta)[0, 0]
    assert rel_l2(_mutant_quadratic(*args, mistake="none"), ref) < 1e-12
    assert rel_l2(_mutant_quadratic(*args, mistake=mistake), ref) > 1e-3


def test_beta_distribution():
    b = make_beta(WORKLOADS["small_bf16"], T=4096, H=2, B=1)
    assert b.dtype == torch.float32 and b.shape == (1, 2, 4096)
    assert float(b.min()) > 0.0 and float(b.max()) < 1.0
    assert abs(float(b.mean()) - 0.5) < 0.02
