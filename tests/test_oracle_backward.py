"""Pins for the oracle's gradients (CPU only).

Each pin compares ``oracle.backward`` with something other than its own
formulas: finite differences of the forward oracle (both forms), identities
that hold for any correct gradient of this operator, and closed forms of
special cases written without the level machinery.
"""

import numpy as np
import pytest
import torch

from fenwick_tree_hierarchical_amd.workloads import WORKLOADS, make_grad_out, make_inputs
from oracle import backward, forms, levels, metrics, special

TINY = WORKLOADS["tiny_f32"]
NAMES = ("q", "k", "v", "log_a", "lam")


def _inp(T, B=1, H=2, d=3, variant=None, seed=5):
    x = make_inputs(TINY, B=B, H=H, T=T, variant=variant, seed=seed)
    g = torch.Generator().manual_seed(seed + 200)
    for name in ("q", "k", "v"):
        x[name] = torch.randn(B, H, T, d, generator=g)
    x = {k: v.double().numpy() for k, v in x.items()}
    x["dout"] = make_grad_out(TINY, B=B, H=H, T=T, seed=seed, d=d).double().numpy()
    return x


def _grads(x):
    return dict(zip(NAMES, backward.backward_quadratic(x["q"], x["k"], x["v"], x["log_a"], x["lam"], x["dout"])))


def _loss_quadratic(x):
    return backward.loss(forms.forward_quadratic(x["q"], x["k"], x["v"], x["log_a"], x["lam"]), x["dout"])


def _loss_recurrent(x):
    o, _ = forms.forward_recurrent(x["q"], x["k"], x["v"], x["lam"], log_a=x["log_a"])
    return backward.loss(o, x["dout"])


def _fd_entry(fn, x, name, idx, h=1e-6):
    xp = {k: v.copy() for k, v in x.items()}
    xm = {k: v.copy() for k, v in x.items()}
    xp[name][idx] += h
    xm[name][idx] -= h
    return (fn(xp) - fn(xm)) / (2 * h)


@pytest.mark.parametrize("T", [1, 6, 11])
@pytest.mark.parametrize("name", NAMES)
def test_every_entry_against_finite_differences(T, name):
    """Each gradient entry against a central difference of the quadratic form."""
    x = _inp(T)
    g = _grads(x)[name]
    fd = np.zeros_like(g)
    for idx in np.ndindex(*x[name].shape):
        fd[idx] = _fd_entry(_loss_quadratic, x, name, idx)
    assert np.allclose(g, fd, rtol=1e-6, atol=1e-8), np.abs(g - fd).max()


@pytest.mark.parametrize("name", NAMES)
def test_directional_derivative_of_recurrent_form(name):
    """A random direction through the Fenwick-state recurrence (the other
    form), at a length where buckets of five levels occur."""
    x = _inp(37, H=1, d=4, seed=9)
    g = _grads(x)[name]
    u = np.random.default_rng(3).standard_normal(x[name].shape)
    h = 1e-6
    xp = {k: v.copy() for k, v in x.items()}
    xm = {k: v.copy() for k, v in x.items()}
    xp[name] += h * u
    xm[name] -= h * u
    fd = (_loss_recurrent(xp) - _loss_recurrent(xm)) / (2 * h)
    assert abs(fd - np.sum(g * u)) <= 1e-6 * max(1.0, abs(fd))


def test_homogeneity_identities():
    """o_t is linear in q_t and in the lambda row of t; the loss is linear in
    k and in v.  So q_t . dq_t = sum_l lambda_t^l dlambda_t^l = dout_t . o_t
    for every t, and sum_s k_s . dk_s = sum_s v_s . dv_s = the loss."""
    x = _inp(100, H=2, d=5, seed=2)
    g = _grads(x)
    o = forms.forward_quadratic(x["q"], x["k"], x["v"], x["log_a"], x["lam"])
    row = np.sum(x["dout"] * o, axis=-1)
    assert np.allclose(np.sum(x["q"] * g["q"], axis=-1), row, rtol=1e-10, atol=1e-12)
    assert np.allclose(np.sum(x["lam"] * g["lam"], axis=-1), row, rtol=1e-10, atol=1e-12)
    tot = np.sum(row, axis=-1)
    assert np.allclose(np.sum(x["k"] * g["k"], axis=(-1, -2)), tot, rtol=1e-10)
    assert np.allclose(np.sum(x["v"] * g["v"], axis=(-1, -2)), tot, rtol=1e-10)


def test_first_gate_and_empty_levels_have_zero_gradient():
    """a_0 multiplies nothing (every gate product starts after the key), and a
    level whose bucket is empty for query t has no key to weight."""
    x = _inp(77, H=2, d=3, seed=4)
    g = _grads(x)
    scale = np.abs(g["log_a"]).max()
    assert np.all(np.abs(g["log_a"][..., 0]) <= 1e-12 * scale)
    lam_g = g["lam"]
    for t in range(77):
        occupied = set(levels.active_levels(t))
        for lv in range(lam_g.shape[-1]):
            if lv not in occupied:
                assert np.all(lam_g[..., t, lv] == 0.0), (t, lv)
            elif lv > 0:
                assert np.all(lam_g[..., t, lv] != 0.0), (t, lv)


def test_level_zero_only_closed_form():
    """lambda nonzero on level 0 only: o_t = lambda0_t (q_t . k_t) v_t."""
    x = _inp(19, H=2, d=4, seed=6)
    x["lam"][..., 1:] = 0.0
    g = _grads(x)
    l0 = x["lam"][..., 0]
    qk = np.sum(x["q"] * x["k"], axis=-1)
    dov = np.sum(x["dout"] * x["v"], axis=-1)
    assert np.allclose(g["q"], (l0 * dov)[..., None] * x["k"], rtol=1e-12, atol=1e-14)
    assert np.allclose(g["k"], (l0 * dov)[..., None] * x["q"], rtol=1e-12, atol=1e-14)
    assert np.allclose(g["v"], (l0 * qk)[..., None] * x["dout"], rtol=1e-12, atol=1e-14)
    assert np.allclose(g["lam"][..., 0], qk * dov, rtol=1e-12, atol=1e-14)
    assert np.allclose(g["log_a"], 0.0, atol=1e-13)


@pytest.mark.parametrize("c", [1.0, 0.3])
def test_constant_lambda_is_mamba2_adjoint(c):
    """lambda = c everywhere: c times the gradients of the Mamba-2
    recurrence, computed by its adjoint recurrence backwards in time; the
    lambda gradients of each row add up to dout_t . mamba2_t."""
    x = _inp(45, H=2, d=4, variant=f"const:{c}", seed=8)
    g = _grads(x)
    c = float(x["lam"].flat[0])                  # the float32 value lambda holds
    ref = special.mamba2_backward(x["q"], x["k"], x["v"], x["log_a"], x["dout"])
    for name, r in zip(("q", "k", "v", "log_a"), ref):
        assert metrics.rel_l2(g[name], c * r) < 1e-12, name
    m2 = special.mamba2(x["q"], x["k"], x["v"], x["log_a"])
    assert np.allclose(g["lam"].sum(axis=-1), np.sum(x["dout"] * m2, axis=-1), rtol=1e-10, atol=1e-12)


def test_row_blocks_do_not_change_the_result():
    """The key-side sums accumulate over query row blocks."""
    x = _inp(70, H=1, d=3, seed=1)
    a = backward.backward_quadratic(x["q"], x["k"], x["v"], x["log_a"], x["lam"], x["dout"])
    b = backward.backward_quadratic(x["q"], x["k"], x["v"], x["log_a"], x["lam"], x["dout"], block=16)
    for u, w in zip(a, b):
        assert np.allclose(u, w, rtol=1e-12, atol=1e-13)


def test_sampled_rows_equal_the_full_gradients():
    x = _inp(300, H=2, d=4, seed=12)
    g = _grads(x)
    rows = np.array([0, 1, 5, 63, 64, 128, 200, 255, 298, 299])
    smp = backward.backward_sampled(x["q"], x["k"], x["v"], x["log_a"], x["lam"], x["dout"], rows)
    for name, full in (("dq", g["q"]), ("dk", g["k"]), ("dv", g["v"]), ("dlam", g["lam"])):
        assert np.allclose(smp[name], full[:, :, rows], rtol=1e-11, atol=1e-13), name


@pytest.mark.parametrize("T", [1, 9, 37, 64])
def test_gate_gradient_rows_equal_the_full_gradient(T):
    """dlog_a_rows (pairs straddling r, through the recurrence with the later
    keys removed) equals backward_quadratic's reverse sum at every position."""
    x = make_inputs(WORKLOADS["small_bf16"], B=1, H=2, T=T, d=8, dtype="f32", variant="weak_decay", seed=40 + T)
    dout = make_grad_out(WORKLOADS["small_bf16"], B=1, H=2, T=T, d=8, dtype="f32", seed=40 + T)
    ref = backward.backward_quadratic(x["q"], x["k"], x["v"], x["log_a"], x["lam"], dout)[3]
    got = backward.dlog_a_rows(x["q"], x["k"], x["v"], x["log_a"], x["lam"], dout, np.arange(T))
    scale = np.abs(ref).max() + 1e-30
    assert np.max(np.abs(got - ref)) <= 1e-12 * max(scale, 1.0)
