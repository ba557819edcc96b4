"""Backward parity: the HIP gradients against the float64 oracle (GPU).

Bars: 1e-4 for float32 inputs, 2e-2 for bfloat16 inputs, on the relative L2
of dq, dk, dv and dlambda over the whole tensor and over each (batch, head),
and five times that on each row (tests/helpers.py).  The gate gradient is a
reverse cumulative sum of differences of two terms that cancel over the
whole sequence (its first entry is exactly zero), so it is held to the same
bar relative to the reverse cumulative sum of the magnitudes of those terms,
which sets the scale its rounding errors follow.  As for the forward, every
shape class also runs with weak or no decay and with lambda one-hot on
single levels, so that distant levels carry the gradients.
"""

import numpy as np
import pytest
import torch

from fenwick_tree_hierarchical_amd.workloads import WORKLOADS, make_grad_out, make_inputs
from oracle import backward, forms
from tests.helpers import TOL, OraclePool, assert_parity, assert_scaled, heads, need_gpu, rel_l2, say, to_cpu

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dlog_a", "dlam")


def gpu_bwd(x, dout, C, dev):
    import fenwick_tree_hierarchical_amd as la
    xd = {k: v.to(dev) for k, v in x.items()}
    g = la.loglinear_bwd(xd["q"], xd["k"], xd["v"], xd["log_a"], xd["lam"], dout.to(dev), chunk=C)
    torch.cuda.synchronize()
    return {n: t.float().cpu().numpy() for n, t in zip(NAMES, g)}


def gate_scale(x, dout, ref):
    """Reverse cumulative sum of |dout_u . o_u| + |v_u . dv_u|: the size of
    the terms whose differences the gate gradient adds up."""
    o = forms.forward_quadratic(x["q"], x["k"], x["v"], x["log_a"], x["lam"])
    row = np.abs(np.sum(dout.double().numpy() * o, axis=-1))
    col = np.abs(np.sum(x["v"].double().numpy() * ref["dv"], axis=-1))
    return np.cumsum((row + col)[..., ::-1], axis=-1)[..., ::-1]


def check(x, dout, C, dtype, dev, label):
    say(f"bwd {label}: shape={tuple(x['q'].shape)} C={C} dtype={dtype}")
    got = gpu_bwd(x, dout, C, dev)
    r = backward.backward_quadratic(x["q"], x["k"], x["v"], x["log_a"], x["lam"], dout)
    ref = dict(zip(NAMES, r))
    errs = {}
    for n in ("dq", "dk", "dv", "dlam"):
        assert np.all(np.isfinite(got[n])), n
        errs[n] = assert_parity(got[n], ref[n], TOL[dtype], f"{label} {n}")["whole"]
    scale = gate_scale(x, dout, ref)
    errs["dlog_a"] = assert_scaled(got["dlog_a"][..., None], ref["dlog_a"][..., None], scale[..., None],
                                   TOL[dtype], f"{label} dlog_a")["whole"]
    # levels with an empty bucket get exactly zero
    T, L = x["lam"].shape[2], x["lam"].shape[3]
    t = np.arange(T)
    for lv in range(1, L):
        empty = ((t >> (lv - 1)) & 1) == 0
        assert np.all(got["dlam"][:, :, empty, lv] == 0.0), lv
    return errs


def case(T, d, dtype, variant=None, B=1, H=2, seed=0):
    x = make_inputs(WORKLOADS["small_bf16"], B=B, H=H, T=T, d=d, dtype=dtype, variant=variant, seed=seed)
    dout = make_grad_out(WORKLOADS["small_bf16"], B=B, H=H, T=T, d=d, dtype=dtype, seed=seed)
    return x, dout


def test_tiny_f32_workload():
    dev = need_gpu()
    w = WORKLOADS["tiny_f32"]
    x = make_inputs(w)
    check(x, make_grad_out(w), w.C, "f32", dev, "tiny_f32")


@pytest.mark.parametrize("variant", [None, "weak_decay", "no_decay"])
def test_small_bf16_shape(variant):
    dev = need_gpu()
    x, dout = case(2048, 64, "bf16", variant, B=1, H=4, seed=1)
    check(x, dout, 64, "bf16", dev, f"small_bf16 shape {variant}")


SHAPES = [(16, 16), (32, 32), (64, 64), (64, 16), (16, 64), (32, 64), (128, 32), (128, 64), (64, 32), (128, 16)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d,C", SHAPES)
def test_shapes_weak_decay_ragged(d, C, dtype):
    """Several full groups, a partial group and a ragged last chunk."""
    dev = need_gpu()
    T = 21 * C + 5
    x, dout = case(T, d, dtype, "weak_decay", seed=100 + d + C)
    check(x, dout, C, dtype, dev, f"d={d} C={C} T={T} weak_decay")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("lev", list(range(12)))
def test_onehot_level_sweep(lev, dtype):
    """lambda one-hot on level `lev` of T = 2048 with C = 64: levels 0..6 inside
    a chunk, 7..9 chunk levels inside a group, 10..11 group levels."""
    dev = need_gpu()
    x, dout = case(2048, 64, dtype, f"weak_decay+onehot:{lev}", seed=300 + lev)
    check(x, dout, 64, dtype, dev, f"onehot level {lev}")


@pytest.mark.parametrize("T,C", [(1, 16), (2, 16), (15, 16), (17, 16), (100, 64), (1000, 64), (129, 32),
                                 (64 * 8 * 4, 64), (64 * 8 * 4 + 64, 64)])
def test_short_ragged_and_power_of_two(T, C):
    dev = need_gpu()
    x, dout = case(T, 32, "f32", "weak_decay", B=2, H=3, seed=T)
    check(x, dout, C, "f32", dev, f"T={T} C={C}")


def test_chunk_size_invariance_f32():
    dev = need_gpu()
    x, dout = case(1500, 32, "f32", "weak_decay", seed=5)
    outs = {C: gpu_bwd(x, dout, C, dev) for C in (16, 32, 64)}
    for C in (32, 64):
        for n in NAMES:
            assert rel_l2(outs[C][n], outs[16][n]) <= 2 * TOL["f32"], (C, n)


def test_empty_problems():
    dev = need_gpu()
    import fenwick_tree_hierarchical_amd as la
    for B, T in [(0, 64), (1, 0)]:
        x, dout = case(T, 64, "bf16", B=B, H=2)
        xd = {k: v.to(dev) for k, v in x.items()}
        g = la.loglinear_bwd(xd["q"], xd["k"], xd["v"], xd["log_a"], xd["lam"], dout.to(dev), chunk=64)
        assert g[0].shape == (B, 2, T, 64) and g[4].shape == x["lam"].shape


def test_deterministic():
    dev = need_gpu()
    x, dout = case(1000, 64, "bf16", "weak_decay", seed=3)
    a = gpu_bwd(x, dout, 64, dev)
    b = gpu_bwd(x, dout, 64, dev)
    for n in NAMES:
        assert np.array_equal(a[n], b[n]), n


@pytest.mark.parametrize("d", [64, 32])
def test_split_key_side_matches_fused(d):
    """Lambda with levels no key reaches (L = 32, the most accepted) makes the
    fused per-chunk kernel's LDS plan too large at C = 64, so the same problem
    runs through the split pair, whose key side reads the transposed nodes the
    key-side node kernels keep for it (the fused kernel gathers them from the
    columns of R).  dq, dk, dv and the used levels of dlambda are the same bits
    as the fused run, the extra levels' gradients are zero, d log_a agrees to
    rounding (its row terms add the levels in other groups), and the run
    matches the oracle."""
    dev = need_gpu()
    T, C = 4096 + 64 * 5 + 11, 64
    x, dout = case(T, d, "bf16", "weak_decay", seed=5)
    L0 = x["lam"].shape[-1]
    a = gpu_bwd(x, dout, C, dev)
    g = torch.Generator().manual_seed(6)
    extra = torch.rand(*x["lam"].shape[:-1], 32 - L0, generator=g, dtype=x["lam"].dtype) + 0.5
    x32 = dict(x, lam=torch.cat([x["lam"], extra], dim=-1).contiguous())
    b = gpu_bwd(x32, dout, C, dev)
    for n in ("dq", "dk", "dv"):
        assert np.array_equal(a[n], b[n]), n
    assert np.array_equal(a["dlam"], b["dlam"][..., :L0])
    assert np.all(b["dlam"][..., L0:] == 0.0)
    scale = np.abs(a["dlog_a"]).max()
    assert np.allclose(a["dlog_a"], b["dlog_a"], rtol=1e-5, atol=1e-6 * scale)
    check(x32, dout, C, "bf16", dev, f"split key side d={d} L=32")


@pytest.mark.parametrize("d, C, T", [(64, 64, 4096 + 64 * 5 + 11), (64, 32, 4096 + 64 * 5 + 11),
                                     (32, 64, 4096 + 64 * 5 + 11), (16, 32, 4096 + 64 * 5 + 11),
                                     (128, 64, 4096 + 64 * 5 + 11), (64, 64, 64), (64, 64, 65), (64, 32, 700)])
def test_backward_from_forward_workspace(d, C, T):
    """loglinear_bwd_from_fwd: the backward reading the forward's bucket
    nodes (their transposes serve the query side) instead of building the
    structure over (v, k); full groups and a ragged tail, one exact chunk, a
    second chunk of one token (no node at all), a few chunks (no full group).  dk and dv come from the key side alone, so they
    are the plain backward's bits; dq, dlambda and dlog_a go through the
    forward's nodes (rounded with the other operand gated) and match the
    oracle.  At d = 128 the fused kernel does not run and the call is the
    plain backward, bit for bit."""
    dev = need_gpu()
    import fenwick_tree_hierarchical_amd as la
    x, dout = case(T, d, "bf16", "weak_decay", seed=8)
    label = f"from fwd d={d} C={C} T={T}"
    say(f"bwd {label}: shape={tuple(x['q'].shape)}")
    plain = gpu_bwd(x, dout, C, dev)
    xd = {k: v.to(dev) for k, v in x.items()}
    B, H = x["q"].shape[:2]
    fws = torch.empty(max(la.loglinear_fwd_workspace(B, H, T, d, d, C, torch.bfloat16), 1), dtype=torch.uint8,
                      device=dev)
    la.loglinear_fwd(xd["q"], xd["k"], xd["v"], xd["log_a"], xd["lam"], chunk=C, workspace=fws)
    g = la.loglinear_bwd(xd["q"], xd["k"], xd["v"], xd["log_a"], xd["lam"], dout.to(dev), chunk=C,
                         fwd_workspace=fws)
    torch.cuda.synchronize()
    got = {n: t.float().cpu().numpy() for n, t in zip(NAMES, g)}
    for n in ("dk", "dv"):
        assert np.array_equal(got[n], plain[n]), n
    if d == 128:
        for n in NAMES:
            assert np.array_equal(got[n], plain[n]), n
    r = backward.backward_quadratic(x["q"], x["k"], x["v"], x["log_a"], x["lam"], dout)
    ref = dict(zip(NAMES, r))
    for n in ("dq", "dlam"):
        assert np.all(np.isfinite(got[n])), n
        assert_parity(got[n], ref[n], TOL["bf16"], f"{label} {n}")
        assert_parity(got[n], plain[n], TOL["bf16"], f"{label} {n} against the plain backward")
    assert_scaled(got["dlog_a"][..., None], ref["dlog_a"][..., None], gate_scale(x, dout, ref)[..., None],
                  TOL["bf16"], f"{label} dlog_a")


# --------------------------------------------------------------- full size
def test_train_16k_full_size_sampled():
    """All 128 heads of the training shape: the gradients at sampled query and
    key rows of three heads against the oracle, the gate gradient at the same
    rows included; on every head, the homogeneity identities q_t . dq_t =
    sum_l lambda dlambda = dout_t . o_t against the GPU forward, and a
    first-gate gradient that is zero up to rounding."""
    dev = need_gpu()
    import fenwick_tree_hierarchical_amd as la
    w = WORKLOADS["train_16k_bf16"]
    say("bwd full size train_16k_bf16: drawing inputs on the host")
    xc = make_inputs(w, device="cpu", variant="weak_decay")
    doutc = make_grad_out(w, device="cpu")
    rows = np.array([0, 1, 63, 64, 511, 512, 4095, 4096, 8191, 8192, 12000, 16320, 16383])
    idx = [(0, 0), (5, 9), (7, 15)]
    sub = heads(xc, idx)
    dsub = torch.stack([doutc[b, h] for b, h in idx])[None]
    say("   oracle gate gradient at sampled rows started (host workers)")
    pool = OraclePool(dict(sub, dout=dsub), kind="dlog_a", rows=rows)
    x = {k: v.to(dev) for k, v in xc.items()}
    dout = doutc.to(dev)
    say("bwd full size train_16k_bf16: backward")
    dq, dk, dv, dla, dlam = la.loglinear_bwd(x["q"], x["k"], x["v"], x["log_a"], x["lam"], dout, chunk=w.C)
    out = la.loglinear_fwd(x["q"], x["k"], x["v"], x["log_a"], x["lam"], chunk=w.C)
    torch.cuda.synchronize()
    for t in (dq, dk, dv, dla, dlam):
        assert torch.isfinite(t.float()).all().item()
    row = (dout.float() * out.float()).sum(-1)
    assert rel_l2((x["q"].float() * dq.float()).sum(-1).cpu().numpy(), row.cpu().numpy()) <= TOL["bf16"]
    assert rel_l2((x["lam"] * dlam).sum(-1).cpu().numpy(), row.cpu().numpy()) <= TOL["bf16"]
    # the first gate's gradient sums row - column terms over the whole
    # sequence and is zero up to rounding: bounded relative to the sum of
    # their magnitudes, the scale its rounding follows
    col = (x["v"].float() * dv.float()).sum(-1)
    mag = row.abs() + col.abs()
    scale = mag.sum(-1)
    assert bool((dla[..., 0].abs() <= TOL["bf16"] * scale).all())
    say("bwd full size train_16k_bf16: oracle at sampled rows")
    ref = backward.backward_sampled(sub["q"], sub["k"], sub["v"], sub["log_a"], sub["lam"], dsub, rows)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv), ("dlam", dlam)):
        got = torch.stack([t[b, h, rows] for b, h in idx])[None].float().cpu().numpy()
        assert_parity(got, ref[name], TOL["bf16"], f"{name} at sampled rows")
    # the gate gradient at the sampled rows: its bar is relative to the
    # reverse sum of |dout_u . o_u| + |v_u . dv_u| over u >= r, the scale its
    # rounding follows (taken from the GPU's o and dv: it sets the unit of
    # the bar, not the expected value)
    rsum = torch.flip(torch.cumsum(torch.flip(mag, [-1]), -1), [-1])
    gsc = torch.stack([rsum[b, h, rows] for b, h in idx])[None].double().cpu().numpy()
    got = torch.stack([dla[b, h, rows] for b, h in idx])[None].double().cpu().numpy()
    say("   waiting for the oracle gate gradient")
    ref_la = pool.result()
    assert_scaled(got[..., None], ref_la[..., None], gsc[..., None], TOL["bf16"], "dlog_a at sampled rows")


def test_long_128k_full_size_sampled():
    """The long-context shape (one batch, 16 heads, T = 131072, d = 128) with
    chunks of 64 in the backward: weak decay so that the group levels carry
    the gradients; one head at sampled query and key rows against the oracle,
    and the homogeneity identity q_t . dq_t = dout_t . o_t on every head."""
    dev = need_gpu()
    import fenwick_tree_hierarchical_amd as la
    w = WORKLOADS["long_128k_bf16"]
    say("bwd full size long_128k_bf16: drawing inputs")
    x = make_inputs(w, device=dev, variant="weak_decay")
    dout = make_grad_out(w, device=dev)
    say("bwd full size long_128k_bf16: backward (C = 64)")
    dq, dk, dv, dla, dlam = la.loglinear_bwd(x["q"], x["k"], x["v"], x["log_a"], x["lam"], dout, chunk=64)
    out = la.loglinear_fwd(x["q"], x["k"], x["v"], x["log_a"], x["lam"], chunk=w.C)
    torch.cuda.synchronize()
    for t in (dq, dk, dv, dla, dlam):
        assert torch.isfinite(t.float()).all().item()
    row = (dout.float() * out.float()).sum(-1)
    assert rel_l2((x["q"].float() * dq.float()).sum(-1).cpu().numpy(), row.cpu().numpy()) <= TOL["bf16"]
    rows = np.array([0, 63, 64, 4095, 4096, 65535, 65536, 98304, 131000, 131071])
    idx = [(0, 11)]
    sub = to_cpu(heads(x, idx))
    dsub = torch.stack([dout[b, h] for b, h in idx])[None].cpu()
    say("bwd full size long_128k_bf16: oracle at sampled rows")
    ref = backward.backward_sampled(sub["q"], sub["k"], sub["v"], sub["log_a"], sub["lam"], dsub, rows)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv), ("dlam", dlam)):
        got = torch.stack([t[b, h, rows] for b, h in idx])[None].float().cpu().numpy()
        assert_parity(got, ref[name], TOL["bf16"], f"{name} at sampled rows")


def test_very_long_sequence_deep_group_trees():
    """T = 2^23 + 37 tokens (d = 16, C = 16, fp32, one head), no decay: the
    query-side group tree over 65537 groups (17 carry levels, its widest
    slot instantiation) and the key-side tree at the same depth.  dq, dk, dv
    and dlambda at 5 sampled rows against the oracle, and the identity
    q_t . dq_t = dout_t . o_t on every row."""
    dev = need_gpu()
    import fenwick_tree_hierarchical_amd as la
    w = WORKLOADS["tiny_f32"]
    T, C = (1 << 23) + 37, 16
    say(f"bwd very long sequence T={T}: drawing inputs")
    x = make_inputs(w, device=dev, B=1, H=1, T=T, d=16, dtype="f32", seed=321, variant="no_decay")
    dout = make_grad_out(w, device=dev, B=1, H=1, T=T, d=16, dtype="f32", seed=322)
    dq, dk, dv, dla, dlam = la.loglinear_bwd(x["q"], x["k"], x["v"], x["log_a"], x["lam"], dout, chunk=C)
    out = la.loglinear_fwd(x["q"], x["k"], x["v"], x["log_a"], x["lam"], chunk=C)
    torch.cuda.synchronize()
    for t in (dq, dk, dv, dla, dlam):
        assert torch.isfinite(t).all().item()
    row = (dout * out).sum(-1)
    assert rel_l2((x["q"] * dq).sum(-1).cpu().double().numpy(), row.cpu().double().numpy()) <= TOL["f32"]
    rows = np.array([17, 1 << 22, (1 << 22) + (1 << 21) + 999, (1 << 23) - 1, T - 1])
    say("   oracle at sampled rows")
    xs = to_cpu(x)
    ref = backward.backward_sampled(xs["q"], xs["k"], xs["v"], xs["log_a"], xs["lam"], dout.cpu(), rows)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv), ("dlam", dlam)):
        assert_parity(t[:, :, rows].cpu().double().numpy(), ref[name], TOL["f32"], f"{name} at sampled rows")
