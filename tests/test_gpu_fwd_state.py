"""Forward with the final recurrent state (GPU): the state loglinear_fwd_state
leaves after T tokens against the oracle recurrence's state, and decode steps
continued from it against the oracle and the GPU forward over the whole
sequence."""

import numpy as np
import pytest
import torch

from fenwick_tree_hierarchical_amd.workloads import WORKLOADS, make_inputs
from oracle import forms
from tests.helpers import TOL, OraclePool, assert_parity, effective_slots, heads, need_gpu, say, to_cpu

pytestmark = pytest.mark.gpu

STALE = 7.0


def gpu_state(x, S, C, dev):
    """loglinear_fwd_state over all of x; returns (out, state)."""
    import fenwick_tree_hierarchical_amd as la
    B, H, T, d = x["q"].shape
    st = la.loglinear_state_init(B, H, d, d, S, dev)
    st.slots.fill_(STALE)               # occupied slots must be overwritten, others kept
    st.scale.fill_(3.0)
    out = la.loglinear_fwd_state(x["q"], x["k"], x["v"], x["log_a"], x["lam"], st, chunk=C)
    torch.cuda.synchronize()
    return out, st


def check_state(st, ost, T, S, tol):
    """GPU slot i against oracle level i+1; slots of empty levels untouched."""
    got = effective_slots(st).double().cpu().numpy()           # [B,H,S,dk,dv]
    B, H = got.shape[:2]
    ref = ost.slots.reshape(B, H, *ost.slots.shape[1:])       # [B,H,nlev+1,dk,dv]
    assert st.t == T
    assert bool((st.scale == 1).all())
    occupied = [i for i in range(S) if (T >> i) & 1]
    raw = st.slots.cpu()
    for i in range(S):
        if i not in occupied:
            assert bool((raw[:, :, i] == STALE).all()), f"slot {i} of an empty level was written"
    if occupied:
        g = got[:, :, occupied]
        r = np.stack([ref[:, :, i + 1] for i in occupied], axis=2)
        say(f"   state over levels {[i + 1 for i in occupied]}")
        assert_parity(g.reshape(B, H * len(occupied), *g.shape[3:]), r.reshape(B, H * len(occupied), *r.shape[3:]),
                      tol, "final state (per head and level)")
    return occupied


# (dtype, d, C, T): full groups, a partial group, a partial chunk (levels inside
# a chunk), one full chunk, one full group, a power of two, short sequences
CASES = [("f32", 32, 16, 16 * 8 * 4), ("f32", 32, 16, 16 * 8 * 3 + 16 * 5 + 11), ("f32", 16, 32, 777),
         ("f32", 64, 64, 64), ("f32", 32, 16, 16 * 8), ("f32", 16, 16, 1), ("f32", 16, 16, 13),
         ("f32", 128, 64, 1000), ("f32", 64, 128, 2 * 128 * 8 + 127),
         ("bf16", 64, 64, 2048), ("bf16", 64, 64, 64 * 8 * 5 + 64 * 3 + 37), ("bf16", 128, 128, 3000),
         ("bf16", 32, 32, 4096 + 1)]


@pytest.mark.parametrize("dtype,d,C,T", CASES)
def test_final_state_matches_oracle(dtype, d, C, T):
    dev = need_gpu()
    import fenwick_tree_hierarchical_amd as la
    S = max(T.bit_length(), 1) + 2                    # two slots more than needed
    x = make_inputs(WORKLOADS["small_bf16"], B=2, H=2, T=T, L=max(T.bit_length(), 1) + 1, d=d, dtype=dtype,
                    variant="weak_decay", seed=T % 97)
    say(f"final state dtype={dtype} d={d} C={C} T={T} S={S}")
    xd = {k: v.to(dev) for k, v in x.items()}
    out, st = gpu_state(xd, S, C, dev)
    plain = la.loglinear_fwd(xd["q"], xd["k"], xd["v"], xd["log_a"], xd["lam"], chunk=C)
    assert torch.equal(out, plain)                    # same kernels, same output
    _, ost = forms.forward_recurrent(x["q"], x["k"], x["v"], x["lam"], log_a=x["log_a"], nlev=S)
    check_state(st, ost, T, S, TOL[dtype])


def test_final_state_empty_sequence():
    dev = need_gpu()
    import fenwick_tree_hierarchical_amd as la
    x = make_inputs(WORKLOADS["tiny_f32"], T=1, device=dev)
    x = {k: v[:, :, :0].contiguous() for k, v in x.items()}
    st = la.loglinear_state_init(1, 1, 16, 16, 4, dev)
    st.slots.fill_(5.0)
    la.loglinear_fwd_state(x["q"], x["k"], x["v"], x["log_a"], x["lam"], st, chunk=16)
    torch.cuda.synchronize()
    assert st.t == 0 and not st.slots.any() and bool((st.scale == 1).all())


@pytest.mark.parametrize("dtype,d,C,P,N", [("f32", 32, 16, 16 * 8 * 2 + 5, 40), ("bf16", 64, 64, 64 * 8 * 3, 70),
                                           ("f32", 64, 32, 1000, 24)])
def test_decode_continues_from_forward_state(dtype, d, C, P, N):
    """Prefill P tokens with loglinear_fwd_state, decode N more: equal to the
    oracle recurrence and to the GPU forward over all P + N tokens."""
    dev = need_gpu()
    import fenwick_tree_hierarchical_amd as la
    from tests.test_gpu_decode import run_decode
    T = P + N
    S = T.bit_length() + 1
    x = make_inputs(WORKLOADS["small_bf16"], B=2, H=3, T=T, L=S + 1, d=d, dtype=dtype, variant="weak_decay",
                    seed=P % 89)
    say(f"hand-off dtype={dtype} d={d} C={C} prefix={P} steps={N}")
    a = torch.exp(x["log_a"])                         # the decode gates, float32
    la_f = torch.log(a)                               # and the forward's view of them
    xd = {k: v.to(dev) for k, v in x.items()}
    pre = {k: v[:, :, :P].contiguous() for k, v in xd.items()}
    pre["log_a"] = la_f[:, :, :P].contiguous().to(dev)
    _, st = gpu_state(pre, S, C, dev)
    got, st = run_decode(xd, S, dev, st=st, t0=P)
    assert st.t == T
    ref, _ = forms.forward_recurrent(x["q"], x["k"], x["v"], x["lam"], a=a, nlev=S)
    assert_parity(got, ref[:, :, P:], TOL[dtype], "decode after hand-off vs oracle")
    full = la.loglinear_fwd(xd["q"], xd["k"], xd["v"], la_f.to(dev), xd["lam"], chunk=C)
    assert_parity(got, full[:, :, P:].float().cpu().numpy(), TOL[dtype], "decode after hand-off vs GPU forward")


def test_decode_32k_handoff_256_steps():
    """Decode workload with the prefix from one forward: 64 x 16 heads, a
    32768-token prefill by loglinear_fwd_state, then 256 decode steps; they
    equal the last 256 rows of the full-sequence forward, and the oracle on
    sampled heads."""
    dev = need_gpu()
    import fenwick_tree_hierarchical_amd as la
    from tests.test_gpu_decode import run_decode
    w = WORKLOADS["decode_32k_bf16"]
    S = 16
    say("decode 32k hand-off: drawing inputs")
    x = make_inputs(w, device=dev)
    a = torch.exp(x["log_a"])
    la_f = torch.log(a)
    say("decode 32k hand-off: forward over 33024 tokens")
    fw = la.loglinear_fwd(x["q"], x["k"], x["v"], la_f, x["lam"], chunk=w.C)
    say("decode 32k hand-off: prefill forward with state")
    pre = {k: v[:, :, :w.prefix].contiguous() for k, v in x.items()}
    pre["log_a"] = la_f[:, :, :w.prefix].contiguous()
    _, st = gpu_state(pre, S, w.C, dev)
    say("decode 32k hand-off: 256 steps")
    got, st = run_decode(x, S, dev, st=st, t0=w.prefix)
    assert_parity(got, fw[:, :, w.prefix:].float().cpu().numpy(), TOL["bf16"], "decode vs forward (all heads)")
    idx = [(b, (3 * b + 1) % 16) for b in range(2, 64, 4)]
    sub = to_cpu(heads(x, idx))
    sub["log_a"] = torch.log(torch.exp(sub["log_a"]))
    ref = OraclePool(sub).result()
    got_s = np.stack([got[b, h] for b, h in idx])[None]
    assert_parity(got_s, ref[:, :, w.prefix:], TOL["bf16"], "decode vs oracle (16 heads)")


def test_handoff_after_very_long_prefill():
    """A prefill of 2^23 + 37 tokens (d = 16, C = 16, fp32, one head, no
    decay: slots 0, 2, 5 and 23 occupied, the last one a bucket of 2^23
    keys), then 40 decode steps; they equal the GPU forward over all
    2^23 + 77 tokens and the oracle at sampled steps."""
    dev = need_gpu()
    import fenwick_tree_hierarchical_amd as la
    from tests.test_gpu_decode import run_decode
    P, N, C = (1 << 23) + 37, 40, 16
    T = P + N
    S = T.bit_length() + 1
    say(f"hand-off after a {P}-token prefill: drawing inputs")
    x = make_inputs(WORKLOADS["tiny_f32"], device=dev, B=1, H=1, T=T, L=S + 1, d=16, dtype="f32", seed=55,
                    variant="no_decay")
    pre = {k: v[:, :, :P].contiguous() for k, v in x.items()}
    _, st = gpu_state(pre, S, C, dev)
    assert st.t == P
    got, st = run_decode(x, S, dev, st=st, t0=P)
    assert st.t == T
    full = la.loglinear_fwd(x["q"], x["k"], x["v"], x["log_a"], x["lam"], chunk=C)
    assert_parity(got, full[:, :, P:].float().cpu().numpy(), TOL["f32"], "decode vs GPU forward")
    steps = np.array([0, 1, 7, 26, 39])
    xs = to_cpu(x)
    ref = forms.forward_quadratic(xs["q"], xs["k"], xs["v"], xs["log_a"], xs["lam"], rows=P + steps, block=4)
    assert_parity(got[:, :, steps], ref, TOL["f32"], f"decode vs oracle ({len(steps)} steps)")
