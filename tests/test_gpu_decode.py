"""Decode-step parity (GPU): against the oracle's recurrence, against the
GPU forward on the same sequence, and save/restore of the state."""

import numpy as np
import pytest
import torch

from fenwick_tree_hierarchical_amd.workloads import WORKLOADS, make_inputs
from oracle import forms
from tests.helpers import TOL, OraclePool, assert_parity, effective_slots, heads, need_gpu, say, to_cpu

pytestmark = pytest.mark.gpu


def run_decode(x, S, dev, st=None, t0=0, t1=None):
    """Decode tokens t0..t1-1 of x (on dev) one at a time; returns outputs
    [B,H,n,dv] (float32 numpy) and the state."""
    import fenwick_tree_hierarchical_amd as la
    B, H, T, dk = x["q"].shape
    t1 = T if t1 is None else t1
    if st is None:
        st = la.loglinear_state_init(B, H, dk, x["v"].shape[-1], S, dev)
    a = torch.exp(x["log_a"])                          # the gate, computed in float32
    lam = x["lam"][..., : S + 1]
    if lam.shape[-1] < S + 1:
        lam = torch.nn.functional.pad(lam, (0, S + 1 - lam.shape[-1]))
    outs = []
    for t in range(t0, t1):
        outs.append(la.loglinear_decode_step(st, x["q"][:, :, t].contiguous(), x["k"][:, :, t].contiguous(),
                                             x["v"][:, :, t].contiguous(), a[:, :, t].contiguous(),
                                             lam[:, :, t].contiguous()))
    torch.cuda.synchronize()
    return torch.stack(outs, dim=2).float().cpu().numpy(), st


@pytest.mark.parametrize("dtype,d", [("f32", 16), ("f32", 64), ("bf16", 64), ("f32", 128), ("bf16", 32)])
def test_decode_matches_oracle_recurrence(dtype, d):
    dev = need_gpu()
    T, S = 300, 10
    x = make_inputs(WORKLOADS["small_bf16"], B=2, H=3, T=T, L=S + 1, d=d, dtype=dtype, variant="weak_decay",
                    seed=d)
    say(f"decode vs oracle dtype={dtype} d={d} T={T}")
    xd = {k: v.to(dev) for k, v in x.items()}
    got, st = run_decode(xd, S, dev)
    a = torch.exp(x["log_a"])                          # same float32 gates the GPU used
    ref, ost = forms.forward_recurrent(x["q"], x["k"], x["v"], x["lam"], a=a, nlev=S)
    assert_parity(got, ref, TOL[dtype], f"decode dtype={dtype} d={d}")
    assert st.t == T
    # the state itself: scale * slots equals the oracle's eagerly gated buckets
    eff = effective_slots(st).cpu().numpy().reshape(2 * 3, S, d, d)
    active = [lv for lv in range(1, S + 1) if (T >> (lv - 1)) & 1]
    for lv in active:
        assert_parity(eff[:, lv - 1], ost.slots[:, lv], TOL[dtype], f"slot of level {lv}", lead=1)


def test_decode_matches_gpu_forward_f32():
    dev = need_gpu()
    import fenwick_tree_hierarchical_amd as la
    T, S = 777, 11
    x = make_inputs(WORKLOADS["small_bf16"], B=2, H=2, T=T, dtype="f32", variant="weak_decay", seed=9)
    xd = {k: v.to(dev) for k, v in x.items()}
    say("decode vs forward f32 T=777")
    got, _ = run_decode(xd, S, dev)
    # the decode takes a = exp(log_a) in float32; feed the forward log(a) of
    # exactly those gates so both see the same numbers
    fw = la.loglinear_fwd(xd["q"], xd["k"], xd["v"], torch.log(torch.exp(xd["log_a"])), xd["lam"], chunk=16)
    assert_parity(got, fw.float().cpu().numpy(), TOL["f32"], "decode vs forward")


def test_state_save_restore_bit_identical():
    dev = need_gpu()
    T, S, k = 200, 9, 77
    x = make_inputs(WORKLOADS["small_bf16"], B=2, H=4, T=T, L=S + 1, variant="weak_decay", seed=3)
    xd = {kk: v.to(dev) for kk, v in x.items()}
    say("decode save/restore")
    full, _ = run_decode(xd, S, dev)
    first, st = run_decode(xd, S, dev, t1=k)
    saved = st.clone()                                  # save
    _ = run_decode(xd, S, dev, st=st, t0=k, t1=k + 30)  # run on, then discard
    rest, _ = run_decode(xd, S, dev, st=saved, t0=k)    # restore and continue
    assert np.array_equal(np.concatenate([first, rest], axis=2), full)


def test_capacity_error_leaves_state_unchanged():
    dev = need_gpu()
    import fenwick_tree_hierarchical_amd as la
    S = 3
    x = make_inputs(WORKLOADS["small_bf16"], B=1, H=1, T=8, L=S + 1, seed=1)
    xd = {k: v.to(dev) for k, v in x.items()}
    _, st = run_decode(xd, S, dev, t1=7)                # t = 7 = 0b111: next merge needs level 4
    before = st.slots.clone()
    with pytest.raises(la.LogAttnError):
        run_decode(xd, S, dev, st=st, t0=7, t1=8)
    assert st.t == 7 and torch.equal(before, st.slots)


def test_decode_32k_prefix_256_steps():
    """Decode workload: 64 x 16 heads, a 32768-token prefix, then 256 steps;
    the steps equal the last 256 rows of the full-sequence forward, and the
    oracle on sampled heads."""
    dev = need_gpu()
    import fenwick_tree_hierarchical_amd as la
    w = WORKLOADS["decode_32k_bf16"]
    S = 16
    say("decode 32k: drawing inputs")
    x = make_inputs(w, device=dev)
    say("decode 32k: forward over 33024 tokens")
    a = torch.exp(x["log_a"])
    fw = la.loglinear_fwd(x["q"], x["k"], x["v"], torch.log(a), x["lam"], chunk=w.C)
    say("decode 32k: prefix by decode steps")
    _, st = run_decode(x, S, dev, t1=w.prefix)
    say("decode 32k: 256 timed-shape steps")
    got, st = run_decode(x, S, dev, st=st, t0=w.prefix)
    ref_fw = fw[:, :, w.prefix:].float().cpu().numpy()
    assert_parity(got, ref_fw, TOL["bf16"], "decode vs forward (all heads)")
    # 16 heads through the oracle recurrence over all 33024 tokens; the
    # decode takes a = exp(log_a) in float32, so the oracle gets log(a)
    idx = [(b, (5 * b) % 16) for b in range(0, 64, 4)]
    sub = to_cpu(heads(x, idx))
    sub["log_a"] = torch.log(torch.exp(sub["log_a"]))
    ref = OraclePool(sub).result()
    got_s = np.stack([got[b, h] for b, h in idx])[None]
    assert_parity(got_s, ref[:, :, w.prefix:], TOL["bf16"], "decode vs oracle (16 heads)")


def test_decode_rejects_a_wrong_out_before_launching():
    """A caller's out of the wrong shape, dtype or device, or k/v of another
    dtype than q, raise in the binding; the state does not move."""
    dev = need_gpu()
    import fenwick_tree_hierarchical_amd as la
    S, B, H, d = 4, 2, 3, 32
    st = la.loglinear_state_init(B, H, d, d, S, dev)
    q = torch.randn(B, H, d, device=dev, dtype=torch.bfloat16)
    a = torch.full((B, H), 0.9, device=dev)
    lam = torch.ones(B, H, S + 1, device=dev)
    bad_outs = [torch.empty(B, H, d - 1, device=dev, dtype=torch.bfloat16),
                torch.empty(B, H, d, device=dev, dtype=torch.float32),
                torch.empty(B, H, d, dtype=torch.bfloat16),
                torch.empty(B, H, 2 * d, device=dev, dtype=torch.bfloat16)[..., ::2]]
    for out in bad_outs:
        with pytest.raises((ValueError, TypeError)):
            la.loglinear_decode_step(st, q, q, q, a, lam, out=out)
    with pytest.raises(TypeError):
        la.loglinear_decode_step(st, q, q.float(), q, a, lam)
    with pytest.raises(TypeError):
        la.loglinear_decode_step(st, q, q, q.float(), a, lam)
    assert st.t == 0
    torch.cuda.synchronize()
