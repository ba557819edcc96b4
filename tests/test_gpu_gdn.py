"""Log-linear Gated DeltaNet forward parity: the HIP path against the float64
oracle (GPU).

Bars (relative L2 over the compared outputs): 1e-4 for float32 inputs, 2e-2
for bfloat16 inputs.  The delta rule's transitions only shrink states, and at
the workloads' strong decays keys a chunk away are nearly invisible, so the
shape sweep runs with weak or no decay and lambda is also made one-hot on
single levels, which makes each intra-chunk level and each block of the
chunk tree carry the output on its own.
"""

import numpy as np
import pytest
import torch

from fenwick_tree_hierarchical_amd.workloads import WORKLOADS, make_beta, make_inputs
from oracle import deltanet as dn
from tests.helpers import TOL, OraclePool, assert_parity, heads, need_gpu, rel_l2, say, to_cpu

pytestmark = pytest.mark.gpu


def inputs(w, **kw):
    x = make_inputs(w, **kw)
    B, H, T = x["log_a"].shape
    x["beta"] = make_beta(w, B=B, H=H, T=T, seed=kw.get("seed"))
    return x


def gpu_gdn(x, C, dev):
    import fenwick_tree_hierarchical_amd as la
    xd = {k: v.to(dev) for k, v in x.items()}
    out = la.loglinear_gdn_fwd(xd["q"], xd["k"], xd["v"], xd["log_a"], xd["beta"], xd["lam"], chunk=C)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def oracle_gdn(x, rows=None):
    """The recurrence (per-level states) for whole sequences; the quadratic
    form (queries carried backwards) for sampled rows.  The two are pinned
    equal to 1e-12 on the CPU."""
    if rows is None:
        return dn.gdn_forward_recurrent(x["q"], x["k"], x["v"], x["log_a"], x["beta"], x["lam"])[0]
    return dn.gdn_forward_quadratic(x["q"], x["k"], x["v"], x["log_a"], x["beta"], x["lam"], rows=rows)


def check(x, C, dtype, dev, label):
    say(f"gdn {label}: shape={tuple(x['q'].shape)} C={C} dtype={dtype}")
    got = gpu_gdn(x, C, dev)
    ref = oracle_gdn(x)
    assert np.all(np.isfinite(got))
    return assert_parity(got, ref, TOL[dtype], label)["whole"]


def test_tiny_f32_workload():
    dev = need_gpu()
    w = WORKLOADS["tiny_f32"]
    check(inputs(w), w.C, "f32", dev, "tiny_f32")


@pytest.mark.parametrize("variant", [None, "weak_decay", "no_decay"])
def test_small_bf16_shape(variant):
    """The small bf16 layer shape (T=2048, d=64, C=64) on 4 of its heads."""
    dev = need_gpu()
    w = WORKLOADS["small_bf16"]
    check(inputs(w, B=1, H=4, variant=variant), w.C, "bf16", dev, f"small_bf16 {variant}")


SHAPES = [(16, 16), (32, 32), (64, 64), (64, 16), (16, 64), (32, 64), (64, 32)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d,C", SHAPES)
def test_shapes_with_ragged_tail(d, C, dtype):
    """13 full chunks (tree levels 0..3, every bit pattern of the chunk index
    up to 13) and a ragged last chunk, weak decay."""
    dev = need_gpu()
    w = WORKLOADS["tiny_f32"]
    T = 13 * C + 7
    x = inputs(w, B=1, H=2, T=T, d=d, dtype=dtype, seed=20 + d + C, variant="weak_decay")
    check(x, C, dtype, dev, f"d={d} C={C} T={T}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("level", list(range(12)))
def test_onehot_levels(level, dtype):
    """lambda one-hot on one level of T=2048 (C=64: levels 0-6 inside a chunk,
    7-11 the blocks of 1, 2, 4, 8 and 16 chunks), no decay."""
    dev = need_gpu()
    w = WORKLOADS["small_bf16"]
    x = inputs(w, B=1, H=2, T=2048, dtype=dtype, seed=40 + level, variant=f"no_decay+onehot:{level}")
    check(x, 64, dtype, dev, f"one-hot level {level}")


@pytest.mark.parametrize("T", [1, 2, 15, 16, 17, 100, 129])
def test_short_and_ragged(T):
    dev = need_gpu()
    w = WORKLOADS["tiny_f32"]
    check(inputs(w, B=2, H=1, T=T, seed=60 + T, variant="weak_decay"), 16, "f32", dev, f"T={T}")


def test_chunk_size_invariance():
    """The chunk size only changes the order of the arithmetic."""
    dev = need_gpu()
    w = WORKLOADS["tiny_f32"]
    x = inputs(w, B=1, H=2, T=1000, d=32, seed=77, variant="weak_decay")
    outs = {C: gpu_gdn(x, C, dev) for C in (16, 32, 64)}
    for C in (32, 64):
        err = rel_l2(outs[C], outs[16])
        say(f"   C={C} vs C=16: {err:.3e}")
        assert err <= TOL["f32"]


def test_constant_lambda_matches_gated_deltanet():
    """lambda constant: the textbook gated delta rule (no buckets) times it."""
    dev = need_gpu()
    w = WORKLOADS["tiny_f32"]
    x = inputs(w, B=1, H=2, T=300, d=16, seed=81, variant="weak_decay+const:0.75")
    got = gpu_gdn(x, 16, dev)
    ref = 0.75 * dn.gated_deltanet(x["q"], x["k"], x["v"], x["log_a"], x["beta"])
    assert_parity(got, ref, TOL["f32"], "gdn const lambda vs gated delta rule")


def test_empty_inputs():
    dev = need_gpu()
    import fenwick_tree_hierarchical_amd as la
    for B, T in ((0, 64), (1, 0)):
        x = inputs(WORKLOADS["tiny_f32"], B=max(B, 1), H=1, T=max(T, 1))
        xd = {k: v[:B, :, :T].contiguous().to(dev) if k != "lam" else v[:B, :, :T].contiguous().to(dev)
              for k, v in x.items()}
        out = la.loglinear_gdn_fwd(xd["q"], xd["k"], xd["v"], xd["log_a"], xd["beta"], xd["lam"], chunk=16)
        torch.cuda.synchronize()
        assert out.numel() == 0


def test_deterministic():
    dev = need_gpu()
    w = WORKLOADS["small_bf16"]
    x = inputs(w, B=1, H=2, T=1024, variant="weak_decay")
    a = gpu_gdn(x, 64, dev)
    b = gpu_gdn(x, 64, dev)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("variant", [None, "weak_decay"])
def test_training_shape_every_row(variant):
    """The 16K training shape (B=8, H=16, T=16384, d=64, C=64, bf16) in one
    launch; every row of all 128 heads against the oracle's recurrence (run
    over the heads in host worker processes while the GPU computes)."""
    dev = need_gpu()
    import fenwick_tree_hierarchical_amd as la
    w = WORKLOADS["train_16k_bf16"]
    say(f"gdn training shape {variant}: drawing inputs on the host")
    x = inputs(w, variant=variant)
    pool = OraclePool(x, kind="gdn")
    say(f"gdn training shape {variant}: full launch")
    got = gpu_gdn(x, w.C, dev)
    assert np.all(np.isfinite(got))
    say("   waiting for the oracle")
    ref = pool.result()
    assert_parity(got, ref, TOL["bf16"], f"gdn training shape {variant} every row")


def test_extra_levels_are_ignored():
    """lambda with more levels than ceil(log2 T) + 1: the extra ones are never read."""
    dev = need_gpu()
    w = WORKLOADS["tiny_f32"]
    x = inputs(w, B=1, H=2, T=300, d=16, seed=91, variant="weak_decay")
    ref = gpu_gdn(x, 16, dev)
    big = dict(x)
    pad = torch.randn(1, 2, 300, 11, generator=torch.Generator().manual_seed(5)).abs()
    big["lam"] = torch.cat([x["lam"], pad], dim=-1).contiguous()     # L = 10 + 11
    got = gpu_gdn(big, 16, dev)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("variant", ["no_decay", "no_decay+onehot:16"])
def test_deep_chunk_tree(variant):
    """T = 2^16 + 5 tokens (d = 16, C = 16, fp32, one head): 4096 full chunks,
    so the chunk tree has levels 0..12 (the tree kernel runs for m = 2..12)
    and chunk indices carry up to 12 set bits.  Without decay every bucket
    contributes; lambda one-hot on level 16 isolates the blocks of 2^11
    chunks.  The whole output against the oracle's recurrence."""
    dev = need_gpu()
    w = WORKLOADS["tiny_f32"]
    T = (1 << 16) + 5
    x = inputs(w, B=1, H=1, T=T, d=16, dtype="f32", seed=97, variant=variant)
    assert x["lam"].shape[-1] == 18
    check(x, 16, "f32", dev, f"deep chunk tree T={T} {variant}")
