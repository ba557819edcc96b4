"""GPU parity of the Log-Linear Mamba-2 layer (loglinear_mamba2_fwd) against
the oracle's parallel form (oracle.layer).

The layer is Mamba-2's block with the log-linear operator in place of its SSM
("Log-Linear Attention", Spanish summary, technical section 2, "Variantes",
item 1).  Every case compares the whole output, per sequence and per token
row (tests/helpers.py bars).  The "D0" variant zeroes the D skip so the
output is the operator's alone through the gate and norm (with the skip, the
operator is a small part of the output); "lam_one" makes every lambda 1.
"""

import dataclasses

import numpy as np
import pytest
import torch

import fenwick_tree_hierarchical_amd as la
from fenwick_tree_hierarchical_amd.workloads import LAYER_WORKLOADS, layer_resized, make_layer
from oracle import layer as olayer
from tests.helpers import TOL, OraclePool, assert_parity, need_gpu, say

pytestmark = pytest.mark.gpu

TINY = LAYER_WORKLOADS["layer_tiny_f32"]
SMALL = LAYER_WORKLOADS["layer_small_bf16"]
TRAIN = LAYER_WORKLOADS["layer_train_16k_bf16"]


def run_gpu(lw, w, dev):
    wd = {k: v.to(dev) for k, v in w.items()}
    out = la.loglinear_mamba2_fwd(wd["u"], wd, lw.H, lw.P, lw.N, lw.G, C=lw.C, eps=lw.eps)
    torch.cuda.synchronize()
    return out.cpu()


def check(lw, variant=None, seed=None, label=""):
    dev = need_gpu()
    say(f"layer {lw.name} B={lw.B} T={lw.T} d_model={lw.d_model} H={lw.H} P={lw.P} G={lw.G} K={lw.K} C={lw.C} "
        f"L={lw.L} {lw.dtype} variant={variant} seed={seed} {label}")
    w = make_layer(lw, variant=variant, seed=seed)
    got = run_gpu(lw, w, dev)
    ref = olayer.layer_forward(w["u"], w, lw, operator="recurrent")
    assert torch.isfinite(got).all()
    return assert_parity(got, ref, TOL[lw.dtype], f"{lw.name} {variant}", lead=1)


@pytest.mark.parametrize("variant", [None, "D0", "lam_one"])
def test_tiny_f32(variant):
    check(TINY, variant)


@pytest.mark.parametrize("variant", [None, "D0"])
def test_small_bf16(variant):
    check(SMALL, variant)


# (H, P, G, K, d_model, C, T): several groups, one group, a group per head,
# every conv width, ragged T, T below one chunk
SWEEP = [
    (4, 16, 2, 4, 64, 16, 333),
    (2, 32, 1, 2, 64, 32, 200),
    (8, 16, 8, 3, 128, 16, 257),
    (2, 64, 2, 4, 128, 64, 700),
    (4, 64, 1, 4, 256, 64, 1000),
    (1, 128, 1, 4, 128, 64, 300),
    (4, 16, 4, 1, 64, 16, 5),
    (4, 32, 2, 4, 192, 32, 1),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SWEEP, ids=[str(s) for s in SWEEP])
def test_shape_sweep(shape, dtype):
    H, P, G, K, d_model, C, T = shape
    lw = layer_resized(TINY, name=f"sweep_{dtype}", B=2, T=T, H=H, P=P, N=P, G=G, K=K, d_model=d_model, C=C,
                       dtype=dtype)
    check(lw, "D0", seed=21)
    check(lw, None, seed=22)


def test_training_shape_every_row():
    """The 16K training layer (B = 8, T = 16384, d_model = 512, 16 heads of 64)
    at full size: every output row of every sequence against the oracle, the
    operator run head by head in worker processes."""
    dev = need_gpu()
    for variant in (None, "D0"):
        say(f"layer {TRAIN.name} full size variant={variant}")
        w = make_layer(TRAIN, variant=variant)
        q, k, v, log_a, lam, x, z = olayer.layer_operator_inputs(w["u"], w, TRAIN)
        pool = OraclePool(dict(q=torch.from_numpy(q), k=torch.from_numpy(k), v=torch.from_numpy(v),
                               log_a=torch.from_numpy(log_a), lam=torch.from_numpy(lam)))
        got = run_gpu(TRAIN, w, dev)
        o = pool.result()
        ref = olayer.layer_output(o, x, z, w, TRAIN)
        assert torch.isfinite(got).all()
        assert_parity(got, ref, TOL["bf16"], f"{TRAIN.name} {variant}", lead=1)


def test_deterministic_and_ragged_batch():
    dev = need_gpu()
    lw = layer_resized(SMALL, B=3, T=777)
    w = make_layer(lw, seed=4)
    a = run_gpu(lw, w, dev)
    b = run_gpu(lw, w, dev)
    assert torch.equal(a, b)


def test_empty_writes_nothing():
    dev = need_gpu()
    lw = layer_resized(TINY, T=0, L=1)
    w = make_layer(layer_resized(TINY, T=1), seed=1)
    wd = {k: v.to(dev) for k, v in w.items()}
    wd["lam_bias"] = torch.zeros(lw.H, 1, device=dev)
    wd["in_proj"] = torch.zeros(lw.d_in_proj, lw.d_model, device=dev)
    u = torch.zeros(1, 0, lw.d_model, device=dev)
    out = la.loglinear_mamba2_fwd(u, wd, lw.H, lw.P, lw.N, lw.G, C=lw.C)
    torch.cuda.synchronize()
    assert out.shape == (1, 0, lw.d_model)


def test_rejects_bad_sizes_before_launching():
    dev = need_gpu()
    lw = layer_resized(TINY, T=16)
    w = {k: v.to(dev) for k, v in make_layer(lw).items()}
    with pytest.raises(ValueError):     # binding: wrong in_proj shape for G
        la.loglinear_mamba2_fwd(w["u"], w, lw.H, lw.P, lw.N, 4, C=lw.C)
    with pytest.raises(la.LogAttnError) as e:   # library: P != N
        la.loglinear_mamba2_fwd_workspace(1, 16, 64, 4, 16, 32, 2, 4, 16, 8, 1e-5, torch.float32)
    assert e.value.code == -2
