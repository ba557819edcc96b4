"""The allocation-free forward (loglinear_fwd_noalloc): the library's fixed
per-GPU scratch in place of a caller's workspace.  Through the C ABI it must
give the same output bits as loglinear_fwd with a workspace, on two calls in
a row (the second smaller, so the scratch holds the first call's contents),
and refuse shapes beyond the scratch with LA_ESCRATCH without writing out."""

import ctypes

import numpy as np
import pytest
import torch

from fenwick_tree_hierarchical_amd.workloads import WORKLOADS, make_inputs
from tests.helpers import need_gpu, say

pytestmark = pytest.mark.gpu

LA_ESCRATCH = -8


def _ptrs(x, out):
    return [x["q"].data_ptr(), x["k"].data_ptr(), x["v"].data_ptr(), x["log_a"].data_ptr(), x["lam"].data_ptr(),
            out.data_ptr()]


def _noalloc(lib, x, out, C, stream):
    B, H, T, d = x["q"].shape
    dt = 1 if x["q"].dtype == torch.bfloat16 else 0
    return lib.loglinear_fwd_noalloc(*_ptrs(x, out), B, H, T, d, d, C, x["lam"].shape[-1], dt, stream)


def test_noalloc_matches_the_workspace_forward_twice():
    dev = need_gpu()
    import fenwick_tree_hierarchical_amd as la
    lib = la.lib()
    stream = torch.cuda.current_stream(dev).cuda_stream
    cases = [("bf16", 2, 8, 9000, 64, 64, 11), ("bf16", 1, 3, 2000, 64, 64, 12), ("f32", 1, 2, 777, 32, 16, 13)]
    for dtype, B, H, T, d, C, seed in cases:
        say(f"noalloc forward dtype={dtype} B={B} H={H} T={T} d={d} C={C}")
        x = make_inputs(WORKLOADS["small_bf16"], device=dev, B=B, H=H, T=T, d=d, dtype=dtype, variant="weak_decay",
                        seed=seed)
        ref = la.loglinear_fwd(x["q"], x["k"], x["v"], x["log_a"], x["lam"], chunk=C)
        out = torch.full_like(ref, float("nan"))
        assert _noalloc(lib, x, out, C, stream) == 0
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "noalloc output differs from the workspace forward"


def test_noalloc_rejects_shapes_beyond_its_scratch():
    dev = need_gpu()
    import fenwick_tree_hierarchical_amd as la
    lib = la.lib()
    stream = torch.cuda.current_stream(dev).cuda_stream
    B, H, T, d, C = 1, 24, 16384, 64, 64             # 24 heads of 2.9 MB > 64 MiB
    assert la.loglinear_fwd_workspace(B, H, T, d, d, C, torch.bfloat16) > (64 << 20)
    x = make_inputs(WORKLOADS["train_16k_bf16"], device=dev, B=B, H=H, T=T)
    out = torch.zeros(B, H, T, d, dtype=torch.bfloat16, device=dev)
    assert _noalloc(lib, x, out, C, stream) == LA_ESCRATCH
    torch.cuda.synchronize()
    assert bool((out == 0).all())
    assert "scratch" in la.loglinear_strerror(LA_ESCRATCH)
