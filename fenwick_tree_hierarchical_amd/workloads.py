"""Seeded synthetic inputs for log-linear Mamba-2 attention.

This module is shared by the tests, the benchmark and the smoke check.  It
holds shapes, value distributions and seeds only -- none of the operator's
arithmetic -- so that the oracle and the GPU path can be fed the same tensors
without sharing any code of the method.

The workloads are shaped like the language-model layers the paper's
experiments use ([LLA-it] Sommario tecnico section 4; [LLA-es] Resumen
tecnico section 4: per-position loss analysed up to 16K tokens, long-context
retrieval); the datasets themselves are not used, synthetic tensors of the
same shapes stand in for them.

Distributions, drawn in float32 from one seeded ``torch.Generator`` in the
order q, k, v, log_a, lambda, each over its full [B, H, T, ...] shape:
  q, k    ~ N(0, 1/d_k), then L2-normalised over d_k
  v       ~ N(0, 1)
  log_a   = -softplus(x), x ~ N(0, 1)          ("A": tiny and small layers)
          = -softplus(0.5 x + 1), x ~ N(0, 1)  ("B": training shape, long
            context, decode)
  lambda  = softplus(x), x ~ N(0, 1), per token and level
q, k, v are then cast to the layer dtype (round to nearest even); log_a and
lambda stay float32.

The backward pass also takes the gradient of the loss with respect to the
output, ``make_grad_out``: dout ~ N(0, 1) over [B, H, T, d_v], drawn from its
own generator seeded with the workload seed + 1000, in the layer dtype.

The Gated DeltaNet form also takes a per-token write strength, ``make_beta``:
beta = sigmoid(x), x ~ N(0, 1) over [B, H, T], float32, from its own generator
seeded with the workload seed + 2000 (the gated delta rule's beta lies in
(0, 1)); its keys are the workload's L2-normalised k.
"""

from __future__ import annotations

import dataclasses
import math

import torch
import torch.nn.functional as F


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    C: int
    L: int
    dtype: str          # "f32" or "bf16" for q, k, v and the output
    dist: str           # "A" or "B" (log_a distribution)
    seed: int
    prefix: int = 0     # decode workloads: tokens before the first step
    steps: int = 0      # decode workloads: single-token steps


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 1, 64, 16, 16, 16, 7, "f32", "A", 0),
    "small_bf16": Workload("small_bf16", 4, 8, 2048, 64, 64, 64, 12, "bf16", "A", 1),
    "train_16k_bf16": Workload("train_16k_bf16", 8, 16, 16384, 64, 64, 64, 15, "bf16", "B", 2),
    "long_128k_bf16": Workload("long_128k_bf16", 1, 16, 131072, 128, 128, 128, 18, "bf16", "B", 3),
    "decode_32k_bf16": Workload("decode_32k_bf16", 64, 16, 32768 + 256, 64, 64, 64, 17, "bf16", "B",
                                4, prefix=32768, steps=256),
}


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def levels_for(T: int) -> int:
    """ceil(log2 T) + 1: the level count a sequence of length T uses."""
    return max(1, math.ceil(math.log2(T)) + 1) if T > 1 else 1


def make_inputs(w: Workload, device="cpu", B=None, H=None, T=None, L=None,
                variant: str | None = None, seed: int | None = None, d: int | None = None,
                dtype: str | None = None):
    """Draw one seeded input set for workload ``w``.

    B, H, T, L, d (d_k = d_v) and dtype ("f32"/"bf16") override the
    workload's (reduced-size and shape-sweep parity cases).
    ``variant`` changes the gates or weights after the draw:
      "weak_decay"  log_a <- 0.01 * log_a   (far buckets matter)
      "no_decay"    log_a <- 0
      "onehot:<l>"  lambda <- 1 on level l, 0 elsewhere
      "const:<c>"   lambda <- c everywhere
    joined with "+" to combine (e.g. "weak_decay+onehot:9").
    Returns a dict of tensors q, k, v (layer dtype), log_a, lam (float32).
    """
    B = w.B if B is None else B
    H = w.H if H is None else H
    T = w.T if T is None else T
    L = (w.L if T == w.T else levels_for(T)) if L is None else L
    dk = w.dk if d is None else d
    dv = w.dv if d is None else d
    g = torch.Generator(device=device)
    g.manual_seed(w.seed if seed is None else seed)
    f32 = dict(device=device, dtype=torch.float32, generator=g)
    q = torch.randn(B, H, T, dk, **f32) * (1.0 / math.sqrt(dk))
    k = torch.randn(B, H, T, dk, **f32) * (1.0 / math.sqrt(dk))
    v = torch.randn(B, H, T, dv, **f32)
    x = torch.randn(B, H, T, **f32)
    log_a = -F.softplus(x) if w.dist == "A" else -F.softplus(0.5 * x + 1.0)
    lam = F.softplus(torch.randn(B, H, T, L, **f32))
    q = q / q.norm(dim=-1, keepdim=True)
    k = k / k.norm(dim=-1, keepdim=True)
    for var in (variant.split("+") if variant else []):
        if var == "weak_decay":
            log_a = 0.01 * log_a
        elif var == "no_decay":
            log_a = torch.zeros_like(log_a)
        elif var.startswith("onehot:"):
            lev = int(var.split(":")[1])
            lam = torch.zeros_like(lam)
            lam[..., lev] = 1.0
        elif var.startswith("const:"):
            lam = torch.full_like(lam, float(var.split(":")[1]))
        else:
            raise ValueError(f"unknown variant {var!r}")
    dt = torch_dtype(w.dtype if dtype is None else dtype)
    return dict(q=q.to(dt).contiguous(), k=k.to(dt).contiguous(), v=v.to(dt).contiguous(),
                log_a=log_a.contiguous(), lam=lam.contiguous())


def make_grad_out(w: Workload, device="cpu", B=None, H=None, T=None, seed: int | None = None,
                  d: int | None = None, dtype: str | None = None):
    """Seeded upstream gradient dout [B, H, T, d_v] ~ N(0, 1) in the layer dtype."""
    B = w.B if B is None else B
    H = w.H if H is None else H
    T = w.T if T is None else T
    dv = w.dv if d is None else d
    g = torch.Generator(device=device)
    g.manual_seed((w.seed if seed is None else seed) + 1000)
    dout = torch.randn(B, H, T, dv, device=device, dtype=torch.float32, generator=g)
    return dout.to(torch_dtype(w.dtype if dtype is None else dtype)).contiguous()


def make_beta(w: Workload, device="cpu", B=None, H=None, T=None, seed: int | None = None):
    """Seeded write strengths beta [B, H, T] = sigmoid(N(0, 1)), float32."""
    B = w.B if B is None else B
    H = w.H if H is None else H
    T = w.T if T is None else T
    g = torch.Generator(device=device)
    g.manual_seed((w.seed if seed is None else seed) + 2000)
    x = torch.randn(B, H, T, device=device, dtype=torch.float32, generator=g)
    return torch.sigmoid(x).contiguous()
