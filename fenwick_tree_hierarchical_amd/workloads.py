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


# --------------------------------------------------------------------------
# Log-Linear Mamba-2 layer: the operator inside a Mamba-2 block
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class LayerWorkload:
    """Sizes of one Log-Linear Mamba-2 layer.

    d_model input width; H heads of head dim P (d_inner = H P); N state size
    (the operator's d_k, with d_v = P); G groups of heads sharing the B and C
    projections; K taps of the causal conv; C the operator's chunk size; L
    levels of lambda; eps of the gated RMS norm.
    """
    name: str
    B: int
    T: int
    d_model: int
    H: int
    P: int
    N: int
    G: int
    K: int
    C: int
    L: int
    dtype: str
    seed: int
    eps: float = 1e-5

    @property
    def d_inner(self) -> int:
        return self.H * self.P

    @property
    def conv_dim(self) -> int:
        return self.H * self.P + 2 * self.G * self.N

    @property
    def d_in_proj(self) -> int:
        return 2 * self.H * self.P + 2 * self.G * self.N + self.H + self.H * self.L


LAYER_WORKLOADS = {
    "layer_tiny_f32": LayerWorkload("layer_tiny_f32", 1, 100, 64, 4, 16, 16, 2, 4, 16, 8, "f32", 10),
    "layer_small_bf16": LayerWorkload("layer_small_bf16", 2, 2048, 256, 4, 64, 64, 1, 4, 64, 12, "bf16", 11),
    "layer_train_16k_bf16": LayerWorkload("layer_train_16k_bf16", 8, 16384, 512, 16, 64, 64, 1, 4, 64, 15,
                                          "bf16", 12),
}


def layer_resized(lw: LayerWorkload, **kw) -> LayerWorkload:
    """``lw`` with some sizes replaced; L follows T unless given."""
    if "T" in kw and "L" not in kw:
        kw["L"] = levels_for(kw["T"])
    return dataclasses.replace(lw, **kw)


def make_layer(lw: LayerWorkload, device="cpu", variant: str | None = None, seed: int | None = None):
    """Seeded input and weights of one layer (Mamba-2's published
    initialisation, restated):

      u         [B, T, d_model]      ~ N(0, 1)
      in_proj   [d_in_proj, d_model] ~ U(-1/sqrt(d_model), 1/sqrt(d_model))
      conv_w    [conv_dim, K]        ~ U(-1/sqrt(K), 1/sqrt(K)), conv_b likewise
      dt_bias   [H]   softplus^-1(dt0), dt0 = exp(U(log 1e-3, log 1e-1))
      A_log     [H]   log U(1, 16)
      D         [H]   1
      lam_bias  [H, L] 0
      norm_w    [d_inner] 1
      out_proj  [d_model, d_inner]   ~ U(-1/sqrt(d_inner), 1/sqrt(d_inner))

    drawn in that order from one generator; u, in_proj, conv_w, conv_b,
    norm_w and out_proj are then cast to the layer dtype, the rest stay
    float32.  ``variant``:
      "lam_one"   the lambda rows of in_proj zeroed and lam_bias set so
                  that every lambda is 1 (the plain Mamba-2 block)
      "D0"        D = 0
    """
    g = torch.Generator(device=device)
    g.manual_seed(lw.seed if seed is None else seed)
    f32 = dict(device=device, dtype=torch.float32, generator=g)

    def unif(shape, bound):
        return (torch.rand(*shape, **f32) * 2.0 - 1.0) * bound

    u = torch.randn(lw.B, lw.T, lw.d_model, **f32)
    in_proj = unif((lw.d_in_proj, lw.d_model), 1.0 / math.sqrt(lw.d_model))
    conv_w = unif((lw.conv_dim, lw.K), 1.0 / math.sqrt(lw.K))
    conv_b = unif((lw.conv_dim,), 1.0 / math.sqrt(lw.K))
    dt0 = torch.exp(torch.rand(lw.H, **f32) * (math.log(1e-1) - math.log(1e-3)) + math.log(1e-3))
    dt0 = dt0.clamp(min=1e-4)
    dt_bias = dt0 + torch.log(-torch.expm1(-dt0))
    A_log = torch.log(torch.rand(lw.H, **f32) * 15.0 + 1.0)
    D = torch.ones(lw.H, device=device)
    lam_bias = torch.zeros(lw.H, lw.L, device=device)
    norm_w = torch.ones(lw.d_inner, device=device)
    out_proj = unif((lw.d_model, lw.d_inner), 1.0 / math.sqrt(lw.d_inner))
    for var in (variant.split("+") if variant else []):
        if var == "lam_one":
            in_proj[lw.d_in_proj - lw.H * lw.L:] = 0.0
            lam_bias = torch.full_like(lam_bias, math.log(math.e - 1.0))
        elif var == "D0":
            D = torch.zeros_like(D)
        else:
            raise ValueError(f"unknown variant {var!r}")
    dt = torch_dtype(lw.dtype)
    return dict(u=u.to(dt).contiguous(), in_proj=in_proj.to(dt).contiguous(), conv_w=conv_w.to(dt).contiguous(),
                conv_b=conv_b.to(dt).contiguous(), dt_bias=dt_bias.contiguous(), A_log=A_log.contiguous(),
                D=D.contiguous(), lam_bias=lam_bias.contiguous(), norm_w=norm_w.to(dt).contiguous(),
                out_proj=out_proj.to(dt).contiguous())
