"""CPU oracle for log-linear Mamba-2 attention (test infrastructure only).

This package is the slow, plain, float64 statement of what the GPU library
computes.  Only the test-suite, the smoke check and the CPU-baseline leg of the
benchmark may import it; the product path never does, and this package imports
nothing from the GPU package.

Sources (the two summaries of the same paper, cited by page and section):

  [LLA-it]  "Log-Linear Attention", gist.science, Italian summary
            (lay part "L'essenziale"; technical summary "Sommario tecnico"
            sections 1-5).
  [LLA-es]  "Log-Linear Attention", gist.science, Spanish summary
            (lay part "Lo esencial"; technical summary "Resumen tecnico"
            sections 1-5).

The operator, with 0-based token indices t (query) and s (key):

  o_t = sum_{s<=t} lambda_t^{(l(t,s))} * M^S[t,s] * (q_t . k_s) * v_s

  * M^S[t,s] = prod_{s<r<=t} a_r, a_r = exp(log_a_r)   (Mamba-2 scalar gate,
    [LLA-es] section 2 "Variantes", item 1; semiseparable mask,
    [LLA-it] section 2 item 2).
  * l(t,s) is the Fenwick-tree bucket that holds key s as seen from query t
    ([LLA-it] section 2 item 1; [LLA-es] section 2 "Conceptos clave").
    Reading used here: bucket 0 is the query token itself; the rest of the
    prefix [0,t) is cut by stripping the lowest set bit of t, bucket l >= 1
    holding 2^(l-1) keys.  Closed form: l = 1 + msb(t xor s).
  * lambda_t^{(l)} is a per-token, per-level weight; the hierarchical mask
    M^H[t,s] = lambda_t^{(l(t,s))} replaces the causal mask ([LLA-it]
    section 2 item 2; [LLA-es] section 2 "Conceptos clave").

Modules:
  levels   -- the level function, two independent derivations, bucket lists
  forms    -- quadratic (masked O(T^2)) form and the Fenwick-state recurrence
  special  -- special-case references written without the level machinery,
              and a pure-Python brute force for tiny inputs
  metrics  -- relative L2 error
  backward -- the gradients of the operator (chain rule on the quadratic form)
  deltanet -- the log-linear Gated DeltaNet form
  layer    -- the Log-Linear Mamba-2 layer around the operator (projections,
              causal conv, gates, lambda, D skip, gated norm)

Pin status (what fixes each function other than itself) is listed in the
header of each module.  Nothing here is "parity unpinned"; the *choice* of the
level reading above is an interpretation of the pages, which print no formula
for it.
"""

from . import levels, forms, special, metrics, backward, deltanet, layer  # noqa: F401
