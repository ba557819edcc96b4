"""Log-Linear Mamba-2 layer around the operator (oracle; test infrastructure only).

The pages name Log-Linear Mamba-2 as one of the two instances of the
framework: Mamba-2's selective (input-dependent) gate combined with the
hierarchical mask ([LLA-es] Resumen tecnico section 2, "Variantes", item 1;
[LLA-it] Sommario tecnico section 2, item 4).  They print no layer.  The
reading used here is the plainest one: the Mamba-2 block as published (Dao
and Gu, 2024, the Mamba-2 block of "Transformers are SSMs"), with its SSM
replaced by the log-linear operator and one more group of projected columns
that supplies the per-token, per-level weights lambda.  Per batch element,
with d_inner = H P and G groups of heads sharing B and C:

  zxbcdt = u W_in^T          columns [ z | x | B | C | dt | lam ]
                             widths  [ H P | H P | G N | G N | H | H L ]
  x|B|C  <- silu(causal depthwise conv over time of x|B|C, plus bias)
             conv[t, c] = bias[c] + sum_j w[c, j] xBC[t - (K-1) + j, c],
             zero before the first token
  dt_h   = softplus(dt_h + dt_bias_h),   A_h = -exp(A_log_h)
  operator inputs of head h (group g = h // (H / G)):
     q = C_g,  k = B_g,  v = dt_h x_h,  log_a = dt_h A_h,
     lambda = softplus(lam_h + lam_bias_h)            (one per level)
  y_h    = operator(q, k, v, log_a, lambda)_h + D_h x_h
  g      = y * silu(z)   (gate before the norm)
  g      <- g / sqrt(mean over each of G channel groups of g^2 + eps) * norm_w
  out    = g W_out^T

Three evaluations, written separately:

* ``layer_forward`` -- the parallel form over whole sequences (numpy array
  operations; the operator by ``forms.forward_quadratic`` or
  ``forms.forward_recurrent``), in two halves around the operator,
  ``layer_operator_inputs`` and ``layer_output``, so that long sequences can
  run the operator head by head.  The GPU layer is compared with this one.
* ``layer_forward_stepwise(ssm="fenwick")`` -- the decoding form: one token
  at a time, a rolling window of the last K conv inputs per channel, the
  operator by its Fenwick-state recurrence (``forms.recurrent_step``), its own
  index arithmetic, softplus and silu.
* ``layer_forward_stepwise(ssm="mamba2")`` -- the same loop with the textbook
  Mamba-2 state h_t = exp(dt A) h_{t-1} + dt x_t B_t^T (P x N per head),
  y_t = h_t C_t + D x_t, and no lambda: the plain Mamba-2 block.

Pins (tests/test_oracle_layer.py): the parallel and stepwise forms agree to
1e-12 (G = 1, 2, H; ragged T; either operator form); with lambda = 1 on every
level the layer equals the plain Mamba-2 block; the convolution equals
numpy.convolve per channel; outputs are causal; the norm gives unit mean
square per group when eps = 0; planted mistakes each fail one of these
(tests/test_oracle_layer.py, mutants).
"""

from __future__ import annotations

import numpy as np

from . import forms as _forms
from .forms import _f64


def _silu(x):
    return x / (1.0 + np.exp(-x))


def _softplus(x):
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def widths(dims):
    """Column widths of the input projection: z, x, B, C, dt, lam."""
    d_inner = dims.H * dims.P
    GN = dims.G * dims.N
    return [d_inner, d_inner, GN, GN, dims.H, dims.H * dims.L]


def split_projection(zxbcdt, dims):
    """Split [B, T, d_in_proj] into z, xBC (the conv input), dt, lam."""
    wz, wx, wb, wc, wdt, wl = widths(dims)
    o = np.cumsum([0, wz, wx + wb + wc, wdt, wl])
    return (zxbcdt[..., o[0]:o[1]], zxbcdt[..., o[1]:o[2]], zxbcdt[..., o[2]:o[3]],
            zxbcdt[..., o[3]:o[4]])


def causal_conv(xbc, conv_w, conv_b):
    """Depthwise causal convolution over time: [B, T, ch] -> [B, T, ch].

    out[t, c] = conv_b[c] + sum_{j<K} conv_w[c, j] * xbc[t - (K-1) + j, c],
    with zeros before the first token.
    """
    Bn, T, ch = xbc.shape
    K = conv_w.shape[1]
    pad = np.concatenate([np.zeros((Bn, K - 1, ch)), xbc], axis=1)
    out = np.broadcast_to(conv_b, (Bn, T, ch)).copy()
    for j in range(K):
        out += conv_w[:, j] * pad[:, j:j + T, :]
    return out


def operator_inputs(xbc, dt_raw, lam_raw, w, dims):
    """q, k, v [B,H,T,.], log_a [B,H,T], lam [B,H,T,L] and x [B,T,H,P]."""
    Bn, T, _ = xbc.shape
    H, P, N, G, L = dims.H, dims.P, dims.N, dims.G, dims.L
    d_inner = H * P
    x = xbc[..., :d_inner].reshape(Bn, T, H, P)
    Bm = xbc[..., d_inner:d_inner + G * N].reshape(Bn, T, G, N)
    Cm = xbc[..., d_inner + G * N:].reshape(Bn, T, G, N)
    group = np.arange(H) // (H // G)
    dt = _softplus(dt_raw + _f64(w["dt_bias"]))                   # [B, T, H]
    A = -np.exp(_f64(w["A_log"]))                                 # [H]
    q = Cm[:, :, group].transpose(0, 2, 1, 3)
    k = Bm[:, :, group].transpose(0, 2, 1, 3)
    v = (x * dt[..., None]).transpose(0, 2, 1, 3)
    log_a = (dt * A).transpose(0, 2, 1)
    lam = _softplus(lam_raw.reshape(Bn, T, H, L) + _f64(w["lam_bias"])).transpose(0, 2, 1, 3)
    return q, k, v, log_a, lam, x


def gated_rmsnorm(y, z, norm_w, G, eps):
    """g = y * silu(z), normalised by the root mean square over each of G
    equal channel groups, times norm_w.  y, z: [B, T, d_inner]."""
    g = y * _silu(z)
    Bn, T, d = g.shape
    gg = g.reshape(Bn, T, G, d // G)
    r = 1.0 / np.sqrt(np.mean(gg * gg, axis=-1, keepdims=True) + eps)
    return (gg * r).reshape(Bn, T, d) * norm_w


def layer_operator_inputs(u, w, dims):
    """The steps before the operator: the input projection, the conv, the
    gates and lambda.  Returns (q, k, v, log_a, lam, x, z) with q, k, v
    [B, H, T, .], log_a [B, H, T], lam [B, H, T, L], x [B, T, H, P] (the
    conv output of the x channels) and z [B, T, H P]."""
    u = _f64(u)
    zxbcdt = u @ _f64(w["in_proj"]).T
    z, xbc, dt_raw, lam_raw = split_projection(zxbcdt, dims)
    xbc = _silu(causal_conv(xbc, _f64(w["conv_w"]), _f64(w["conv_b"])))
    q, k, v, log_a, lam, x = operator_inputs(xbc, dt_raw, lam_raw, w, dims)
    return q, k, v, log_a, lam, x, z


def layer_output(o, x, z, w, dims):
    """The steps after the operator: the D skip, the gated norm and the output
    projection.  o [B, H, T, P] -> [B, T, d_model]."""
    o = _f64(o)
    Bn, H, T, P = o.shape
    y = o.transpose(0, 2, 1, 3) + _f64(w["D"])[:, None] * x        # [B, T, H, P]
    g = gated_rmsnorm(y.reshape(Bn, T, H * P), z, _f64(w["norm_w"]), dims.G, dims.eps)
    return g @ _f64(w["out_proj"]).T


def layer_forward(u, w, dims, operator: str = "quadratic"):
    """The layer over whole sequences; u [B, T, d_model] -> [B, T, d_model].

    ``w`` maps names to arrays or tensors: in_proj [d_in_proj, d_model],
    conv_w [ch, K], conv_b [ch], dt_bias [H], A_log [H], D [H],
    lam_bias [H, L], norm_w [H P], out_proj [d_model, H P].  ``dims`` has
    the attributes H, P, N, G, L, eps.  ``operator`` picks the operator's
    quadratic or recurrent form.
    """
    q, k, v, log_a, lam, x, z = layer_operator_inputs(u, w, dims)
    if operator == "quadratic":
        o = _forms.forward_quadratic(q, k, v, log_a, lam)
    elif operator == "recurrent":
        o, _ = _forms.forward_recurrent(q, k, v, lam, log_a=log_a)
    else:
        raise ValueError(operator)
    return layer_output(o, x, z, w, dims)


def layer_forward_stepwise(u, w, dims, ssm: str = "fenwick"):
    """The layer one token at a time (the decoding form).

    Per channel a window of the last K conv inputs slides by one on every
    token; the operator is the Fenwick-state recurrence (ssm="fenwick"), or
    the textbook Mamba-2 state with lambda ignored (ssm="mamba2").
    """
    u = _f64(u)
    W_in, W_out = _f64(w["in_proj"]), _f64(w["out_proj"])
    conv_w, conv_b = _f64(w["conv_w"]), _f64(w["conv_b"])
    dt_bias, A_log, Dsk = _f64(w["dt_bias"]), _f64(w["A_log"]), _f64(w["D"])
    lam_bias, norm_w = _f64(w["lam_bias"]), _f64(w["norm_w"])
    Bn, T, _ = u.shape
    H, P, N, G, L, eps = dims.H, dims.P, dims.N, dims.G, dims.L, dims.eps
    K = conv_w.shape[1]
    di = H * P
    ch = di + 2 * G * N
    heads_per_group = H // G
    window = np.zeros((Bn, ch, K))
    if ssm == "fenwick":
        state = _forms.FenwickState(Bn * H, N, P, max(1, T).bit_length() + 1)
    elif ssm == "mamba2":
        h = np.zeros((Bn, H, P, N))
    else:
        raise ValueError(ssm)
    out = np.zeros((Bn, T, W_out.shape[0]))
    for t in range(T):
        proj = np.einsum("ij,bj->bi", W_in, u[:, t])
        zt = proj[:, 0:di]
        xbct = proj[:, di:di + ch]
        dtt = proj[:, di + ch:di + ch + H]
        lamt = proj[:, di + ch + H:di + ch + H + H * L].reshape(Bn, H, L)
        window[:, :, :K - 1] = window[:, :, 1:].copy()
        window[:, :, K - 1] = xbct
        c = np.einsum("bck,ck->bc", window, conv_w) + conv_b
        c = c * 0.5 * (1.0 + np.tanh(0.5 * c))                   # silu
        xt = c[:, :di].reshape(Bn, H, P)
        Bt = c[:, di:di + G * N].reshape(Bn, G, N)
        Ct = c[:, di + G * N:].reshape(Bn, G, N)
        dt = np.logaddexp(0.0, dtt + dt_bias)                     # softplus, [B, H]
        a = np.exp(-dt * np.exp(A_log))                           # [B, H]
        yt = np.zeros((Bn, H, P))
        if ssm == "fenwick":
            qh = np.stack([Ct[:, hh // heads_per_group] for hh in range(H)], axis=1)
            kh = np.stack([Bt[:, hh // heads_per_group] for hh in range(H)], axis=1)
            lam = np.logaddexp(0.0, lamt + lam_bias)
            o = _forms.recurrent_step(state, qh.reshape(Bn * H, N), kh.reshape(Bn * H, N),
                                      (xt * dt[..., None]).reshape(Bn * H, P), a.reshape(Bn * H),
                                      lam.reshape(Bn * H, L))
            yt = o.reshape(Bn, H, P)
        else:
            for hh in range(H):
                gi = hh // heads_per_group
                h[:, hh] = (a[:, hh, None, None] * h[:, hh]
                            + dt[:, hh, None, None] * xt[:, hh, :, None] * Bt[:, gi, None, :])
                yt[:, hh] = np.einsum("bpn,bn->bp", h[:, hh], Ct[:, gi])
        yt = yt + Dsk[None, :, None] * xt
        gt = yt.reshape(Bn, di) * (zt / (1.0 + np.exp(-zt)))
        size = di // G
        for gi in range(G):
            seg = gt[:, gi * size:(gi + 1) * size]
            gt[:, gi * size:(gi + 1) * size] = seg / np.sqrt((seg ** 2).sum(axis=1, keepdims=True) / size + eps)
        out[:, t] = (gt * norm_w) @ W_out.T
    return out
