"""Python binding of liblogattn (log-linear Mamba-2 attention on gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``liblogattn.so``.  PyTorch provides device memory and streams.
The functions carry the C ABI's names (see include/logattn.h).  There is no
CPU fallback: if the library is missing or the tensors are not on a GPU, the
call raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "LogAttnError", "lib", "loglinear_fwd", "loglinear_fwd_workspace", "loglinear_fwd_num_stages",
    "loglinear_fwd_staged", "loglinear_fwd_noalloc", "loglinear_bwd", "loglinear_bwd_workspace", "LogLinearState", "loglinear_state_init", "loglinear_decode_step",
    "loglinear_level_table", "loglinear_strerror", "loglinear_gdn_fwd", "loglinear_gdn_fwd_workspace",
    "loglinear_mamba2_fwd", "loglinear_mamba2_fwd_workspace", "MAMBA2_WEIGHTS", "LA_F32", "LA_BF16",
]

LA_F32, LA_BF16 = 0, 1
_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblogattn.so")
_lib = None

_i, _i64, _p, _sz = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t


class _LaState(ctypes.Structure):
    _fields_ = [("t", _i64), ("B", _i), ("H", _i), ("dk", _i), ("dv", _i), ("S", _i),
                ("slots", _p), ("scale", _p)]


class _Mamba2Dims(ctypes.Structure):
    _fields_ = [("B", _i), ("T", _i64), ("d_model", _i), ("H", _i), ("P", _i), ("N", _i), ("G", _i), ("K", _i),
                ("C", _i), ("L", _i), ("eps", ctypes.c_float), ("dtype", _i)]


MAMBA2_WEIGHTS = ("in_proj", "conv_w", "conv_b", "dt_bias", "A_log", "D", "lam_bias", "norm_w", "out_proj")


class _Mamba2Weights(ctypes.Structure):
    _fields_ = [(n, _p) for n in MAMBA2_WEIGHTS]


_SIGS = {
    "loglinear_strerror": ([_i], ctypes.c_char_p),
    "loglinear_version": ([], _i),
    "loglinear_fwd_workspace": ([_i, _i, _i64, _i, _i, _i, _i, ctypes.POINTER(_sz)], _i),
    "loglinear_fwd_num_stages": ([_i, _i, _i64, _i, _i, _i, _i, ctypes.POINTER(_i)], _i),
    "loglinear_fwd": ([_p, _p, _p, _p, _p, _p, _i, _i, _i64, _i, _i, _i, _i, _i, _p, _sz, _p], _i),
    "loglinear_fwd_staged": ([_p, _p, _p, _p, _p, _p, _i, _i, _i64, _i, _i, _i, _i, _i, _p, _sz,
                              ctypes.POINTER(_p), _i, _p], _i),
    "loglinear_fwd_noalloc": ([_p, _p, _p, _p, _p, _p, _i, _i, _i64, _i, _i, _i, _i, _i, _p], _i),
    "loglinear_fwd_state": ([_p, _p, _p, _p, _p, _p, _i, _i, _i64, _i, _i, _i, _i, _i, _p, _sz,
                             ctypes.POINTER(_LaState), _p], _i),
    "loglinear_bwd_workspace": ([_i, _i, _i64, _i, _i, _i, _i, ctypes.POINTER(_sz)], _i),
    "loglinear_bwd": ([_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i64, _i, _i, _i, _i, _i, _p, _sz, _p], _i),
    "loglinear_bwd_from_fwd": ([_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i64, _i, _i, _i, _i, _i, _p, _sz,
                                _p, _sz, _p], _i),
    "loglinear_state_bytes": ([_i, _i, _i, _i, _i, ctypes.POINTER(_sz), ctypes.POINTER(_sz)], _i),
    "loglinear_state_init": ([ctypes.POINTER(_LaState), _i, _i, _i, _i, _i, _p, _p, _p], _i),
    "loglinear_decode_step": ([ctypes.POINTER(_LaState), _p, _p, _p, _p, _p, _p, _i, _p], _i),
    "loglinear_level_table": ([_i64, _i, _p, _p], _i),
    "loglinear_gdn_fwd_workspace": ([_i, _i, _i64, _i, _i, _i, _i, ctypes.POINTER(_sz)], _i),
    "loglinear_gdn_fwd": ([_p, _p, _p, _p, _p, _p, _p, _i, _i, _i64, _i, _i, _i, _i, _i, _p, _sz, _p], _i),
    "loglinear_mamba2_fwd_workspace": ([ctypes.POINTER(_Mamba2Dims), ctypes.POINTER(_sz)], _i),
    "loglinear_mamba2_fwd": ([_p, ctypes.POINTER(_Mamba2Weights), _p, ctypes.POINTER(_Mamba2Dims), _p, _sz, _p], _i),
}


class LogAttnError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: liblogattn error {code} ({loglinear_strerror(code)})")


def lib() -> ctypes.CDLL:
    """Load liblogattn.so (built in-tree by ``python -m fenwick_tree_hierarchical_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run `python -m fenwick_tree_hierarchical_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def loglinear_strerror(code: int) -> str:
    return lib().loglinear_strerror(int(code)).decode()


def _check(rc: int, where: str) -> None:
    if rc != 0:
        raise LogAttnError(rc, where)


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return LA_F32
    if t == torch.bfloat16:
        return LA_BF16
    raise TypeError(f"unsupported dtype {t}; use float32 or bfloat16")


def _dev(*ts: torch.Tensor) -> torch.device:
    dev = ts[0].device
    for t in ts:
        if t.device.type != "cuda":
            raise ValueError("liblogattn runs on the GPU only: pass device tensors")
        if t.device != dev:
            raise ValueError("all tensors must be on the same device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    return dev


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def loglinear_fwd_workspace(B: int, H: int, T: int, dk: int, dv: int, C: int, dtype: torch.dtype) -> int:
    n = _sz(0)
    _check(lib().loglinear_fwd_workspace(B, H, T, dk, dv, C, _dtype_code(dtype), ctypes.byref(n)),
           "loglinear_fwd_workspace")
    return n.value


def loglinear_fwd_num_stages(B: int, H: int, T: int, dk: int, dv: int, C: int, dtype: torch.dtype) -> int:
    n = _i(0)
    _check(lib().loglinear_fwd_num_stages(B, H, T, dk, dv, C, _dtype_code(dtype), ctypes.byref(n)),
           "loglinear_fwd_num_stages")
    return n.value


def _fwd_args(q, k, v, log_a, lam, out, chunk, workspace):
    dev = _dev(q, k, v, log_a, lam)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or log_a.shape != (B, H, T) or lam.shape[:3] != (B, H, T):
        raise ValueError("shape mismatch between q, k, v, log_a and lambda")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    if log_a.dtype != torch.float32 or lam.dtype != torch.float32:
        raise TypeError("log_a and lambda must be float32")
    if out is None:
        out = torch.empty(B, H, T, dv, dtype=q.dtype, device=dev)
    _dev(q, out)
    if out.shape != (B, H, T, dv) or out.dtype != q.dtype:
        raise ValueError("out has the wrong shape or dtype")
    nws = loglinear_fwd_workspace(B, H, T, dk, dv, chunk, q.dtype)
    if workspace is None or workspace.numel() < nws:
        workspace = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(log_a), _ptr(lam), _ptr(out), B, H, T, dk, dv, chunk,
            lam.shape[-1], _dtype_code(q.dtype), _ptr(workspace), workspace.numel()]
    return args, out, workspace, dev


def loglinear_fwd(q, k, v, log_a, lam, out=None, chunk: int = 64, workspace=None):
    """out = (Q K^T . M^S . M^H) V for every (batch, head).

    q, k: [B,H,T,dk]; v: [B,H,T,dv] (float32 or bfloat16); log_a: [B,H,T]
    float32; lam: [B,H,T,L] float32.  Returns out [B,H,T,dv] in q's dtype.
    """
    args, out, _, dev = _fwd_args(q, k, v, log_a, lam, out, chunk, workspace)
    _check(lib().loglinear_fwd(*args, _stream(dev)), "loglinear_fwd")
    return out


def loglinear_fwd_staged(q, k, v, log_a, lam, events, out=None, chunk: int = 64, workspace=None):
    """loglinear_fwd recording the given torch.cuda.Events around each stage
    (len(events) == number of stages + 1) on the current stream."""
    args, out, _, dev = _fwd_args(q, k, v, log_a, lam, out, chunk, workspace)
    s = torch.cuda.current_stream(dev)
    for e in events:                       # torch creates the HIP event lazily
        if e.cuda_event == 0:
            e.record(s)
    arr = (_p * len(events))(*[e.cuda_event for e in events])
    _check(lib().loglinear_fwd_staged(*args, arr, len(events), s.cuda_stream), "loglinear_fwd_staged")
    return out


def loglinear_fwd_noalloc(q, k, v, log_a, lam, out, chunk: int = 64):
    """loglinear_fwd into the caller's ``out`` with the library's fixed
    per-GPU scratch instead of a workspace (nothing is allocated).  Calls that
    overlap in time on one GPU share that scratch and must not overlap."""
    dev = _dev(q, k, v, log_a, lam, out)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or log_a.shape != (B, H, T) or lam.shape[:3] != (B, H, T):
        raise ValueError("shape mismatch between q, k, v, log_a and lambda")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    if log_a.dtype != torch.float32 or lam.dtype != torch.float32:
        raise TypeError("log_a and lambda must be float32")
    if out.shape != (B, H, T, dv) or out.dtype != q.dtype:
        raise ValueError("out has the wrong shape or dtype")
    _check(lib().loglinear_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(log_a), _ptr(lam), _ptr(out), B, H, T, dk,
                                       dv, chunk, lam.shape[-1], _dtype_code(q.dtype), _stream(dev)),
           "loglinear_fwd_noalloc")
    return out


def loglinear_gdn_fwd_workspace(B: int, H: int, T: int, dk: int, dv: int, C: int, dtype: torch.dtype) -> int:
    n = _sz(0)
    _check(lib().loglinear_gdn_fwd_workspace(B, H, T, dk, dv, C, _dtype_code(dtype), ctypes.byref(n)),
           "loglinear_gdn_fwd_workspace")
    return n.value


def loglinear_gdn_fwd(q, k, v, log_a, beta, lam, out=None, chunk: int = 64, workspace=None):
    """Log-linear Gated DeltaNet forward for every (batch, head).

    q, k: [B,H,T,dk]; v: [B,H,T,dv] (float32 or bfloat16); log_a, beta:
    [B,H,T] float32; lam: [B,H,T,L] float32.  Returns out [B,H,T,dv] in q's
    dtype.
    """
    dev = _dev(q, k, v, log_a, beta, lam)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or log_a.shape != (B, H, T) or \
            beta.shape != (B, H, T) or lam.shape[:3] != (B, H, T):
        raise ValueError("shape mismatch between q, k, v, log_a, beta and lambda")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    if log_a.dtype != torch.float32 or beta.dtype != torch.float32 or lam.dtype != torch.float32:
        raise TypeError("log_a, beta and lambda must be float32")
    if out is None:
        out = torch.empty(B, H, T, dv, dtype=q.dtype, device=dev)
    _dev(q, out)
    if out.shape != (B, H, T, dv) or out.dtype != q.dtype:
        raise ValueError("out has the wrong shape or dtype")
    nws = loglinear_gdn_fwd_workspace(B, H, T, dk, dv, chunk, q.dtype)
    if workspace is None or workspace.numel() < nws:
        workspace = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    _check(lib().loglinear_gdn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_a), _ptr(beta), _ptr(lam), _ptr(out),
                                   B, H, T, dk, dv, chunk, lam.shape[-1], _dtype_code(q.dtype),
                                   _ptr(workspace), workspace.numel(), _stream(dev)), "loglinear_gdn_fwd")
    return out


def loglinear_bwd_workspace(B: int, H: int, T: int, dk: int, dv: int, C: int, dtype: torch.dtype) -> int:
    n = _sz(0)
    _check(lib().loglinear_bwd_workspace(B, H, T, dk, dv, C, _dtype_code(dtype), ctypes.byref(n)),
           "loglinear_bwd_workspace")
    return n.value


def loglinear_bwd(q, k, v, log_a, lam, dout, chunk: int = 64, workspace=None, grads=None, fwd_workspace=None):
    """Gradients of a loss with respect to q, k, v, log_a and lam, given
    dout = dL/dout of the forward.  Returns (dq, dk, dv, dlog_a, dlam): dq,
    dk, dv in q's dtype, dlog_a [B,H,T] and dlam [B,H,T,L] float32.  ``grads``
    optionally supplies those five output tensors.  ``fwd_workspace``: the
    workspace of the loglinear_fwd call on these inputs (same chunk), kept
    unchanged since; the backward then reuses its bucket structure
    (loglinear_bwd_from_fwd)."""
    dev = _dev(q, k, v, log_a, lam, dout)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    L = lam.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or log_a.shape != (B, H, T) or lam.shape[:3] != (B, H, T):
        raise ValueError("shape mismatch between q, k, v, log_a and lambda")
    if dout.shape != v.shape or dout.dtype != q.dtype or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v and dout must share one dtype, dout the shape of v")
    if log_a.dtype != torch.float32 or lam.dtype != torch.float32:
        raise TypeError("log_a and lambda must be float32")
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
                 torch.empty(B, H, T, dtype=torch.float32, device=dev),
                 torch.empty(B, H, T, L, dtype=torch.float32, device=dev))
    gq, gk, gv, gla, glam = grads
    _dev(q, gq, gk, gv, gla, glam)
    if (gq.shape, gk.shape, gv.shape, gla.shape, glam.shape) != (q.shape, k.shape, v.shape, log_a.shape, lam.shape):
        raise ValueError("gradient tensors have the wrong shapes")
    if gq.dtype != q.dtype or gk.dtype != q.dtype or gv.dtype != q.dtype or gla.dtype != torch.float32 \
            or glam.dtype != torch.float32:
        raise TypeError("gradient tensors have the wrong dtypes")
    nws = loglinear_bwd_workspace(B, H, T, dk, dv, chunk, q.dtype)
    if workspace is None or workspace.numel() < nws:
        workspace = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    if fwd_workspace is None:
        _check(lib().loglinear_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_a), _ptr(lam), _ptr(dout), _ptr(gq),
                                   _ptr(gk), _ptr(gv), _ptr(gla), _ptr(glam), B, H, T, dk, dv, chunk, L,
                                   _dtype_code(q.dtype), _ptr(workspace), workspace.numel(), _stream(dev)),
               "loglinear_bwd")
    else:
        _dev(q, fwd_workspace)
        if fwd_workspace.dtype != torch.uint8 or not fwd_workspace.is_contiguous():
            raise TypeError("fwd_workspace must be a contiguous uint8 tensor")
        _check(lib().loglinear_bwd_from_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_a), _ptr(lam), _ptr(dout), _ptr(gq),
                                            _ptr(gk), _ptr(gv), _ptr(gla), _ptr(glam), B, H, T, dk, dv, chunk, L,
                                            _dtype_code(q.dtype), _ptr(fwd_workspace), fwd_workspace.numel(),
                                            _ptr(workspace), workspace.numel(), _stream(dev)),
               "loglinear_bwd_from_fwd")
    return gq, gk, gv, gla, glam


class LogLinearState:
    """Decode state: t, slots [B,H,S,dk,dv] float32 and scale [B,H,S] float32
    on the device.  ``clone()`` copies it (save/restore)."""

    def __init__(self, B: int, H: int, dk: int, dv: int, S: int, device):
        self.slots = torch.empty(B, H, S, dk, dv, dtype=torch.float32, device=device)
        self.scale = torch.empty(B, H, S, dtype=torch.float32, device=device)
        self._st = _LaState(0, B, H, dk, dv, S, self.slots.data_ptr(), self.scale.data_ptr())

    @property
    def t(self) -> int:
        return self._st.t

    @t.setter
    def t(self, value: int) -> None:
        self._st.t = int(value)

    def clone(self) -> "LogLinearState":
        st = self._st
        c = LogLinearState.__new__(LogLinearState)
        c.slots = self.slots.clone()
        c.scale = self.scale.clone()
        c._st = _LaState(st.t, st.B, st.H, st.dk, st.dv, st.S, c.slots.data_ptr(), c.scale.data_ptr())
        return c


def loglinear_fwd_state(q, k, v, log_a, lam, state: LogLinearState, out=None, chunk: int = 64,
                        workspace=None):
    """loglinear_fwd that also leaves in ``state`` the recurrent state after
    the T tokens (slots of the occupied levels, scales 1, ``state.t = T``), so
    that ``loglinear_decode_step`` continues at position T.  Returns out."""
    args, out, _, dev = _fwd_args(q, k, v, log_a, lam, out, chunk, workspace)
    _dev(q, state.slots, state.scale)
    _check(lib().loglinear_fwd_state(*args, ctypes.byref(state._st), _stream(dev)), "loglinear_fwd_state")
    return out


def loglinear_state_init(B: int, H: int, dk: int, dv: int, S: int, device) -> LogLinearState:
    st = LogLinearState(B, H, dk, dv, S, device)
    _check(lib().loglinear_state_init(ctypes.byref(st._st), B, H, dk, dv, S, _ptr(st.slots), _ptr(st.scale),
                                      _stream(st.slots.device)), "loglinear_state_init")
    return st


def loglinear_decode_step(state: LogLinearState, q, k, v, a, lam, out=None):
    """One token for every (batch, head): q, k [B,H,dk]; v [B,H,dv]; a [B,H]
    float32 gates in (0,1]; lam [B,H,S+1] float32.  Returns out [B,H,dv]."""
    st = state._st
    dev = _dev(q, k, v, a, lam, state.slots)
    if q.shape != (st.B, st.H, st.dk) or k.shape != q.shape or v.shape != (st.B, st.H, st.dv):
        raise ValueError("q, k, v shapes do not match the state")
    if a.shape != (st.B, st.H) or lam.shape != (st.B, st.H, st.S + 1):
        raise ValueError("a or lambda shape does not match the state")
    if a.dtype != torch.float32 or lam.dtype != torch.float32:
        raise TypeError("a and lambda must be float32")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    if out is None:
        out = torch.empty(st.B, st.H, st.dv, dtype=q.dtype, device=dev)
    _dev(q, out)
    if out.shape != (st.B, st.H, st.dv) or out.dtype != q.dtype:
        raise ValueError("out has the wrong shape or dtype")
    _check(lib().loglinear_decode_step(ctypes.byref(st), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(lam),
                                       _ptr(out), _dtype_code(q.dtype), _stream(dev)), "loglinear_decode_step")
    return out


def loglinear_level_table(T: int, C: int, device="cuda") -> torch.Tensor:
    """int8 [T,T] Fenwick level table computed on the device (-1 above the diagonal)."""
    out = torch.empty(T, T, dtype=torch.int8, device=device)
    _check(lib().loglinear_level_table(T, C, _ptr(out), _stream(out.device)), "loglinear_level_table")
    return out


def _mamba2_dims(B, T, d_model, H, P, N, G, K, C, L, eps, dtype) -> _Mamba2Dims:
    return _Mamba2Dims(B, T, d_model, H, P, N, G, K, C, L, float(eps), _dtype_code(dtype))


def loglinear_mamba2_fwd_workspace(B: int, T: int, d_model: int, H: int, P: int, N: int, G: int, K: int, C: int,
                                   L: int, eps: float, dtype: torch.dtype) -> int:
    n = _sz(0)
    d = _mamba2_dims(B, T, d_model, H, P, N, G, K, C, L, eps, dtype)
    _check(lib().loglinear_mamba2_fwd_workspace(ctypes.byref(d), ctypes.byref(n)), "loglinear_mamba2_fwd_workspace")
    return n.value


def loglinear_mamba2_fwd(u, weights, H: int, P: int, N: int, G: int, C: int = 64, eps: float = 1e-5, out=None,
                         workspace=None):
    """Log-Linear Mamba-2 layer forward: u [B, T, d_model] -> [B, T, d_model].

    ``weights`` maps the names in MAMBA2_WEIGHTS to device tensors:
    in_proj [2HP + 2GN + H + HL, d_model], conv_w [HP + 2GN, K],
    conv_b [HP + 2GN], norm_w [HP], out_proj [d_model, HP] in u's dtype;
    dt_bias, A_log, D [H] and lam_bias [H, L] float32.  K and L are read
    from conv_w and lam_bias.
    """
    w = [weights[n] for n in MAMBA2_WEIGHTS]
    dev = _dev(u, *w)
    B, T, d_model = u.shape
    K, L = weights["conv_w"].shape[1], weights["lam_bias"].shape[1]
    d_inner, conv_dim = H * P, H * P + 2 * G * N
    shapes = dict(in_proj=(2 * d_inner + 2 * G * N + H + H * L, d_model), conv_w=(conv_dim, K), conv_b=(conv_dim,),
                  dt_bias=(H,), A_log=(H,), D=(H,), lam_bias=(H, L), norm_w=(d_inner,), out_proj=(d_model, d_inner))
    for n, shp in shapes.items():
        if tuple(weights[n].shape) != shp:
            raise ValueError(f"{n} has shape {tuple(weights[n].shape)}, expected {shp}")
        want = torch.float32 if n in ("dt_bias", "A_log", "D", "lam_bias") else u.dtype
        if weights[n].dtype != want:
            raise TypeError(f"{n} must be {want}")
    if out is None:
        out = torch.empty(B, T, d_model, dtype=u.dtype, device=dev)
    _dev(u, out)
    if out.shape != (B, T, d_model) or out.dtype != u.dtype:
        raise ValueError("out has the wrong shape or dtype")
    d = _mamba2_dims(B, T, d_model, H, P, N, G, K, C, L, eps, u.dtype)
    nws = loglinear_mamba2_fwd_workspace(B, T, d_model, H, P, N, G, K, C, L, eps, u.dtype)
    if workspace is None or workspace.numel() < nws:
        workspace = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    wts = _Mamba2Weights(*[_ptr(t) for t in w])
    _check(lib().loglinear_mamba2_fwd(_ptr(u), ctypes.byref(wts), _ptr(out), ctypes.byref(d), _ptr(workspace),
                                      workspace.numel(), _stream(dev)), "loglinear_mamba2_fwd")
    return out
