"""Shared helpers of the GPU parity tests (test infrastructure only)."""

from __future__ import annotations

import multiprocessing as mp
import os
import sys

import numpy as np
import pytest
import torch

TOL = {"f32": 1e-4, "bf16": 2e-2}   # relative L2 bars for float32 / bfloat16 inputs
ROW_FACTOR = 5.0                    # per-row bar: ROW_FACTOR * TOL
ROW_FLOOR = 0.1                     # rows are judged against max(|ref row|, ROW_FLOOR * head RMS row norm)


def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but no GPU is visible")
    return torch.device("cuda:0")


def say(*a):
    """Name the case before the GPU runs it (flushed, so it survives a crash)."""
    print(*a, file=sys.stderr, flush=True)


def to_cpu(x: dict) -> dict:
    return {k: v.detach().cpu() for k, v in x.items()}


def heads(x: dict, idx) -> dict:
    """Select (b, h) pairs (a list of tuples) as a [1, n, ...] batch."""
    out = {}
    for k, v in x.items():
        out[k] = torch.stack([v[b, h] for b, h in idx])[None]
    return out


def effective_slots(state) -> torch.Tensor:
    """scale * slots of a decode state: the bucket matrices themselves
    ([B, H, S, dk, dv]); the library keeps each slot's gate as a lazy scale."""
    return state.slots * state.scale[..., None, None]


def _f64(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def rel_l2(x, ref) -> float:
    x = _f64(x)
    ref = _f64(ref)
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-300))


def parity(got, ref, lead: int = 2) -> dict:
    """Three views of the error of ``got`` against ``ref``:

    * ``whole``: relative L2 over the whole tensor;
    * ``head``: the worst relative L2 over the leading ``lead`` axes (one
      value per (batch, head)), so that one wrong head cannot hide under the
      norm of the others;
    * ``row``: the worst relative error of one row (the last axis), each row
      judged against max(|ref row|, ROW_FLOOR * the RMS row norm of its head),
      so that one wrong row cannot hide under the norm of its head.
    Returns the three values and where the worst head and row are."""
    g, r = _f64(got), _f64(ref)
    if g.shape != r.shape:
        raise AssertionError(f"shape {g.shape} != reference shape {r.shape}")
    res = {"whole": rel_l2(g, r), "head": 0.0, "row": 0.0, "worst_head": None, "worst_row": None}
    if g.size == 0:
        return res
    nh = int(np.prod(g.shape[:lead])) if lead else 1
    gh = g.reshape(nh, -1, g.shape[-1]) if g.ndim > lead else g.reshape(nh, -1, 1)
    rh = r.reshape(gh.shape)
    dn = np.linalg.norm(gh - rh, axis=-1)            # [heads, rows]
    rn = np.linalg.norm(rh, axis=-1)
    hd = np.sqrt((dn ** 2).sum(-1))
    hr = np.sqrt((rn ** 2).sum(-1))
    per_head = np.where(hr > 0, hd / np.where(hr > 0, hr, 1.0), np.where(hd > 0, np.inf, 0.0))
    i = int(np.argmax(per_head))
    res["head"], res["worst_head"] = float(per_head[i]), np.unravel_index(i, g.shape[:lead]) if lead else ()
    rms = np.sqrt((rn ** 2).mean(-1, keepdims=True))
    den = np.maximum(rn, ROW_FLOOR * rms)
    per_row = np.where(den > 0, dn / np.where(den > 0, den, 1.0), np.where(dn > 0, np.inf, 0.0))
    j = int(np.argmax(per_row))
    res["row"], res["worst_row"] = float(per_row.flat[j]), np.unravel_index(j, per_row.shape)
    return res


def assert_parity(got, ref, tol: float, label: str, lead: int = 2) -> dict:
    """Whole-tensor relative L2 <= tol, worst (batch, head) relative L2 <= tol
    and worst row relative error <= ROW_FACTOR * tol; prints all three.  A
    head of a single row is a row, and is held to the row bar."""
    p = parity(got, ref, lead)
    say(f"   {label}: rel_l2 whole={p['whole']:.3e} worst head={p['head']:.3e} (at {p['worst_head']}) "
        f"worst row={p['row']:.3e} (at {p['worst_row']})")
    g = np.shape(got)
    rows_per_head = int(np.prod(g[lead:-1])) if len(g) > lead + 1 else 1
    head_tol = tol if rows_per_head > 1 else ROW_FACTOR * tol
    assert p["whole"] <= tol, f"{label}: rel_l2 {p['whole']:.3e} > {tol}"
    assert p["head"] <= head_tol, f"{label}: worst head rel_l2 {p['head']:.3e} > {head_tol} at {p['worst_head']}"
    assert p["row"] <= ROW_FACTOR * tol, \
        f"{label}: worst row error {p['row']:.3e} > {ROW_FACTOR * tol} at {p['worst_row']}"
    return p


def assert_scaled(got, ref, scale, tol: float, label: str, lead: int = 2) -> dict:
    """For a quantity whose rounding follows a separate scale (the gate
    gradient: a reverse sum of terms that cancel): ||got - ref|| / ||scale||
    <= tol over the whole tensor and over each (batch, head), and every
    element |got - ref| <= ROW_FACTOR * tol * max(scale, ROW_FLOOR * the RMS
    scale of its head)."""
    g, r, sc = _f64(got), _f64(ref), np.abs(_f64(scale))
    nh = int(np.prod(g.shape[:lead]))
    d = np.abs(g - r).reshape(nh, -1)
    sc = sc.reshape(nh, -1)
    whole = float(np.linalg.norm(d) / max(np.linalg.norm(sc), 1e-300))
    per_head = np.linalg.norm(d, axis=-1) / np.maximum(np.linalg.norm(sc, axis=-1), 1e-300)
    rms = np.sqrt((sc ** 2).mean(-1, keepdims=True))
    per_el = d / np.maximum(np.maximum(sc, ROW_FLOOR * rms), 1e-300)
    j = int(np.argmax(per_el))
    res = {"whole": whole, "head": float(per_head.max()), "row": float(per_el.flat[j]),
           "worst_row": np.unravel_index(j, per_el.shape)}
    say(f"   {label}: scaled error whole={whole:.3e} worst head={res['head']:.3e} "
        f"worst element={res['row']:.3e} (at {res['worst_row']})")
    assert whole <= tol, f"{label}: scaled error {whole:.3e} > {tol}"
    assert res["head"] <= tol, f"{label}: worst head scaled error {res['head']:.3e} > {tol}"
    assert res["row"] <= ROW_FACTOR * tol, f"{label}: worst element {res['row']:.3e} > {ROW_FACTOR * tol}"
    return res


# ------------------------------------------------- oracle over a process pool
def _task_recurrent(q, k, v, log_a, lam):
    """One (batch, head) through the oracle's token-by-token recurrence."""
    from oracle import forms
    out, _ = forms.forward_recurrent(q[None, None], k[None, None], v[None, None], lam[None, None],
                                     log_a=log_a[None, None])
    return out[0, 0]


def _task_gdn(q, k, v, log_a, beta, lam):
    """One (batch, head) through the Gated DeltaNet oracle's recurrence."""
    from oracle import deltanet
    out, _ = deltanet.gdn_forward_recurrent(q[None, None], k[None, None], v[None, None], log_a[None, None],
                                            beta[None, None], lam[None, None])
    return out[0, 0]


def _task_dlog_a(q, k, v, log_a, lam, dout, r):
    """The gate gradient of one (batch, head) at position r."""
    from oracle import backward
    return backward.dlog_a_rows(q[None, None], k[None, None], v[None, None], log_a[None, None],
                                lam[None, None], dout[None, None], [r])[0, 0, 0]


_TASKS = {"recurrent": _task_recurrent, "gdn": _task_gdn, "dlog_a": _task_dlog_a}


def _run_task(item):
    kind, args = item
    return _TASKS[kind](*args)


def host_workers() -> int:
    """Worker processes for the oracle: the host cores this process may use,
    at most 16 (the host share of one GPU)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _np64(t):
    return t.detach().cpu().double().numpy() if isinstance(t, torch.Tensor) else np.asarray(t)


class OraclePool:
    """Oracle calls over independent (batch, head) tasks in worker processes
    started fresh (spawn: they never touch the GPU), one thread each.
    Submitted before the GPU call, so both run at once.

    kind "recurrent": x holds q, k, v, log_a, lam of CPU tensors [B, H, ...];
    the result is the recurrence's output [B, H, T, dv].
    kind "gdn": the same plus beta; the Gated DeltaNet recurrence's output.
    kind "dlog_a": the same plus dout and ``rows``; the gate gradient at those
    rows, [B, H, len(rows)]."""

    def __init__(self, x: dict, workers: int | None = None, kind: str = "recurrent", rows=None):
        names = {"recurrent": ("q", "k", "v", "log_a", "lam"), "gdn": ("q", "k", "v", "log_a", "beta", "lam"),
                 "dlog_a": ("q", "k", "v", "log_a", "lam", "dout")}[kind]
        B, H = x["q"].shape[:2]
        if kind == "dlog_a":
            rows = [int(r) for r in rows]
            self.shape = (B, H, len(rows))
            tasks = [(kind, tuple(_np64(x[n][b, h]) for n in names) + (r,))
                     for b in range(B) for h in range(H) for r in rows]
        else:
            self.shape = (B, H, x["q"].shape[2], x["v"].shape[3])
            tasks = [(kind, tuple(_np64(x[n][b, h]) for n in names)) for b in range(B) for h in range(H)]
        n = min(workers or host_workers(), max(1, len(tasks)))
        saved = {v: os.environ.get(v) for v in _THREAD_VARS}
        os.environ.update({v: "1" for v in _THREAD_VARS})      # inherited by the spawned workers
        try:
            self._pool = mp.get_context("spawn").Pool(n)
        finally:
            for v, val in saved.items():
                if val is None:
                    os.environ.pop(v, None)
                else:
                    os.environ[v] = val
        self._res = self._pool.map_async(_run_task, tasks, chunksize=1)

    def result(self, timeout: float = 900.0) -> np.ndarray:
        try:
            outs = self._res.get(timeout)
        finally:
            self._pool.terminate()
            self._pool.join()
        return np.asarray(np.stack(outs)).reshape(self.shape)


_THREAD_VARS = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")
