"""Benchmark of log-linear Mamba-2 attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-decode] [--no-backward] [--no-gdn]

One step is one forward (``loglinear_fwd``, all of its kernels) over the
training-shape layer B=8, H=16, T=16384, d_k=d_v=64, C=64 in bfloat16, with
every input already resident in HBM.  Prints ONE JSON line:

  value          tokens/s, a token being one sequence position across all
                 H heads (B*T per step)
  roofline       for the dominant kernel (fwd_chunk_output): algorithmic
                 bytes per launch / its mean duration from HIP events
                 recorded on the launch stream around each kernel, over a
                 second pass of as many steps right after the timed ones
                 (the timed steps run without events; `ms_per_step_staged`
                 is that pass).  The events are timing-only ones created
                 with hipEventDisableSystemFence, so recording one writes
                 back and invalidates no caches (`stage_events` says which
                 kind ran),
                 against 8 TB/s; `traffic` is the counter-measured HBM
                 bytes per launch from profiles/ when those counters were
                 taken on the current kernel source, else null
  cpu_baseline   the float64 oracle timed on the host cores (worker
                 processes, one thread each): its recurrence over every
                 head of the same workload in full, plus the tiny, small and
                 decode workloads
  stages         per kernel (chunk_states, group_tree, chunk_output): mean
                 time, algorithmic bytes, GB/s and counter traffic
  layer_frac     the layer's essential bytes (q, k, v, out, log_a, lambda)
                 per timed step against 8 TB/s
  mfma           the matrix-core share of the whole forward (per timed step)
  configs        the other forward workloads (tiny fp32, small bf16, the
                 128K long-context shape): time, tokens/s, per-kernel HBM
                 fractions and layer_frac
  backward       the backward (loglinear_bwd) on the same layer with a
                 seeded upstream gradient: mean time, tokens/s and its ratio
                 to the forward; `from_forward` the same backward handed the
                 forward's workspace (loglinear_bwd_from_fwd)
  gdn            the log-linear Gated DeltaNet forward (loglinear_gdn_fwd)
                 on the same layer shape with seeded beta: mean time,
                 tokens/s, algorithmic TFLOP/s against the bf16 peak
  decode         the decode workload (64 x 16 heads): the 32768-token
                 prefill handing its state to decode (loglinear_fwd_state),
                 then 256 decode steps, positions 32768..33023

Other modes (profiling helpers):
  --pmc-summary DIR   parse a rocprofv3 --pmc output directory (FETCH_SIZE
                      or WRITE_SIZE) and print per-kernel counters
  --copy-calibration  also run a plain 1 GiB device copy each step, so a
                      counter run sees a kernel of known traffic
  --rocpd-summary F   markdown table of kernel statistics from a rocprofv3
                      results database (.db) or kernel_stats.csv
  --trace-summary F   markdown table of a rocprofv3 kernel_trace.csv, one row
                      per kernel and grid size
  --pmc-profile FETCH_DIR WRITE_DIR
                      write profiles/fwd_chunk_output_train16k_pmc.json from
                      a FETCH_SIZE and a WRITE_SIZE run (both taken with
                      --copy-calibration)
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fwd tokens/s, log-linear Mamba-2 attn, T=16K, H=16, d=64; % MFMA peak"
HBM_PEAK_GBPS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2516.6      # 256 CU x 2.4 GHz x 4096 flop/clk (dense)
KERNEL_SOURCES = ["fenwick_tree_hierarchical_amd/csrc/la_fwd_impl.hpp",
                  "fenwick_tree_hierarchical_amd/csrc/la_device.hpp",
                  "fenwick_tree_hierarchical_amd/csrc/la_plan.hpp"]
PMC_FILE = os.path.join(ROOT, "profiles", "fwd_chunk_output_train16k_pmc.json")
# kernel name fragment -> stage name used in the JSON line
KERNELS = {"fwd_chunk_states": "chunk_states", "fwd_group_tree": "group_tree", "fwd_chunk_output": "chunk_output"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class TimingEvent:
    """A HIP event used only to time the kernels between two records,
    created with hipEventDisableSystemFence: its record performs no
    system-scope cache writeback and invalidation, which would otherwise add
    to the span it measures and leave the next kernel with cold caches.  It
    is read only after a device synchronize.  Exposes the two members the
    staged entry point and the bench use (`cuda_event`, `elapsed_time`)."""
    FLAGS = 0x20000000      # hipEventDisableSystemFence
    _hip = None

    def __init__(self):
        import ctypes
        if TimingEvent._hip is None:
            TimingEvent._hip = ctypes.CDLL("libamdhip64.so")
        h = ctypes.c_void_p()
        rc = TimingEvent._hip.hipEventCreateWithFlags(ctypes.byref(h), ctypes.c_uint(self.FLAGS))
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.cuda_event = h.value

    def elapsed_time(self, end) -> float:
        import ctypes
        ms = ctypes.c_float()
        rc = TimingEvent._hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.cuda_event),
                                                  ctypes.c_void_p(end.cuda_event))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        h = getattr(self, "cuda_event", None)
        if TimingEvent._hip is not None and h:
            import ctypes
            TimingEvent._hip.hipEventDestroy(ctypes.c_void_p(h))


def stage_events(torch, n: int):
    """n timing events for the staged steps, and their kind: fence-free HIP
    events, or torch's when the HIP runtime library cannot be opened."""
    try:
        return [TimingEvent() for _ in range(n)], "hip, hipEventDisableSystemFence"
    except (OSError, AttributeError, RuntimeError):
        return [torch.cuda.Event(enable_timing=True) for _ in range(n)], "torch.cuda.Event"


def _code_only(text: str) -> str:
    """C++ source without comments and whitespace: what the compiler sees."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return "".join(text.split())


def kernel_source_hash(read=None) -> str:
    """Hash of the forward kernels' source, comments and whitespace ignored."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        if read is None:
            with open(os.path.join(ROOT, p)) as f:
                text = f.read()
        else:
            text = read(p)
        h.update(_code_only(text).encode())
    return h.hexdigest()[:16]


def algorithmic_counts(w, B, H, T, d, C, L, es, G=8):
    """Work the method itself does (no dense-equivalent inflation).

    Bytes: the essential I/O -- q, k, v, out in the layer dtype plus log_a
    and lambda in float32 -- and, per kernel, the state bytes it must move:
      chunk_states   reads k, v, log_a; writes the bucket node ending at each
                     full chunk inside its group of G chunks (bf16) and each
                     full group's state (fp32) and gate total
      group_tree     reads the full groups' states; writes the bucket node
                     ending at each of them (bf16) and the gate prefix
      chunk_output   reads q, k, v, log_a, lambda and every bucket node some
                     later chunk needs, once; writes out
    Flops: the dense C x C intra-chunk tiles 2 C^2 (d_k + d_v) per chunk, one
    chunk state 2 C d_k d_v per chunk, and 2 C d_k d_v per chunk for each
    occupied chunk-or-group level (popcount of the chunk index)."""
    n_chunks = math.ceil(T / C)
    n_groups = math.ceil(n_chunks / G)
    BH = B * H
    per_head_token_bytes = 4 * d * es + 4 + 4 * L
    bytes_io = BH * T * per_head_token_bytes
    node = d * d * es
    n_full = T // C
    n_full_groups = n_full // G
    nodes_w = sum(1 for c in range(n_full) if c % G != G - 1)                  # written
    nodes_in = sum(1 for c in range(n_chunks) if c % G != G - 1 and c + 1 < n_chunks)   # read
    nodes_grp = max(n_groups - 1, 0)                                           # read
    kern = {
        "chunk_states": BH * (T * (2 * d * es + 4) + nodes_w * node + n_full_groups * (d * d * 4 + 4)
                              + n_chunks * 4),
        "group_tree": BH * (n_full_groups * (d * d * 4 + 4 + node) + (n_full_groups + 1) * 8),
        "chunk_output": bytes_io + BH * ((nodes_in + nodes_grp) * node + n_chunks * 4 + (n_groups + 1) * 8),
    }
    intra = n_chunks * 2 * C * C * (d + d)
    states = n_chunks * 2 * C * d * d
    contr = sum(bin(c).count("1") for c in range(n_chunks)) * 2 * C * d * d
    flops = BH * (intra + states + contr)
    return dict(per_head_token_bytes=per_head_token_bytes, bytes_io=bytes_io, kernel_bytes=kern,
                node_bytes_per_bh=(nodes_in + nodes_grp) * node, flops_intra=BH * intra,
                flops_states=BH * states, flops_contractions=BH * contr, flops=flops)


def host_cores() -> int:
    """Host cores this process may use, at most 16 (the host share of one GPU)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_task(item):
    """One oracle call in a worker process; returns (seconds, checksum)."""
    import numpy as np
    from oracle import forms
    kind, args = item
    t0 = time.perf_counter()
    if kind == "recurrent":
        q, k, v, la, lam = args
        out, _ = forms.forward_recurrent(q, k, v, lam, log_a=la)
    elif kind == "quadratic":
        q, k, v, la, lam = args
        out = forms.forward_quadratic(q, k, v, la, lam)
    else:                                   # "decode": steps from a state at position t0
        q, k, v, a, lam, t_start, nlev, seed = args
        BH, steps, d = q.shape
        st = forms.FenwickState(BH, d, v.shape[-1], nlev, t=t_start)
        rng = np.random.default_rng(seed)
        for lv in range(1, nlev + 1):       # the occupied levels of position t_start, values of scale 0.01
            if (t_start >> (lv - 1)) & 1:
                st.slots[:, lv] = 0.01 * rng.standard_normal(st.slots[:, lv].shape)
        out = np.stack([forms.recurrent_step(st, q[:, i], k[:, i], v[:, i], a[:, i], lam[:, i])
                        for i in range(steps)], axis=1)
    return time.perf_counter() - t0, float(np.sum(out))


def _pool_map(tasks, n):
    """Run oracle tasks over n spawned worker processes with one BLAS thread
    each; returns (wall seconds, per-task results)."""
    import multiprocessing as mp
    names = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")
    saved = {v: os.environ.get(v) for v in names}
    os.environ.update({v: "1" for v in names})
    try:
        ctx = mp.get_context("spawn")
        with ctx.Pool(min(n, len(tasks))) as pool:
            import numpy as np
            warm = tuple(np.zeros(sh, dtype=np.float32) for sh in ((1, 1, 4, 4), (1, 1, 4, 4), (1, 1, 4, 4),
                                                                   (1, 1, 4), (1, 1, 4, 3)))
            pool.map(_oracle_task, [("recurrent", warm)] * min(n, len(tasks)))     # workers started and warm
            t0 = time.perf_counter()
            res = pool.map(_oracle_task, tasks, chunksize=1)
            wall = time.perf_counter() - t0
    finally:
        for v, val in saved.items():
            if val is None:
                os.environ.pop(v, None)
            else:
                os.environ[v] = val
    return wall, res


def _head_tasks(x, kind):
    import numpy as np
    B, H = x["q"].shape[:2]
    f = lambda t: t.float().numpy()
    return [(kind, tuple(f(x[n][b:b + 1, h:h + 1]) for n in ("q", "k", "v", "log_a", "lam")))
            for b in range(B) for h in range(H)]


def cpu_baseline():
    """The float64 oracle on the host cores, as it stands: its token-by-token
    recurrence over every head of the training shape (the metric's workload,
    in full), the tiny and small workloads (recurrence and quadratic form) and
    the decode workload's 256 steps over all 1024 heads (from a state with
    the occupancy of position 32768).  Heads are spread over n worker
    processes, one thread each; wall time from the first task to the last."""
    import torch
    from fenwick_tree_hierarchical_amd.workloads import WORKLOADS, make_inputs
    n = host_cores()
    res = {"cores": n, "cpu_model": cpu_model(), "threads_per_worker": 1}
    for name in ("tiny_f32", "small_bf16", "train_16k_bf16"):
        w = WORKLOADS[name]
        x = make_inputs(w, device="cpu")
        entry = {}
        kinds = ("recurrent", "quadratic") if name != "train_16k_bf16" else ("recurrent",)
        for kind in kinds:
            wall, r = _pool_map(_head_tasks(x, kind), n)
            entry[kind] = {"seconds": wall, "tokens_per_s": w.B * w.T / wall, "heads": w.B * w.H,
                           "task_seconds": sum(t for t, _ in r)}
        res[name] = entry
        del x
    # decode: 256 steps of all 64 x 16 heads, split into n groups of heads
    w = WORKLOADS["decode_32k_bf16"]
    x = make_inputs(w, device="cpu", T=w.steps, L=17)
    BH = w.B * w.H
    q, k, v = (x[nm].float().reshape(BH, w.steps, -1).numpy() for nm in ("q", "k", "v"))
    a = torch.exp(x["log_a"]).reshape(BH, w.steps).double().numpy()
    lam = x["lam"].reshape(BH, w.steps, -1).double().numpy()
    parts = [range(i * BH // n, (i + 1) * BH // n) for i in range(n)]
    tasks = [("decode", (q[p.start:p.stop], k[p.start:p.stop], v[p.start:p.stop], a[p.start:p.stop],
                         lam[p.start:p.stop], w.prefix, 16, i)) for i, p in enumerate(parts)]
    wall, r = _pool_map(tasks, n)
    res["decode_32k_bf16"] = {"recurrent_steps": {"seconds": wall, "tokens_per_s": w.B * w.steps / wall,
                                                  "heads": BH, "steps": w.steps,
                                                  "task_seconds": sum(t for t, _ in r)}}
    main = res["train_16k_bf16"]["recurrent"]
    return {"value": main["tokens_per_s"], "unit": "tokens/s", "cores": n, "kind": "oracle",
            "sample": f"float64 Fenwick recurrence over all {main['heads']} heads of train_16k_bf16 "
                      f"(B=8, H=16, T=16384, d=64), in full: {main['seconds']:.1f} s wall on {n} worker "
                      f"processes of one thread ({main['task_seconds']:.0f} CPU-s)",
            "cpu_model": res["cpu_model"], "configs": {k: v for k, v in res.items() if k not in
                                                       ("cores", "cpu_model", "threads_per_worker")}}


def pmc_traffic(src_hash: str):
    """HBM traffic per launch of each forward kernel from the committed
    counter summary, when it was taken on the current kernel source."""
    if not os.path.exists(PMC_FILE):
        return None, "no counter summary"
    with open(PMC_FILE) as f:
        s = json.load(f)
    if s.get("kernel_source_hash") != src_hash:
        return None, "kernel changed since the counters were taken"
    return s.get("per_kernel_traffic_bytes"), None


def bench_decode(la, torch, dev, steps=256, reps=5):
    """The decode workload: a 32768-token prefill on 64 x 16 heads that hands
    its final state to decode (loglinear_fwd_state, timed against the plain
    forward over the same prefix), then 256 decode steps from that state."""
    from fenwick_tree_hierarchical_amd.workloads import WORKLOADS, make_inputs

    w = WORKLOADS["decode_32k_bf16"]
    S = 16
    B, H, d, P = w.B, w.H, w.dk, w.prefix
    x = make_inputs(w, device=dev, L=S + 1)                  # T = prefix + steps
    a = torch.exp(x["log_a"])
    pre = {k: v[:, :, :P].contiguous() for k, v in x.items()}
    pre["log_a"] = torch.log(a[:, :, :P]).contiguous()
    nws = la.loglinear_fwd_workspace(B, H, P, d, d, w.C, torch.bfloat16)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    out = torch.empty_like(pre["v"])
    st = la.loglinear_state_init(B, H, d, d, S, dev)
    stream = torch.cuda.current_stream(dev)

    def prefill(with_state):
        if with_state:
            la.loglinear_fwd_state(pre["q"], pre["k"], pre["v"], pre["log_a"], pre["lam"], st, out=out,
                                   chunk=w.C, workspace=ws)
        else:
            la.loglinear_fwd(pre["q"], pre["k"], pre["v"], pre["log_a"], pre["lam"], out=out, chunk=w.C,
                             workspace=ws)

    ms = {}
    for with_state in (False, True, False, True):            # interleaved, twice
        prefill(with_state)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            prefill(with_state)
        e1.record(stream)
        torch.cuda.synchronize()
        ms.setdefault(with_state, []).append(e0.elapsed_time(e1) / reps)
    fwd_ms, state_ms = min(ms[False]), min(ms[True])
    assert st.t == P
    # the final-state kernel: each occupied bucket's node read once (bfloat16)
    # and its slot written once (float32), every scale written
    occ = bin(P).count("1")
    st_bytes = B * H * (occ * d * d * (2 + 4) + S * 4)
    handoff = {"workload": f"{w.name} prefill", "prefix": P, "heads": B * H,
               "fwd_ms": fwd_ms, "fwd_state_ms": state_ms, "final_state_ms": state_ms - fwd_ms,
               "prefill_tokens_per_s": B * P / (state_ms * 1e-3),
               "final_state_alg_bytes": st_bytes,
               "note": "final_state_ms is the difference of the two timed calls (best of two rounds of "
                       f"{reps}); the kernel alone is in the kernel trace",
               "replaces_decode_steps": P}

    per = [(x["q"][:, :, P + i].contiguous(), x["k"][:, :, P + i].contiguous(), x["v"][:, :, P + i].contiguous(),
            a[:, :, P + i].contiguous(), x["lam"][:, :, P + i].contiguous(),
            torch.empty(B, H, d, dtype=x["q"].dtype, device=dev)) for i in range(steps)]
    L = la.lib()
    args = [(ctypes_byref(la, st), q.data_ptr(), k.data_ptr(), v.data_ptr(), aa.data_ptr(), lm.data_ptr(),
             o.data_ptr()) for q, k, v, aa, lm, o in per]
    # warm-up on a copy so the timed steps start at the workload's position
    warm = st.clone()
    for i in range(8):
        rc = L.loglinear_decode_step(ctypes_byref(la, warm), *args[i][1:], la.LA_BF16, stream.cuda_stream)
        assert rc == 0, rc
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        rc = L.loglinear_decode_step(args[i][0], *args[i][1:], la.LA_BF16, stream.cuda_stream)
        if rc:
            raise RuntimeError(la.loglinear_strerror(rc))
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = e0.elapsed_time(e1)
    # algorithmic bytes: occupied slots read once, the merged slot written once,
    # plus q, k, v, out, gate, lambda and the slot scales
    slot = d * d * 4
    tot = 0
    for t in range(P, P + steps):
        tot += (bin(t).count("1") + 1) * slot + 4 * d * 2 + 4 + (S + 1) * 4 + 2 * S * 4
    tot *= B * H
    return {"workload": w.name, "steps": steps, "launch": "eager, one launch per step",
            "state": "from the prefill hand-off", "tokens_per_s": B * steps / wall,
            "us_per_step_wall": wall / steps * 1e6, "us_per_step_gpu": gpu_ms / steps * 1e3,
            "achieved_gbps": tot / (gpu_ms * 1e-3) / 1e9, "peak_gbps": HBM_PEAK_GBPS,
            "frac": tot / (gpu_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, "alg_bytes_per_step": tot / steps,
            "handoff": handoff}


def bench_decode_large(la, torch, dev, B=256, steps=64):
    """Decode steps at batch 256 x 16 heads (1 GiB of slots, four times the
    256 MB MALL), so the slots cannot stay in the last-level cache.  The
    slots are filled with values of the right scale; the work depends only
    on which levels are occupied."""
    from fenwick_tree_hierarchical_amd.workloads import WORKLOADS, make_inputs

    w = WORKLOADS["decode_32k_bf16"]
    S, H, d, P = 16, w.H, w.dk, w.prefix
    st = la.loglinear_state_init(B, H, d, d, S, dev)
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed)
    st.slots.normal_(0, 0.01, generator=g)
    st.t = P
    x = make_inputs(w, device=dev, B=B, T=steps, L=S + 1)
    a = torch.exp(x["log_a"])
    per = [(x["q"][:, :, i].contiguous(), x["k"][:, :, i].contiguous(), x["v"][:, :, i].contiguous(),
            a[:, :, i].contiguous(), x["lam"][:, :, i].contiguous(),
            torch.empty(B, H, d, dtype=x["q"].dtype, device=dev)) for i in range(steps)]
    L = la.lib()
    stream = torch.cuda.current_stream(dev)
    warm = st.clone()
    for i in range(4):
        assert L.loglinear_decode_step(ctypes_byref(la, warm), *[t.data_ptr() for t in per[i][:5]],
                                       per[i][5].data_ptr(), la.LA_BF16, stream.cuda_stream) == 0
    del warm
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        rc = L.loglinear_decode_step(ctypes_byref(la, st), *[t.data_ptr() for t in per[i][:5]], per[i][5].data_ptr(),
                                     la.LA_BF16, stream.cuda_stream)
        if rc:
            raise RuntimeError(la.loglinear_strerror(rc))
    e1.record(stream)
    torch.cuda.synchronize()
    gpu_ms = e0.elapsed_time(e1)
    slot = d * d * 4
    tot = sum((bin(t).count("1") + 1) * slot + 4 * d * 2 + 4 + (S + 1) * 4 + 2 * S * 4
              for t in range(P, P + steps)) * B * H
    return {"batch": B, "heads": B * H, "steps": steps, "slot_bytes": B * H * S * slot,
            "us_per_step_gpu": gpu_ms / steps * 1e3, "achieved_gbps": tot / (gpu_ms * 1e-3) / 1e9,
            "frac": tot / (gpu_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}


def bench_backward(la, torch, dev, w, x, reps=10):
    """The backward (loglinear_bwd, all of its kernels) on the training shape
    with a seeded upstream gradient, timed with HIP events on the launch
    stream; then the same backward handed the forward's workspace
    (loglinear_bwd_from_fwd: the forward's bucket nodes serve its query side,
    as in a training step that keeps them).  Essential bytes: q, k, v, dout,
    log_a, lambda read and dq, dk, dv, dlog_a, dlambda written once."""
    from fenwick_tree_hierarchical_amd.workloads import make_grad_out
    dout = make_grad_out(w, device=dev)
    nws = la.loglinear_bwd_workspace(w.B, w.H, w.T, w.dk, w.dv, w.C, torch.bfloat16)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    fws = torch.empty(max(la.loglinear_fwd_workspace(w.B, w.H, w.T, w.dk, w.dv, w.C, torch.bfloat16), 1),
                      dtype=torch.uint8, device=dev)
    la.loglinear_fwd(x["q"], x["k"], x["v"], x["log_a"], x["lam"], chunk=w.C, workspace=fws)
    grads = la.loglinear_bwd(x["q"], x["k"], x["v"], x["log_a"], x["lam"], dout, chunk=w.C, workspace=ws)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream(dev)

    def timed(kw):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        la.loglinear_bwd(x["q"], x["k"], x["v"], x["log_a"], x["lam"], dout, chunk=w.C, workspace=ws, grads=grads,
                         **kw)
        torch.cuda.synchronize()
        ev[0].record(s)
        for i in range(reps):
            la.loglinear_bwd(x["q"], x["k"], x["v"], x["log_a"], x["lam"], dout, chunk=w.C, workspace=ws,
                             grads=grads, **kw)
            ev[i + 1].record(s)
        torch.cuda.synchronize()
        return [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]

    ms = timed({})
    ms_ff = timed({"fwd_workspace": fws})
    mean = sum(ms) / reps
    mean_ff = sum(ms_ff) / reps
    es = 2
    per_tok = 7 * w.dk * es + 2 * 4 + 2 * 4 * w.L
    nbytes = w.B * w.H * w.T * per_tok
    return {"workload": w.name, "chunk": w.C, "reps": reps, "ms": mean, "median_ms": sorted(ms)[reps // 2],
            "min_ms": min(ms), "tokens_per_s": w.B * w.T / (mean * 1e-3), "ratio_to_forward": None,
            "essential_bytes": nbytes, "essential_gbps": nbytes / (mean * 1e-3) / 1e9,
            "essential_bytes_note": f"{per_tok} B per head-token: q, k, v, dout read and dq, dk, dv written "
                                    f"(bf16), log_a, lambda read and dlog_a, dlambda written (fp32)",
            "from_forward": {"ms": mean_ff, "median_ms": sorted(ms_ff)[reps // 2], "min_ms": min(ms_ff),
                             "tokens_per_s": w.B * w.T / (mean_ff * 1e-3), "ratio_to_forward": None,
                             "note": "loglinear_bwd_from_fwd: the forward's workspace handed over, its bucket "
                                     "nodes serve the query side (no state and tree kernels over (v, k))"}}


def gdn_counts(B, H, T, d, C, L, es):
    """Algorithmic work of the log-linear Gated DeltaNet forward, each needed
    product counted once.  Per chunk: tril(Q K^T), K K^T, the unit-lower
    solve (about C^3), Ahat = S T (2 C^3), the carried queries Ahat K and the
    masked tile times V; per full chunk its state K^T U and transition K^T W
    with U = T (gated beta V), W = T (beta K); per merge of two blocks two
    d x d x d products; per query chunk one contraction per set bit of its
    index and one carry of the queries between consecutive set bits.
    Essential bytes: q, k, v, out in the layer dtype, log_a, beta, lambda."""
    n_chunks = -(-T // C)
    n_full = T // C
    intra = n_chunks * (8 * C * C * d + 2 * C ** 3 + C ** 3)
    prep = n_full * (4 * C * C * d + 4 * C * d * d)
    merges = sum(n_full >> m for m in range(1, 40))
    tree = merges * 4 * d ** 3
    pc = [bin(c).count("1") for c in range(n_chunks)]
    levels = sum(p * 2 * C * d * d + max(p - 1, 0) * 2 * C * d * d for p in pc)
    bh = B * H
    per_tok = 4 * d * es + 4 + 4 + 4 * L
    return {"flops": bh * (intra + prep + tree + levels),
            "split_tflop": {"intra": bh * intra / 1e12, "chunk_nodes": bh * prep / 1e12,
                            "tree": bh * tree / 1e12, "levels": bh * levels / 1e12},
            "essential_bytes": bh * T * per_tok, "per_head_token_bytes": per_tok}


def bench_gdn(la, torch, dev, w, reps=10, warmup=5):
    """The log-linear Gated DeltaNet forward (loglinear_gdn_fwd, all of its
    kernels) on the training shape, beta ~ sigmoid(N(0,1)); HIP events on the
    launch stream around each call."""
    from fenwick_tree_hierarchical_amd.workloads import make_beta, make_inputs
    x = make_inputs(w, device=dev)
    beta = make_beta(w, device=dev)
    out = torch.empty_like(x["v"])
    nws = la.loglinear_gdn_fwd_workspace(w.B, w.H, w.T, w.dk, w.dv, w.C, torch.bfloat16)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)

    def call():
        la.loglinear_gdn_fwd(x["q"], x["k"], x["v"], x["log_a"], beta, x["lam"], out=out, chunk=w.C, workspace=ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(s)
    for i in range(reps):
        call()
        ev[i + 1].record(s)
    torch.cuda.synchronize()
    ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]
    mean = sum(ms) / reps
    cnt = gdn_counts(w.B, w.H, w.T, w.dk, w.C, w.L, 2)
    tf = cnt["flops"] / (mean * 1e-3) / 1e12
    return {"workload": w.name, "chunk": w.C, "reps": reps, "ms": mean, "median_ms": sorted(ms)[reps // 2],
            "min_ms": min(ms), "tokens_per_s": w.B * w.T / (mean * 1e-3), "workspace_bytes": nws,
            "alg_tflop": cnt["flops"] / 1e12, "split_tflop": cnt["split_tflop"], "achieved_tflops": tf,
            "frac_of_bf16_peak": tf / BF16_MFMA_PEAK_TFLOPS,
            "essential_bytes": cnt["essential_bytes"],
            "essential_gbps": cnt["essential_bytes"] / (mean * 1e-3) / 1e9,
            "essential_bytes_note": f"{cnt['per_head_token_bytes']} B per head-token: q, k, v, out (bf16), "
                                    f"log_a, beta, lambda (fp32)"}


def layer_counts(lw):
    """Algorithmic work of one Log-Linear Mamba-2 layer forward: the two
    projections (2 M K N each), the conv (2 K flops per channel and token) and
    the operator's products (algorithmic_counts); essential bytes: the input
    and output activations and the weights, each once."""
    M = lw.B * lw.T
    gemm = 2 * M * lw.d_model * lw.d_in_proj + 2 * M * lw.d_inner * lw.d_model
    conv = 2 * lw.K * M * lw.conv_dim
    op = algorithmic_counts(None, lw.B, lw.H, lw.T, lw.N, lw.C, lw.L, 2, G=8 if lw.N <= 64 else 4)["flops"]
    es = 2 if lw.dtype == "bf16" else 4
    weights = (lw.d_in_proj * lw.d_model + lw.conv_dim * (lw.K + 1) + lw.d_inner + lw.d_model * lw.d_inner) * es \
        + (3 * lw.H + lw.H * lw.L) * 4
    return {"flops": gemm + conv + op, "split_tflop": {"projections": gemm / 1e12, "conv": conv / 1e12,
                                                       "operator": op / 1e12},
            "essential_bytes": 2 * M * lw.d_model * es + weights}


def bench_layer(la, torch, dev, lw, reps=10, warmup=5):
    """The Log-Linear Mamba-2 layer forward (loglinear_mamba2_fwd: projections,
    conv and gates, the operator, gate and norm) on its training shape; HIP
    events on the launch stream around each call."""
    from fenwick_tree_hierarchical_amd.workloads import make_layer
    w = {k: v.to(dev) for k, v in make_layer(lw).items()}
    out = torch.empty_like(w["u"])
    nws = la.loglinear_mamba2_fwd_workspace(lw.B, lw.T, lw.d_model, lw.H, lw.P, lw.N, lw.G, lw.K, lw.C, lw.L,
                                            lw.eps, w["u"].dtype)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)

    def call():
        la.loglinear_mamba2_fwd(w["u"], w, lw.H, lw.P, lw.N, lw.G, C=lw.C, eps=lw.eps, out=out, workspace=ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(s)
    for i in range(reps):
        call()
        ev[i + 1].record(s)
    torch.cuda.synchronize()
    ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]
    mean = sum(ms) / reps
    cnt = layer_counts(lw)
    tf = cnt["flops"] / (mean * 1e-3) / 1e12
    return {"workload": lw.name, "B": lw.B, "T": lw.T, "d_model": lw.d_model, "H": lw.H, "P": lw.P, "N": lw.N,
            "G": lw.G, "K": lw.K, "chunk": lw.C, "reps": reps, "ms": mean, "median_ms": sorted(ms)[reps // 2],
            "min_ms": min(ms), "tokens_per_s": lw.B * lw.T / (mean * 1e-3), "workspace_bytes": nws,
            "alg_tflop": cnt["flops"] / 1e12, "split_tflop": cnt["split_tflop"], "achieved_tflops": tf,
            "frac_of_bf16_peak": tf / BF16_MFMA_PEAK_TFLOPS, "essential_bytes": cnt["essential_bytes"]}


def bench_config(la, torch, dev, w, steps=20, warmup=10):
    """One forward workload (not the metric's): wall time per forward over
    `steps` calls after `warmup`, then the kernels' durations from HIP events
    between the stages over as many calls; algorithmic bytes per kernel and
    the layer's essential bytes against the HBM peak."""
    from fenwick_tree_hierarchical_amd.workloads import make_inputs, torch_dtype
    x = make_inputs(w, device=dev)
    dt = torch_dtype(w.dtype)
    es = 2 if w.dtype == "bf16" else 4
    out = torch.empty_like(x["v"])
    nws = la.loglinear_fwd_workspace(w.B, w.H, w.T, w.dk, w.dv, w.C, dt)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    n_st = la.loglinear_fwd_num_stages(w.B, w.H, w.T, w.dk, w.dv, w.C, dt)
    names = {3: ["chunk_states", "group_tree", "chunk_output"], 2: ["chunk_states", "chunk_output"],
             1: ["chunk_output"]}[n_st]

    def call(ev=None):
        if ev is None:
            la.loglinear_fwd(x["q"], x["k"], x["v"], x["log_a"], x["lam"], out=out, chunk=w.C, workspace=ws)
        else:
            la.loglinear_fwd_staged(x["q"], x["k"], x["v"], x["log_a"], x["lam"], ev, out=out, chunk=w.C,
                                    workspace=ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    flat, ev_kind = stage_events(torch, steps * (n_st + 1))
    evs = [flat[i * (n_st + 1):(i + 1) * (n_st + 1)] for i in range(steps)]
    for i in range(steps):
        call(evs[i])
    torch.cuda.synchronize()
    st_ms = [sum(e[j].elapsed_time(e[j + 1]) for e in evs) / steps for j in range(n_st)]
    G = 8 if w.dk <= 64 else 4
    cnt = algorithmic_counts(w, w.B, w.H, w.T, w.dk, w.C, w.L, es, G=G)
    stages = {}
    for n, m in zip(names, st_ms):
        b = cnt["kernel_bytes"][n]
        stages[n] = {"ms": m, "alg_bytes": b, "alg_gbps": b / (m * 1e-3) / 1e9,
                     "frac_hbm": b / (m * 1e-3) / 1e9 / HBM_PEAK_GBPS}
    return {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "d": w.dk, "chunk": w.C, "dtype": w.dtype,
            "steps": steps, "warmup": warmup, "ms_per_step": ms, "tokens_per_s": w.B * w.T / (ms * 1e-3),
            "essential_bytes": cnt["bytes_io"],
            "layer_frac": cnt["bytes_io"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "alg_tflops": cnt["flops"] / (ms * 1e-3) / 1e12,
            "frac_of_bf16_peak": cnt["flops"] / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS if es == 2 else None,
            "stages": stages, "stage_events": ev_kind}


def ctypes_byref(la, st):
    import ctypes
    return ctypes.byref(st._st)


def pmc_summary(d: str):
    """Per-kernel mean of the counters in a rocprofv3 --pmc output directory."""
    import csv
    rows = []
    for p in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(p) as f:
            rows += list(csv.DictReader(f))
    agg = {}
    for r in rows:
        key = (r.get("Kernel_Name", "?"), r.get("Counter_Name", "?"))
        agg.setdefault(key, []).append(float(r.get("Counter_Value", 0)))
    out = {}
    for (k, c), v in agg.items():
        out.setdefault(k[:120], {})[c] = {"mean": sum(v) / len(v), "n": len(v)}
    print(json.dumps(out, indent=1))


def _pmc_values(d: str, counter: str):
    """Per kernel name, the counter's value for every dispatch in a run."""
    import csv
    acc = {}
    for p in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(p) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") == counter:
                    acc.setdefault(r.get("Kernel_Name", "?"), []).append(float(r.get("Counter_Value", 0)))
    return acc


def _pmc_means(d: str, counter: str):
    return {k: sum(v) / len(v) for k, v in _pmc_values(d, counter).items()}


def _copy_calibration(fetch_dir: str, write_dir: str):
    """FETCH_SIZE and WRITE_SIZE of the 1 GiB device copies (the largest copy
    dispatches of the run; other copies, e.g. of a decode state, differ)."""
    fv = _pmc_values(fetch_dir, "FETCH_SIZE").get("__amd_rocclr_copyBuffer", [])
    wv = _pmc_values(write_dir, "WRITE_SIZE").get("__amd_rocclr_copyBuffer", [])
    gib_kib = float(1 << 20)
    w_big = [x for x in wv if abs(x - gib_kib) < 0.01 * gib_kib]
    if not fv or not w_big:
        raise SystemExit("no 1 GiB copy in the counter runs: run them with --copy-calibration")
    f_big = sorted(fv)[-len(w_big):]
    fk, wk = sum(f_big) / len(f_big), sum(w_big) / len(w_big)
    return fk, wk, gib_kib / fk, gib_kib / wk


def pmc_profile(fetch_dir: str, write_dir: str, out_path: str):
    """Write the counter summary bench.py reads: per forward kernel, HBM bytes
    per launch from FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled
    by what the same counter reads for a plain device copy of known size (the
    1 GiB copy that --copy-calibration adds to every step)."""
    fetch, write = _pmc_means(fetch_dir, "FETCH_SIZE"), _pmc_means(write_dir, "WRITE_SIZE")
    big = "__amd_rocclr_copyBuffer"
    fk, wk, ff, wf = _copy_calibration(fetch_dir, write_dir)
    per_kib, traffic = {}, {}
    for frag, stage in KERNELS.items():
        names = [k for k in fetch if frag in k]
        if not names:
            continue
        n = names[0]
        per_kib[stage] = {"kernel": n, "FETCH_SIZE": fetch[n], "WRITE_SIZE": write.get(n, 0.0)}
        traffic[stage] = (fetch[n] * ff + write.get(n, 0.0) * wf) * 1024
    res = {"workload": "train_16k_bf16 (B=8,H=16,T=16384,d=64,C=64,bf16)",
           "kernel_source_hash": kernel_source_hash(),
           "calibration": {"kernel": big, "bytes": "1 GiB read + 1 GiB written",
                           "fetch_kib": fk, "write_kib": wk, "fetch_factor": ff, "write_factor": wf},
           "per_launch_kib": per_kib, "per_kernel_traffic_bytes": traffic,
           "commands": [
               f"cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d $REPO/{fetch_dir} "
               "-o fetch -- python3 $REPO/bench.py --steps 2 --warmup 1 --no-cpu --no-decode --no-backward --no-gdn --no-configs --no-layer --copy-calibration",
               f"cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv -d $REPO/{write_dir} "
               "-o write -- python3 $REPO/bench.py --steps 2 --warmup 1 --no-cpu --no-decode --no-backward --no-gdn --no-configs --no-layer --copy-calibration",
               f"python bench.py --pmc-profile {fetch_dir} {write_dir}"]}
    with open(out_path, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res, indent=1))


def trace_summary(path: str):
    """Markdown table of a rocprofv3 kernel_trace.csv grouped by kernel and
    grid size (one kernel at several shapes gets one row per shape)."""
    import csv
    agg = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            key = (r["Kernel_Name"], int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]),
                   int(r["Workgroup_Size_X"]))
            agg.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    print("| kernel | grid (threads) | block | calls | average us | min us | max us |")
    print("|---|---|---|---|---|---|---|")
    for (name, grid, block), v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        short = name if len(name) < 70 else name[:67] + "..."
        print(f"| `{short}` | {grid} | {block} | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")


def rocpd_summary(path: str):
    """Markdown table of per-kernel dispatch statistics from a rocprofv3
    output (SQLite database from the default format, or a kernel_stats.csv)."""
    rows = []
    if path.endswith(".db"):
        import sqlite3
        cur = sqlite3.connect(path).cursor()
        for name, calls, total, avg, pct in cur.execute(
                "select name, total_calls, total_duration, average, percentage from top_kernels"):
            # the top_kernels view reports microseconds
            rows.append((name, int(calls), float(total) / 1e3, float(avg), float(pct)))
    else:
        import csv
        with open(path) as f:
            for r in csv.DictReader(f):
                rows.append((r["Name"], int(r["Calls"]), float(r["TotalDurationNs"]) / 1e6,
                             float(r["AverageNs"]) / 1e3, float(r["Percentage"])))
    print("| kernel | calls | total ms | average us | % of GPU time |")
    print("|---|---|---|---|---|")
    for name, calls, total, avg, pct in rows:
        short = name if len(name) < 90 else name[:87] + "..."
        print(f"| `{short}` | {calls} | {total:.3f} | {avg:.1f} | {pct:.1f} |")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the GPU reaches steady clocks after about 25 forwards at this shape
    ap.add_argument("--warmup", type=int, default=25)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-gdn", action="store_true")
    ap.add_argument("--no-configs", action="store_true")
    ap.add_argument("--no-layer", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--pmc-summary", default=None)
    ap.add_argument("--pmc-profile", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"), default=None)
    ap.add_argument("--rocpd-summary", default=None)
    ap.add_argument("--trace-summary", default=None)
    args = ap.parse_args()
    if args.rocpd_summary:
        rocpd_summary(args.rocpd_summary)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.pmc_summary:
        pmc_summary(args.pmc_summary)
        return
    if args.pmc_profile:
        pmc_profile(args.pmc_profile[0], args.pmc_profile[1], PMC_FILE)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    import fenwick_tree_hierarchical_amd as la
    from fenwick_tree_hierarchical_amd.workloads import WORKLOADS, make_inputs

    dev = torch.device("cuda:0")
    w = WORKLOADS["train_16k_bf16"]
    log(f"bench: drawing {w.name} inputs on the GPU")
    x = make_inputs(w, device=dev)
    out = torch.empty_like(x["v"])
    nws = la.loglinear_fwd_workspace(w.B, w.H, w.T, w.dk, w.dv, w.C, torch.bfloat16)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    n_st = la.loglinear_fwd_num_stages(w.B, w.H, w.T, w.dk, w.dv, w.C, torch.bfloat16)
    stage_names = {3: ["chunk_states", "group_tree", "chunk_output"], 2: ["chunk_states", "chunk_output"],
                   1: ["chunk_output"]}[n_st]
    copy_src = copy_dst = None
    if args.copy_calibration:
        copy_src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        copy_dst = torch.empty_like(copy_src)

    def step(events=None):
        if events is None:
            la.loglinear_fwd(x["q"], x["k"], x["v"], x["log_a"], x["lam"], out=out, chunk=w.C, workspace=ws)
        else:
            la.loglinear_fwd_staged(x["q"], x["k"], x["v"], x["log_a"], x["lam"], events, out=out, chunk=w.C,
                                    workspace=ws)
        if copy_dst is not None:
            copy_dst.copy_(copy_src)

    # the other GPU legs first: the light decode legs early, the other forward
    # shapes last, so that the timed forward steps below follow forwards (each
    # kind of load brings its own clock transient over the first dozens of
    # launches; after forwards of the other shapes the 16K forward starts settled)
    secondary = {}
    if not args.no_decode:
        log("bench: decode 256 steps")
        secondary["decode"] = bench_decode(la, torch, dev)
        log("bench: decode at batch 256")
        secondary["decode"]["batch_256"] = bench_decode_large(la, torch, dev)
    if not args.no_backward:
        log("bench: backward")
        secondary["backward"] = bench_backward(la, torch, dev, w, x)
    if not args.no_gdn:
        log("bench: gated deltanet forward")
        secondary["gdn"] = bench_gdn(la, torch, dev, w)
    if not args.no_layer:
        from fenwick_tree_hierarchical_amd.workloads import LAYER_WORKLOADS
        log("bench: log-linear mamba-2 layer")
        secondary["layer"] = bench_layer(la, torch, dev, LAYER_WORKLOADS["layer_train_16k_bf16"])
        torch.cuda.empty_cache()
    if not args.no_configs:
        secondary["configs"] = {}
        for name in ("tiny_f32", "small_bf16", "long_128k_bf16"):
            log(f"bench: forward at {name}")
            secondary["configs"][name] = bench_config(la, torch, dev, WORKLOADS[name])
    torch.cuda.empty_cache()

    log(f"bench: warm-up {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"bench: timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # kernel durations: as many steps again, with timing-only HIP events
    # recorded on the launch stream between the kernels (the timed steps
    # above run without them)
    flat, ev_kind = stage_events(torch, args.steps * (n_st + 1))
    evs = [flat[i * (n_st + 1):(i + 1) * (n_st + 1)] for i in range(args.steps)]
    log(f"bench: {args.steps} staged steps for the kernel durations ({ev_kind} events)")
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall_staged = time.perf_counter() - t1
    per_step = [[e[j].elapsed_time(e[j + 1]) for e in evs] for j in range(n_st)]
    stage_ms = [sum(v) / args.steps for v in per_step]
    stage_med = [sorted(v)[len(v) // 2] for v in per_step]
    stage_min = [min(v) for v in per_step]
    ms_per_step = wall / args.steps * 1e3
    tokens = w.B * w.T
    value = tokens / (wall / args.steps)
    cnt = algorithmic_counts(w, w.B, w.H, w.T, w.dk, w.C, w.L, 2)
    st_ms = dict(zip(stage_names, stage_ms))
    src_hash = kernel_source_hash()
    traffic, why = pmc_traffic(src_hash)
    out_ms = st_ms["chunk_output"]
    out_bytes = cnt["kernel_bytes"]["chunk_output"]
    achieved = out_bytes / (out_ms * 1e-3) / 1e9
    fwd_ms = sum(stage_ms)
    result = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "ms_per_step_staged": wall_staged / args.steps * 1e3,
        "stage_events": ev_kind,
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "d_k": w.dk, "d_v": w.dv, "chunk": w.C,
                   "levels": w.L, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "fwd_chunk_output", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": traffic.get("chunk_output") if traffic else None,
                     "alg_bytes_per_launch": out_bytes,
                     "alg_bytes_note": f"{cnt['per_head_token_bytes']} B per head-token of q, k, v, out, log_a, "
                                       f"lambda plus one read of every bucket node "
                                       f"({cnt['node_bytes_per_bh']} B per (b,h))",
                     "mean_launch_ms": out_ms, "traffic_note": why, "kernel_source_hash": src_hash},
        "stages": {n: {"ms": m, "median_ms": stage_med[i], "min_ms": stage_min[i], "alg_bytes": cnt["kernel_bytes"][n],
                       "alg_gbps": cnt["kernel_bytes"][n] / (m * 1e-3) / 1e9,
                       "frac_hbm": cnt["kernel_bytes"][n] / (m * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                       "traffic_bytes": (traffic or {}).get(n)}
                   for i, (n, m) in enumerate(st_ms.items())},
        "layer_frac": cnt["bytes_io"] / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "layer_frac_note": f"essential bytes ({cnt['per_head_token_bytes']} B per head-token: q, k, v, out, "
                           f"log_a, lambda) / ms_per_step / 8 TB/s",
        "mfma": {"alg_tflop": cnt["flops"] / 1e12,
                 "achieved_tflops_whole_fwd": cnt["flops"] / (ms_per_step * 1e-3) / 1e12,
                 "frac_of_bf16_peak_whole_fwd": cnt["flops"] / (ms_per_step * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                 "peak_tflops": BF16_MFMA_PEAK_TFLOPS, "time_base": "ms_per_step",
                 "split_tflop": {"intra": cnt["flops_intra"] / 1e12, "states": cnt["flops_states"] / 1e12,
                                 "contractions": cnt["flops_contractions"] / 1e12}},
    }
    result.update(secondary)
    if "backward" in result:
        result["backward"]["ratio_to_forward"] = result["backward"]["ms"] / ms_per_step
        result["backward"]["from_forward"]["ratio_to_forward"] = result["backward"]["from_forward"]["ms"] / ms_per_step
    result["order"] = ("the other legs (decode, backward, gdn, layer, configs) ran before the warm-up and the "
                       "timed steps; the CPU baseline after them")
    if not args.no_cpu:
        log(f"bench: oracle CPU baseline on {host_cores()} host cores")
        result["cpu_baseline"] = cpu_baseline()
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result))


if __name__ == "__main__":
    main()
