"""Host-side checks of the C ABI (CPU only: no kernel is launched).

The library must load, export every function include/logattn.h declares, and
return each documented error code from its host-side checks, which run before
anything is enqueued.  Pointers below are fake addresses: the calls must fail
validation before any of them is used.
"""

import ctypes
import os
import re

import pytest
import torch  # noqa: F401  (binds the library to torch's HIP runtime)

import fenwick_tree_hierarchical_amd as la

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "logattn.h")

OK, EINVAL, ESHAPE, EDTYPE, EALIGN, EWS, ECAP = 0, -1, -2, -3, -4, -5, -6
A = 1 << 20          # a fake, 256-byte aligned "device" address
L = la.lib()


def declared_functions():
    src = open(HEADER).read()
    return re.findall(r"LA_API\s+[\w\s\*]+?\b(\w+)\s*\(", src)


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n


def test_strerror_and_version():
    for code in (OK, EINVAL, ESHAPE, EDTYPE, EALIGN, EWS, ECAP, -7):
        assert la.loglinear_strerror(code)
    assert "unknown" in la.loglinear_strerror(12345)
    assert L.loglinear_version() >= 100


def ws(B, H, T, d, C, dt=1):
    n = ctypes.c_size_t(0)
    rc = L.loglinear_fwd_workspace(B, H, T, d, d, C, dt, ctypes.byref(n))
    return rc, n.value


def test_workspace_query():
    rc, n = ws(8, 16, 16384, 64, 64)
    assert rc == OK
    # per-chunk bucket nodes (bf16) + per-group states (fp32) and nodes (bf16)
    # + gate totals: 256 chunks in 32 groups of 8
    nch, ng, BH, DD = 256, 32, 128, 64 * 64
    need = BH * nch * DD * 2 + BH * ng * DD * 4 + BH * ng * DD * 2
    assert need <= n < need * 1.05
    assert ws(1, 1, 64, 16, 16, 0)[0] == OK
    assert ws(1, 1, 100, 16, 16, 0)[0] == OK        # ragged T is accepted
    assert ws(0, 4, 100, 64, 64)[1] == 0             # empty problem needs nothing
    assert ws(3, 2, 63, 64, 64)[1] == 0              # a single partial chunk needs nothing
    # one full chunk: its bucket node (read by the final state) and gate total
    assert ws(3, 2, 64, 64, 64)[1] == 3 * 2 * 64 * 64 * 2 + 256
    assert ws(1, 1, 64, 16, 16, 7)[0] == EDTYPE
    assert ws(1, 1, 64, 24, 64)[0] == ESHAPE          # unsupported head dim
    assert ws(1, 1, 64, 64, 48)[0] == ESHAPE          # unsupported chunk
    assert ws(-1, 1, 64, 64, 64)[0] == EINVAL
    assert L.loglinear_fwd_workspace(1, 1, 64, 64, 32, 64, 1, ctypes.byref(ctypes.c_size_t())) == ESHAPE
    assert L.loglinear_fwd_workspace(1, 1, 64, 64, 64, 64, 1, None) == EINVAL


def test_tile_shapes_that_fit():
    """Every bf16 tile shape fits in LDS; fp32 does too except C = d = 128
    (its fp32 tiles exceed 160 KB), which is rejected."""
    for dt in (0, 1):
        for d in (16, 32, 64, 128):
            for C in (16, 32, 64, 128):
                want = ESHAPE if (dt == 0 and C == 128 and d == 128) else OK
                assert ws(1, 1, 1000, d, C, dt)[0] == want, (dt, d, C)


def fwd(q=A, k=A, v=A, la_=A, lam=A, out=A, B=1, H=1, T=64, d=16, C=16, Lv=7, dt=0, w=A, wb=1 << 30):
    return L.loglinear_fwd(q, k, v, la_, lam, out, B, H, T, d, d, C, Lv, dt, w, wb, None)


def test_fwd_validation_codes():
    assert fwd(q=None) == EINVAL
    assert fwd(out=None) == EINVAL
    assert fwd(lam=None) == EINVAL
    assert fwd(q=A + 8) == EALIGN
    assert fwd(out=A + 4) == EALIGN
    assert fwd(la_=A + 2) == EALIGN
    assert fwd(dt=5) == EDTYPE
    assert fwd(Lv=6) == ESHAPE                           # T=64 needs 7 levels
    assert fwd(Lv=33) == ESHAPE
    assert fwd(d=48) == ESHAPE
    assert fwd(C=8) == ESHAPE
    assert fwd(T=-1) == EINVAL
    # workspace: T=1024 with C=16 has several groups, so a workspace is needed
    assert fwd(T=1024, Lv=11, w=None) == EWS
    assert fwd(T=1024, Lv=11, wb=16) == EWS
    assert fwd(T=1024, Lv=11, w=A + 16) == EALIGN
    # empty problems return OK without touching any pointer
    assert fwd(q=None, k=None, v=None, la_=None, lam=None, out=None, B=0) == OK
    assert fwd(q=None, k=None, v=None, la_=None, lam=None, out=None, T=0, Lv=0) == OK


def test_num_stages():
    n = ctypes.c_int(-1)
    assert L.loglinear_fwd_num_stages(1, 1, 16, 16, 16, 16, 0, ctypes.byref(n)) == OK and n.value == 1
    assert L.loglinear_fwd_num_stages(1, 1, 64, 16, 16, 16, 0, ctypes.byref(n)) == OK and n.value == 2
    assert L.loglinear_fwd_num_stages(8, 16, 16384, 64, 64, 64, 1, ctypes.byref(n)) == OK and n.value == 3
    assert L.loglinear_fwd_num_stages(0, 16, 16384, 64, 64, 64, 1, ctypes.byref(n)) == OK and n.value == 0


def test_staged_requires_matching_event_count():
    ev = (ctypes.c_void_p * 2)(A, A)
    rc = L.loglinear_fwd_staged(A, A, A, A, A, A, 8, 16, 16384, 64, 64, 64, 15, 1, A, 1 << 34, ev, 2, None)
    assert rc == EINVAL                                   # three stages need four events
    ev0 = (ctypes.c_void_p * 4)(A, None, A, A)
    rc = L.loglinear_fwd_staged(A, A, A, A, A, A, 8, 16, 16384, 64, 64, 64, 15, 1, A, 1 << 34, ev0, 4, None)
    assert rc == EINVAL


def fwd_state(st, B=1, H=1, T=64, d=16, C=16, Lv=7, dt=0, q=A, w=A, wb=1 << 30):
    return L.loglinear_fwd_state(q, A, A, A, A, A, B, H, T, d, d, C, Lv, dt, w, wb,
                                 ctypes.byref(st) if st is not None else None, None)


def test_fwd_state_validation_codes():
    st = la._LaState(0, 1, 1, 16, 16, 7, A, A)
    assert fwd_state(None) == EINVAL
    assert fwd_state(st, q=None) == EINVAL
    assert fwd_state(la._LaState(0, 1, 2, 16, 16, 7, A, A)) == ESHAPE       # H differs
    assert fwd_state(la._LaState(0, 1, 1, 32, 32, 7, A, A)) == ESHAPE       # head dim differs
    assert fwd_state(la._LaState(0, 1, 1, 16, 16, 6, A, A)) == ECAP         # T=64 needs 7 slots
    assert fwd_state(la._LaState(0, 1, 1, 16, 16, 41, A, A)) == ESHAPE      # beyond the slot limit
    assert fwd_state(la._LaState(0, 1, 1, 16, 16, 7, A + 4, A)) == EALIGN
    assert fwd_state(la._LaState(0, 1, 1, 16, 16, 7, None, A)) == EINVAL
    assert fwd_state(st, T=1024, Lv=11) == ECAP                               # 11 slots needed
    assert st.t == 0                                  # unchanged on every error
    # empty batch: only the host position moves to T
    st0 = la._LaState(0, 0, 1, 16, 16, 7, None, None)
    assert L.loglinear_fwd_state(None, None, None, None, None, None, 0, 1, 50, 16, 16, 16, 7, 0, None, 0,
                                 ctypes.byref(st0), None) == OK
    assert st0.t == 50


def test_state_bytes_and_init_validation():
    sb, cb = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.loglinear_state_bytes(64, 16, 64, 64, 16, ctypes.byref(sb), ctypes.byref(cb)) == OK
    assert sb.value == 64 * 16 * 16 * 64 * 64 * 4 and cb.value == 64 * 16 * 16 * 4
    assert L.loglinear_state_bytes(1, 1, 64, 64, 0, ctypes.byref(sb), ctypes.byref(cb)) == ESHAPE
    assert L.loglinear_state_bytes(1, 1, 64, 64, 41, ctypes.byref(sb), ctypes.byref(cb)) == ESHAPE
    assert L.loglinear_state_bytes(1, 1, 64, 32, 4, ctypes.byref(sb), ctypes.byref(cb)) == ESHAPE
    st = la._LaState()
    assert L.loglinear_state_init(ctypes.byref(st), 1, 1, 64, 64, 4, None, A, None) == EINVAL
    assert L.loglinear_state_init(ctypes.byref(st), 1, 1, 64, 64, 4, A + 4, A, None) == EALIGN
    assert L.loglinear_state_init(None, 1, 1, 64, 64, 4, A, A, None) == EINVAL
    # empty state: initialised on the host only
    assert L.loglinear_state_init(ctypes.byref(st), 0, 4, 64, 64, 4, None, None, None) == OK
    assert st.t == 0 and st.S == 4


def test_decode_validation_codes():
    st = la._LaState(0, 1, 1, 64, 64, 3, A, A)
    step = lambda **kw: L.loglinear_decode_step(ctypes.byref(st), kw.get("q", A), A, A, A, A, kw.get("out", A),
                                                kw.get("dt", 1), None)
    assert step(dt=3) == EDTYPE
    assert step(q=None) == EINVAL
    assert step(out=A + 2) == EALIGN
    st.t = 7                      # 0b111: merging needs level 4 > S = 3
    assert step() == ECAP and st.t == 7
    st.t = 8                      # level 4 occupied: already beyond capacity
    assert step() == ECAP
    st.t = -1
    assert step() == EINVAL
    # empty batch: only the host position advances
    st0 = la._LaState(5, 0, 1, 64, 64, 3, None, None)
    assert L.loglinear_decode_step(ctypes.byref(st0), None, None, None, None, None, None, 1, None) == OK
    assert st0.t == 6


def test_level_table_validation_codes():
    assert L.loglinear_level_table(0, 16, A, None) == EINVAL
    assert L.loglinear_level_table(64, 0, A, None) == EINVAL
    assert L.loglinear_level_table(64, 24, A, None) == ESHAPE
    assert L.loglinear_level_table(16385, 16, A, None) == ESHAPE
    assert L.loglinear_level_table(64, 16, None, None) == EINVAL


def test_binding_refuses_cpu_tensors():
    x = torch.zeros(1, 1, 16, 16)
    with pytest.raises(ValueError):
        la.loglinear_fwd(x, x, x, torch.zeros(1, 1, 16), torch.zeros(1, 1, 16, 5))


def bws(B, H, T, d, C, dt=1):
    n = ctypes.c_size_t(0)
    rc = L.loglinear_bwd_workspace(B, H, T, d, d, C, dt, ctypes.byref(n))
    return rc, n.value


def test_bwd_workspace_query():
    rc, n = bws(8, 16, 16384, 64, 64)
    assert rc == OK
    fwd_part = ws(8, 16, 16384, 64, 64)[1]
    # forward structure, key-side chunk nodes (bf16, and transposed), group
    # shares (fp32, 5 group levels for 32 groups; in bf16 one per half group),
    # group nodes (and transposed), column terms
    BH, nch, ng, DD = 128, 256, 32, 64 * 64
    need = fwd_part + 2 * BH * nch * DD * 2 + 2 * BH * ng * 5 * DD * 4 + 2 * BH * ng * DD * 2 + BH * 16384 * 4
    assert need <= n < need * 1.01
    # fp32: one share per group and level
    rc, n32 = bws(8, 16, 16384, 64, 64, 0)
    need32 = ws(8, 16, 16384, 64, 64, 0)[1] + 2 * BH * nch * DD * 4 + BH * ng * 5 * DD * 4 + 2 * BH * ng * DD * 4 \
        + BH * 16384 * 4
    assert rc == OK and need32 <= n32 < need32 * 1.01
    assert bws(2, 3, 50, 64, 64)[1] == 1280              # one partial chunk: 2*3*50 column terms, 256-aligned
    assert bws(1, 1, 64, 64, 128)[0] == ESHAPE              # chunks above 64
    for dt in (0, 1):
        for d in (16, 32, 64, 128):
            for C in (16, 32, 64):
                assert bws(1, 1, 1000, d, C, dt)[0] == OK, (dt, d, C)
    assert bws(0, 4, 100, 64, 64)[1] == 0
    assert L.loglinear_bwd_workspace(1, 1, 64, 64, 64, 64, 1, None) == EINVAL


def bwd(B=1, H=1, T=64, d=16, C=16, Lv=7, dt=0, w=A, wb=1 << 30, **kw):
    p = {n: kw.get(n, A) for n in ("q", "k", "v", "la", "lam", "g", "gq", "gk", "gv", "gla", "glam")}
    return L.loglinear_bwd(p["q"], p["k"], p["v"], p["la"], p["lam"], p["g"], p["gq"], p["gk"], p["gv"], p["gla"],
                           p["glam"], B, H, T, d, d, C, Lv, dt, w, wb, None)


def test_bwd_validation_codes():
    assert bwd(g=None) == EINVAL
    assert bwd(glam=None) == EINVAL
    assert bwd(gq=A + 8) == EALIGN
    assert bwd(g=A + 8) == EALIGN
    assert bwd(gla=A + 2) == EALIGN
    assert bwd(dt=4) == EDTYPE
    assert bwd(Lv=6) == ESHAPE
    assert bwd(C=128) == ESHAPE
    assert bwd(w=None) == EWS
    assert bwd(wb=16) == EWS
    assert bwd(w=A + 16) == EALIGN
    assert bwd(q=None, k=None, v=None, la=None, lam=None, g=None, gq=None, gk=None, gv=None, gla=None, glam=None,
               B=0) == OK
    assert bwd(q=None, k=None, v=None, la=None, lam=None, g=None, gq=None, gk=None, gv=None, gla=None, glam=None,
               T=0, Lv=0) == OK


def bwd_ff(B=1, H=1, T=64, d=16, C=16, Lv=7, dt=0, w=A, wb=1 << 30, fw=A, fwb=1 << 30, **kw):
    p = {n: kw.get(n, A) for n in ("q", "k", "v", "la", "lam", "g", "gq", "gk", "gv", "gla", "glam")}
    return L.loglinear_bwd_from_fwd(p["q"], p["k"], p["v"], p["la"], p["lam"], p["g"], p["gq"], p["gk"], p["gv"],
                                    p["gla"], p["glam"], B, H, T, d, d, C, Lv, dt, fw, fwb, w, wb, None)


def test_bwd_from_fwd_validation_codes():
    """The backward reusing a forward's workspace: the backward's own checks
    first, then the forward workspace's size (that forward's plan) and
    alignment; empty problems succeed without reading anything."""
    fn = ctypes.c_size_t(0)
    assert L.loglinear_fwd_workspace(1, 1, 64, 16, 16, 16, 0, ctypes.byref(fn)) == OK and fn.value > 0
    assert bwd_ff(g=None) == EINVAL
    assert bwd_ff(w=None) == EWS
    assert bwd_ff(fw=None) == EWS
    assert bwd_ff(fwb=fn.value - 1) == EWS
    assert bwd_ff(fw=A + 16) == EALIGN
    assert bwd_ff(Lv=6) == ESHAPE
    assert bwd_ff(q=None, k=None, v=None, la=None, lam=None, g=None, gq=None, gk=None, gv=None, gla=None, glam=None,
                  fw=None, fwb=0, B=0) == OK


def gws(B, H, T, d, C, dt=1):
    n = ctypes.c_size_t(0)
    rc = L.loglinear_gdn_fwd_workspace(B, H, T, d, d, C, dt, ctypes.byref(n))
    return rc, n.value


def test_gdn_workspace_query():
    # a C x C matrix per chunk, a state and a transition per aligned block
    # of 2^m full chunks (256 + 128 + ... + 1 = 511 per head), all bf16,
    # plus an fp32 gate total per block
    rc, n = gws(8, 16, 16384, 64, 64)
    assert rc == OK
    nodes = 128 * 511
    need = 128 * 256 * 64 * 64 * 2 + nodes * 2 * 64 * 64 * 2 + nodes * 4
    assert need <= n < need + 4 * 256
    assert gws(1, 1, 63, 64, 64)[1] == 64 * 64 * 2  # no full chunk: the chunk's matrix only
    assert gws(0, 3, 640, 64, 64)[1] == 0          # empty problem
    assert gws(2, 1, 100, 16, 16)[0] == OK         # ragged T
    assert gws(1, 1, 64, 128, 64)[0] == ESHAPE     # d = 128 is not supported here
    assert gws(1, 1, 64, 64, 128)[0] == ESHAPE     # nor C = 128
    assert gws(1, 1, 64, 16, 16, 3)[0] == EDTYPE
    assert gws(-1, 1, 64, 16, 16)[0] == EINVAL
    assert L.loglinear_gdn_fwd_workspace(1, 1, 64, 64, 64, 64, 1, None) == EINVAL
    for dt in (0, 1):                              # every supported shape fits in LDS
        for d in (16, 32, 64):
            for C in (16, 32, 64):
                assert gws(1, 1, 1000, d, C, dt)[0] == OK, (dt, d, C)


def gdn(q=A, k=A, v=A, la_=A, beta=A, lam=A, out=A, B=1, H=1, T=64, d=16, C=16, Lv=7, dt=0, w=A, wb=1 << 30):
    return L.loglinear_gdn_fwd(q, k, v, la_, beta, lam, out, B, H, T, d, d, C, Lv, dt, w, wb, None)


def test_gdn_validation_codes():
    assert gdn(q=None) == EINVAL
    assert gdn(beta=None) == EINVAL
    assert gdn(out=None) == EINVAL
    assert gdn(k=A + 8) == EALIGN
    assert gdn(beta=A + 2) == EALIGN
    assert gdn(dt=4) == EDTYPE
    assert gdn(Lv=6) == ESHAPE
    assert gdn(d=128, C=64) == ESHAPE
    assert gdn(T=-5) == EINVAL
    assert gdn(T=64, w=None) == EWS                # every non-empty problem needs a workspace
    assert gdn(T=64, wb=100) == EWS
    assert gdn(T=64, w=A + 64) == EALIGN
    assert gdn(q=None, k=None, v=None, la_=None, beta=None, lam=None, out=None, B=0) == OK
    assert gdn(q=None, k=None, v=None, la_=None, beta=None, lam=None, out=None, T=0, Lv=0) == OK
