"""Host-side checks of the C ABI: the library loads without a GPU, exports every
symbol that include/dspark.h declares, and returns each validation status
before touching a device. No call here reaches a kernel launch: every call
carries at least one argument that the host-side checks reject.
"""
import ctypes
import os
import re

import pytest

import __graft_entry__  # noqa: F401  (puts the repo root on sys.path)
import confidence_scheduled_ragged_amd as dspark

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dspark.h")

OK, ENULL, ESHAPE, EARG, EALIGN, EWS, EHIP = range(7)
A = 0x10000          # a fake, 256-byte aligned "device" address; never dereferenced
P = ctypes.c_void_p


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(dspark.LIB_PATH):
        __graft_entry__.build()
    return dspark.lib()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(dspark_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    syms = declared_symbols()
    assert {"dspark_confidence", "dspark_schedule", "dspark_compact", "dspark_accept",
            "dspark_step"} <= set(syms)
    for s in syms:
        assert hasattr(L, s), s


def test_status_strings(L):
    for st in range(7):
        assert L.dspark_status_string(st)
    assert L.dspark_status_string(99) == b"unknown status"


def test_workspace_bytes(L):
    assert L.dspark_workspace_bytes(0, 16, 10) == 0
    assert L.dspark_workspace_bytes(4, 0, 10) == 0
    assert L.dspark_workspace_bytes(4, 300, 10) == 0
    assert L.dspark_workspace_bytes(4, 8, 0) == 0
    prev = 0
    for B in (1, 2, 64, 256, 1024):
        n = L.dspark_workspace_bytes(B, 16, 151936)
        assert n > prev and n % 256 == 0
        prev = n
    assert L.dspark_workspace_bytes(256, 16, 1) <= L.dspark_workspace_bytes(256, 16, 151936)
    assert L.dspark_workspace_bytes(256, 32, 8) > L.dspark_workspace_bytes(256, 16, 8)


def conf_call(L, hidden=A, w=A, bias=0.0, temps=A, B=4, g=8, d=256, conf=A, surv=A):
    return L.dspark_confidence(P(hidden) if hidden else None, P(w) if w else None, bias,
                               P(temps) if temps else None, B, g, d,
                               P(conf) if conf else None, P(surv) if surv else None, None)


def test_confidence_validation(L):
    assert conf_call(L, hidden=0) == ENULL
    assert conf_call(L, surv=0) == ENULL
    assert conf_call(L, B=0) == ESHAPE
    assert conf_call(L, g=0) == ESHAPE
    assert conf_call(L, g=257) == ESHAPE
    assert conf_call(L, d=0) == ESHAPE
    assert conf_call(L, B=1 << 24) == ESHAPE
    assert conf_call(L, bias=float("nan")) == EARG
    assert conf_call(L, bias=float("inf")) == EARG
    assert conf_call(L, hidden=A + 1) == EALIGN
    assert conf_call(L, temps=A + 2) == EALIGN
    assert conf_call(L, conf=A + 2) == EALIGN


def sched_call(L, surv=A, B=4, g=8, mode=0, cutoff=A, budget=0, lengths=A):
    return L.dspark_schedule(P(surv) if surv else None, B, g, mode,
                             P(cutoff) if cutoff else None, budget,
                             P(lengths) if lengths else None, None)


def test_schedule_validation(L):
    assert sched_call(L, surv=0) == ENULL
    assert sched_call(L, lengths=0) == ENULL
    assert sched_call(L, cutoff=0, mode=0) == ENULL
    assert sched_call(L, B=-1) == ESHAPE
    assert sched_call(L, mode=4, cutoff=0) == EARG
    assert sched_call(L, mode=-1, cutoff=0) == EARG
    assert sched_call(L, mode=3, cutoff=0) == ENULL         # combined needs the cutoffs
    assert sched_call(L, mode=3, budget=-1) == EARG         # and a budget
    assert sched_call(L, mode=1, cutoff=0, budget=-1) == EARG
    assert sched_call(L, lengths=A + 1) == EALIGN
    assert sched_call(L, mode=1, cutoff=0, surv=A + 2) == EALIGN


def compact_call(L, lengths=A, tokens=A, B=4, g=8, cu=A, ptok=A, psrc=A, logits=0, V=0, plog=0):
    f = lambda x: P(x) if x else None
    return L.dspark_compact(f(lengths), f(tokens), B, g, f(cu), f(ptok), f(psrc), f(logits), V,
                            f(plog), None)


def test_compact_validation(L):
    assert compact_call(L, tokens=0) == ENULL
    assert compact_call(L, logits=A, V=8) == ENULL          # logits without packed_logits
    assert compact_call(L, plog=A, V=8) == ENULL            # packed_logits without logits
    assert compact_call(L, g=0) == ESHAPE
    assert compact_call(L, logits=A, plog=A, V=0) == ESHAPE
    assert compact_call(L, cu=A + 1) == EALIGN
    assert compact_call(L, logits=A + 1, plog=A, V=8) == EALIGN


def accept_call(L, logits=A, psrc=A, cu=A, tok=A, B=4, g=8, V=1024, pam=A, acc=A, bonus=A,
                ws=A, wsb=1 << 30):
    f = lambda x: P(x) if x else None
    return L.dspark_accept(f(logits), f(psrc), f(cu), f(tok), B, g, V, f(pam), f(acc), f(bonus),
                           f(ws), wsb, None)


def test_accept_validation(L):
    assert accept_call(L, logits=0) == ENULL
    assert accept_call(L, ws=0) == ENULL
    assert accept_call(L, V=0) == ESHAPE
    assert accept_call(L, g=300) == ESHAPE
    assert accept_call(L, ws=A + 8) == EALIGN
    assert accept_call(L, logits=A + 1) == EALIGN
    need = L.dspark_workspace_bytes(4, 8, 1024)
    assert accept_call(L, wsb=need - 1) == EWS


def step_call(L, **kw):
    a = dict(hidden=A, w=A, bias=0.0, temps=A, tokens=A, logits=A, B=4, g=8, d=256, V=1024,
             mode=0, cutoff=A, budget=0, conf=A, surv=A, lengths=A, cu=A, ptok=A, psrc=A, pam=A,
             acc=A, bonus=A, ws=A, wsb=1 << 30)
    a.update(kw)
    f = lambda x: P(x) if x else None
    return L.dspark_step(f(a["hidden"]), f(a["w"]), a["bias"], f(a["temps"]), f(a["tokens"]),
                         f(a["logits"]), a["B"], a["g"], a["d"], a["V"], a["mode"],
                         f(a["cutoff"]), a["budget"], f(a["conf"]), f(a["surv"]),
                         f(a["lengths"]), f(a["cu"]), f(a["ptok"]), f(a["psrc"]), f(a["pam"]),
                         f(a["acc"]), f(a["bonus"]), f(a["ws"]), a["wsb"], None)


def test_step_validation(L):
    assert step_call(L, logits=0) == ENULL
    assert step_call(L, cutoff=0) == ENULL
    assert step_call(L, B=0) == ESHAPE
    assert step_call(L, d=0) == ESHAPE
    assert step_call(L, V=0) == ESHAPE
    assert step_call(L, mode=7) == EARG
    assert step_call(L, mode=1, cutoff=0, budget=-5) == EARG
    assert step_call(L, bias=float("nan")) == EARG
    assert step_call(L, tokens=A + 2) == EALIGN
    assert step_call(L, ws=A + 4) == EALIGN
    assert step_call(L, wsb=100) == EWS


def test_step_ex_validation(L):
    # the same checks as dspark_step (events are optional handles), and the form
    # must be 0, 1 or 2
    base = dict(hidden=A, w=A, bias=0.0, temps=A, tokens=A, logits=A, B=4, g=8, d=256, V=1024,
                mode=0, cutoff=A, budget=0, conf=A, surv=A, lengths=A, cu=A, ptok=A, psrc=A,
                pam=A, acc=A, bonus=A, ws=A, wsb=1 << 30)
    f = lambda x: P(x) if x else None

    def call(**kw):
        a = dict(base)
        a.update(kw)
        return L.dspark_step_ex(
            f(a["hidden"]), f(a["w"]), a["bias"], f(a["temps"]), f(a["tokens"]), f(a["logits"]),
            a["B"], a["g"], a["d"], a["V"], a["mode"], f(a["cutoff"]), a["budget"], f(a["conf"]),
            f(a["surv"]), f(a["lengths"]), f(a["cu"]), f(a["ptok"]), f(a["psrc"]), f(a["pam"]),
            f(a["acc"]), f(a["bonus"]), f(a["ws"]), a["wsb"], None, None, None,
            a.get("launches", 0), a.get("ticks", 0))

    assert call(logits=0) == ENULL
    assert call(launches=3) == EARG
    assert call(launches=-1) == EARG
    assert call(B=0) == ESHAPE
    assert call(mode=9) == EARG
    assert call(ws=A + 4) == EALIGN
    assert call(wsb=100) == EWS


def test_step_noalloc_validation(L):
    # the dspark_step checks, then the size of the library's scratch; every call
    # here is rejected before the scratch (a device symbol) is looked up
    f = lambda x: P(x) if x else None

    def call(B=4, g=8, logits=A, status=0, mode=0, launches=None):
        return L.dspark_step_noalloc(
            f(A), f(A), 0.0, f(A), f(A), f(logits), B, g, 256, 1024, mode, f(A), 0, f(A), f(A),
            f(A), f(A), f(A), f(A), f(A), f(A), f(A), f(status), None)

    assert call(logits=0) == ENULL
    assert call(B=0) == ESHAPE
    assert call(mode=9) == EARG
    assert call(B=20000, g=16) == EWS          # workspace beyond the 4 MiB scratch
    assert call(B=200000, g=1) == EWS
    assert call(status=A + 2) == EALIGN


def test_step_status_validation(L):
    assert L.dspark_step_status(None, P(A), None) == ENULL
    assert L.dspark_step_status(P(A), None, None) == ENULL
    assert L.dspark_step_status(P(A + 4), P(A), None) == EALIGN
    assert L.dspark_step_status(P(A), P(A + 2), None) == EALIGN


def cap_call(L, pam=A, tok=A, lengths=A, B=4, g=8, acc=A, bon=A, full=A, sums=0):
    f = lambda x: P(x) if x else None
    return L.dspark_cap_accept(f(pam), f(tok), f(lengths), B, g, f(acc), f(bon), f(full),
                               f(sums), None)


def test_cap_accept_validation(L):
    assert cap_call(L, pam=0) == ENULL
    assert cap_call(L, full=0) == ENULL
    assert cap_call(L, B=0) == ESHAPE
    assert cap_call(L, g=0) == ESHAPE
    assert cap_call(L, g=300) == ESHAPE
    assert cap_call(L, acc=A + 2) == EALIGN
    assert cap_call(L, B=-3, sums=A + 4) == ESHAPE     # shape is checked before alignment
    assert cap_call(L, sums=A + 4) == EALIGN


def gather_call(L, src=A, psrc=A, cu=A, B=4, g=8, row_bytes=64, dst=A):
    f = lambda x: P(x) if x else None
    return L.dspark_gather_rows(f(src), f(psrc), f(cu), B, g, row_bytes, f(dst), None)


def test_gather_rows_validation(L):
    assert gather_call(L, src=0) == ENULL
    assert gather_call(L, dst=0) == ENULL
    assert gather_call(L, B=0) == ESHAPE
    assert gather_call(L, row_bytes=0) == ESHAPE
    assert gather_call(L, row_bytes=-8) == ESHAPE
    assert gather_call(L, B=1 << 20, g=15, row_bytes=1 << 25) == ESHAPE   # 2^49 bytes
    assert gather_call(L, psrc=A + 2) == EALIGN
    assert gather_call(L, cu=A + 1) == EALIGN


def tier_call(L, cu=A, B=4, g=8, tiers=A, n=3, pad=0, padded=A, idx=A, ptok=0, psrc=0):
    f = lambda x: P(x) if x else None
    return L.dspark_tier_select(f(cu), B, g, f(tiers), n, pad, f(padded), f(idx), f(ptok),
                                f(psrc), None)


def test_tier_select_validation(L):
    assert tier_call(L, tiers=0) == ENULL
    assert tier_call(L, idx=0) == ENULL
    assert tier_call(L, n=0) == ESHAPE
    assert tier_call(L, n=5000) == ESHAPE
    assert tier_call(L, B=0) == ESHAPE
    assert tier_call(L, tiers=A + 2) == EALIGN
    assert tier_call(L, ptok=A + 1) == EALIGN


def test_cost_cutoff_validation(L):
    f = lambda x: P(x) if x else None
    assert L.dspark_cost_cutoff(None, 3, f(A), 4, f(A), None) == ENULL
    assert L.dspark_cost_cutoff(f(A), 0, f(A), 4, f(A), None) == ESHAPE
    assert L.dspark_cost_cutoff(f(A), 3, f(A), 0, f(A), None) == ESHAPE
    assert L.dspark_cost_cutoff(f(A), 3, f(A + 2), 4, f(A), None) == EALIGN


def test_workspace_init_validation(L):
    assert L.dspark_workspace_init(None, 1024, None) == ENULL
    assert L.dspark_workspace_init(P(A + 8), 1024, None) == EALIGN


def test_binding_names_match_header():
    for s in declared_symbols():
        assert hasattr(dspark, s), s


def test_binding_rejects_cpu_tensors():
    import torch
    h = torch.zeros((1, 2, 8), dtype=torch.bfloat16)
    w = torch.zeros(8, dtype=torch.bfloat16)
    t = torch.ones(2)
    with pytest.raises(ValueError):
        dspark.dspark_confidence(h, w, 0.0, t)
