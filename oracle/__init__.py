"""Plain fp64 CPU oracle of the confidence-scheduled ragged verify step.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package. It shares no code with the HIP
path; it takes numpy arrays (copies of generated inputs) and returns numpy
arrays. The arithmetic lives in ``dspark_oracle.c``; this module only
marshals arguments.

Sources: "DFlash to DSpark in SGLang: 4.3x faster decode, and DeepSeek-V4
support" (the DSpark and ragged-verify sections) and SGLang's DSpark
announcement; each C function names the section it writes out.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import LIB, build

_lib = None

ERRORS = {1: "shape", 2: "argument", 3: "non-finite input", 4: "range"}


class OracleError(RuntimeError):
    pass


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        lib = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        L = ctypes.c_longlong
        F = ctypes.c_float
        lib.oracle_confidence.argtypes = [P, P, F, P, I, I, I, P, P]
        lib.oracle_survival.argtypes = [P, I, I, P]
        lib.oracle_cut_threshold.argtypes = [P, P, I, I, P]
        lib.oracle_cut_budget.argtypes = [P, I, I, L, P]
        lib.oracle_compact.argtypes = [P, P, I, I, P, P, P, P]
        lib.oracle_argmax_rows.argtypes = [P, P, ctypes.c_int64, ctypes.c_int64, P]
        lib.oracle_accept.argtypes = [P, P, P, I, I, P, P]
        lib.oracle_step.argtypes = [P, P, F, P, P, P, I, I, I, ctypes.c_int64, I, P, L,
                                    P, P, P, P, P, P, P, P, P]
        lib.oracle_cut_static.argtypes = [I, I, P]
        lib.oracle_cap_accept.argtypes = [P, P, P, I, I, P, P, P]
        lib.oracle_gather_rows.argtypes = [P, P, P, I, I, ctypes.c_int64, P]
        lib.oracle_tier_select.argtypes = [P, I, I, P, I, ctypes.c_int32, P, P, P, P]
        lib.oracle_cut_combined.argtypes = [P, P, I, I, L, P]
        lib.oracle_cost_cutoff.argtypes = [P, I, ctypes.c_int32, I, P]
        for f in (lib.oracle_confidence, lib.oracle_survival, lib.oracle_cut_threshold,
                  lib.oracle_cut_budget, lib.oracle_compact, lib.oracle_argmax_rows,
                  lib.oracle_accept, lib.oracle_step, lib.oracle_cut_static,
                  lib.oracle_cap_accept, lib.oracle_gather_rows, lib.oracle_tier_select,
                  lib.oracle_cut_combined, lib.oracle_cost_cutoff):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _arr(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what}: {ERRORS.get(rc, rc)}")


def confidence(hidden_bits, w_bits, bias, temps):
    """z and conf ([B, gamma] float64) of the confidence head with STS."""
    h = _arr(hidden_bits, np.uint16)
    B, g, d = h.shape
    w = _arr(w_bits, np.uint16)
    t = _arr(temps, np.float32)
    assert w.shape == (d,) and t.shape == (g,)
    z = np.empty((B, g), np.float64)
    p = np.empty((B, g), np.float64)
    _check(_load().oracle_confidence(_p(h), _p(w), float(bias), _p(t), B, g, d, _p(z), _p(p)),
           "confidence")
    return z, p


def survival(conf):
    c = _arr(conf, np.float64)
    B, g = c.shape
    s = np.empty((B, g), np.float64)
    _check(_load().oracle_survival(_p(c), B, g, _p(s)), "survival")
    return s


def cut_threshold(surv, cutoff):
    s = _arr(surv, np.float64)
    B, g = s.shape
    c = _arr(cutoff, np.float32)
    assert c.shape == (B,)
    L = np.empty(B, np.int32)
    _check(_load().oracle_cut_threshold(_p(s), _p(c), B, g, _p(L)), "cut_threshold")
    return L


def cut_budget(surv, budget):
    s = _arr(surv, np.float64)
    B, g = s.shape
    L = np.empty(B, np.int32)
    _check(_load().oracle_cut_budget(_p(s), B, g, int(budget), _p(L)), "cut_budget")
    return L


def cut_combined(surv, cutoff, budget):
    """Cutoffs and budget together: the top-`budget` of the positions that pass
    their request's cutoff."""
    s = _arr(surv, np.float64)
    B, g = s.shape
    c = _arr(cutoff, np.float32)
    assert c.shape == (B,)
    L = np.empty(B, np.int32)
    _check(_load().oracle_cut_combined(_p(s), _p(c), B, g, int(budget), _p(L)), "cut_combined")
    return L


def cost_cutoff(table, load, B):
    """Every request's cutoff from the cost table at the step's load level."""
    t = _arr(table, np.float32)
    c = np.empty(B, np.float32)
    _check(_load().oracle_cost_cutoff(_p(t), t.shape[0], int(load), int(B), _p(c)), "cost_cutoff")
    return c


def cut_static(B, gamma):
    L = np.empty(B, np.int32)
    _check(_load().oracle_cut_static(int(B), int(gamma), _p(L)), "cut_static")
    return L


def cap_accept(lengths, tokens, amax_full):
    """Cap-accept verify mode: (accepted, bonus, accepted_full) from the argmax of
    every row of the full block ([B*(gamma+1)], static packing) and the window
    lengths."""
    L = _arr(lengths, np.int32)
    tok = _arr(tokens, np.int32)
    B, g1 = tok.shape
    am = _arr(amax_full, np.int32)
    assert L.shape == (B,) and am.shape == (B * g1,)
    acc = np.empty(B, np.int32)
    bon = np.empty(B, np.int32)
    full = np.empty(B, np.int32)
    _check(_load().oracle_cap_accept(_p(L), _p(tok), _p(am), B, g1 - 1, _p(acc), _p(bon),
                                     _p(full)), "cap_accept")
    return acc, bon, full


def utilization(accepted, accepted_full):
    """The audit metric: tokens committed under the window over the tokens that
    verifying the whole block accepts (1.0 when that is none)."""
    a = int(np.sum(np.asarray(accepted, np.int64)))
    f = int(np.sum(np.asarray(accepted_full, np.int64)))
    return 1.0 if f == 0 else a / f


def compact(lengths, tokens):
    L = _arr(lengths, np.int32)
    tok = _arr(tokens, np.int32)
    B, g1 = tok.shape
    assert L.shape == (B,)
    cap = B * g1
    cu = np.empty(B + 1, np.int32)
    ptok = np.full(cap, -1, np.int32)
    psrc = np.full(cap, -1, np.int32)
    total = ctypes.c_int64(0)
    _check(_load().oracle_compact(_p(L), _p(tok), B, g1 - 1, _p(cu), _p(ptok), _p(psrc),
                                  ctypes.cast(ctypes.pointer(total), ctypes.c_void_p)),
           "compact")
    return cu, ptok, psrc


def gather_rows(src, packed_src_row, cu_seqlens, dst=None):
    """Packed row gather of a [B*(gamma+1), ...] array of any dtype: row r <
    cu[B] of the result is row packed_src_row[r] of src; the rest of dst (a
    copy of the given one, or zeros) is left as it is."""
    a = np.ascontiguousarray(src)
    cu = _arr(cu_seqlens, np.int32)
    ps = _arr(packed_src_row, np.int32)
    B = cu.shape[0] - 1
    cap = ps.shape[0]
    g = cap // B - 1
    assert cap == B * (g + 1) and a.shape[0] == cap
    out = np.zeros_like(a) if dst is None else np.array(dst, dtype=a.dtype, copy=True)
    row_bytes = a.nbytes // cap
    _check(_load().oracle_gather_rows(_p(a), _p(ps), _p(cu), B, g, row_bytes, _p(out)),
           "gather_rows")
    return out


def tier_select(cu_seqlens, gamma, tiers, pad_token, packed_tokens=None, packed_src_row=None):
    """(padded_total, tier_index, packed_tokens, packed_src_row): the smallest
    captured tier holding the packed total, and copies of the packed arrays
    with the rows up to that tier padded."""
    cu = _arr(cu_seqlens, np.int32)
    B = cu.shape[0] - 1
    t = _arr(tiers, np.int32)
    pt = None if packed_tokens is None else np.array(packed_tokens, np.int32, copy=True)
    ps = None if packed_src_row is None else np.array(packed_src_row, np.int32, copy=True)
    padded = np.zeros(1, np.int32)
    idx = np.zeros(1, np.int32)
    _check(_load().oracle_tier_select(_p(cu), B, int(gamma), _p(t), t.shape[0], int(pad_token),
                                      _p(padded), _p(idx), _p(pt), _p(ps)), "tier_select")
    return int(padded[0]), int(idx[0]), pt, ps


def argmax_rows(logits_bits, src_rows=None):
    """Lowest-index argmax of each listed row of a [rows, V] bf16-bit array."""
    lg = np.asarray(logits_bits)
    assert lg.dtype == np.uint16 and lg.flags.c_contiguous
    V = lg.shape[-1]
    lg2 = lg.reshape(-1, V)
    if src_rows is None:
        n = lg2.shape[0]
        src = None
    else:
        src = _arr(src_rows, np.int32)
        n = src.shape[0]
        assert n == 0 or (src.min() >= 0 and src.max() < lg2.shape[0])
    out = np.empty(n, np.int32)
    _check(_load().oracle_argmax_rows(_p(lg2), _p(src), n, V, _p(out)), "argmax_rows")
    return out


def accept(cu_seqlens, tokens, amax):
    cu = _arr(cu_seqlens, np.int32)
    tok = _arr(tokens, np.int32)
    B, g1 = tok.shape
    am = _arr(amax, np.int32)
    acc = np.empty(B, np.int32)
    bon = np.empty(B, np.int32)
    _check(_load().oracle_accept(_p(cu), _p(tok), _p(am), B, g1 - 1, _p(acc), _p(bon)),
           "accept")
    return acc, bon


def step(hidden_bits, w_bits, bias, temps, tokens, logits_bits, mode, cutoff=None, budget=0):
    """The whole step through the single C entry; returns a dict of outputs."""
    h = _arr(hidden_bits, np.uint16)
    B, g, d = h.shape
    w = _arr(w_bits, np.uint16)
    t = _arr(temps, np.float32)
    tok = _arr(tokens, np.int32)
    lg = np.asarray(logits_bits)
    assert lg.dtype == np.uint16 and lg.flags.c_contiguous and lg.shape[:2] == (B, g + 1)
    V = lg.shape[-1]
    m = ({"threshold": 0, "budget": 1, "static": 2, "combined": 3}[mode] if isinstance(mode, str)
         else int(mode))
    c = _arr(cutoff if cutoff is not None else np.zeros(B), np.float32)
    cap = B * (g + 1)
    out = dict(conf=np.empty((B, g)), survival=np.empty((B, g)),
               lengths=np.empty(B, np.int32), cu_seqlens=np.empty(B + 1, np.int32),
               packed_tokens=np.full(cap, -1, np.int32),
               packed_src_row=np.full(cap, -1, np.int32),
               packed_argmax=np.full(cap, -1, np.int32),
               accepted=np.empty(B, np.int32), bonus=np.empty(B, np.int32))
    _check(_load().oracle_step(
        _p(h), _p(w), float(bias), _p(t), _p(tok), _p(lg), B, g, d, V, m, _p(c), int(budget),
        _p(out["conf"]), _p(out["survival"]), _p(out["lengths"]), _p(out["cu_seqlens"]),
        _p(out["packed_tokens"]), _p(out["packed_src_row"]), _p(out["packed_argmax"]),
        _p(out["accepted"]), _p(out["bonus"])), "step")
    return out
