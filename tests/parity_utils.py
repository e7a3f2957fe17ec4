"""End-to-end comparison of one GPU verify step with the oracle.

The oracle only ever sees generated inputs (host copies of a StepInputs) and
its own intermediate results; nothing computed by the HIP path is fed into it.
Floating-point outputs (conf, survival) must lie within 1e-5 of the fp64
oracle. Integer outputs must match exactly. The only tolerated integer
difference is a verify length that flips on a request holding an "ambiguous"
position, i.e. one whose fp64 survival lies within 1e-5 of its cutoff
(threshold mode) or of the budget's cut value tau (budget mode); such flips are
counted and returned, and every request whose length agrees is still compared
row by row.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List

import numpy as np

import oracle

FP_TOL = 1e-5
BAND = 1e-5


@dataclass
class OracleStep:
    conf: np.ndarray
    surv: np.ndarray
    lengths: np.ndarray
    cu: np.ndarray
    ptok: np.ndarray
    psrc: np.ndarray
    amax: np.ndarray
    accepted: np.ndarray
    bonus: np.ndarray
    ambiguous_positions: int
    ambiguous_requests: np.ndarray


@dataclass
class HostStep:
    """Host copies of one generated step (generated data only)."""
    cfg: object
    hidden: np.ndarray
    w: np.ndarray
    bias: float
    temps: np.ndarray
    cutoff: np.ndarray
    budget: int
    tokens: np.ndarray
    plant: np.ndarray


def snapshot(s) -> HostStep:
    return HostStep(s.cfg, s.host("hidden"), s.host("w"), s.bias, s.host("temps"),
                    s.host("cutoff"), s.budget, s.host("tokens"), s.plant)


def oracle_front(h: HostStep):
    """Oracle steps 1-4: returns (conf, surv, lengths, cu, ptok, psrc, n_amb, amb_req)."""
    _, conf = oracle.confidence(h.hidden, h.w, h.bias, h.temps)
    surv = oracle.survival(conf)
    if h.cfg.mode == "threshold":
        L = oracle.cut_threshold(surv, h.cutoff)
        amb = np.abs(surv - h.cutoff.astype(np.float64)[:, None]) <= BAND
    elif h.cfg.mode == "combined":
        L = oracle.cut_combined(surv, h.cutoff, h.budget)
        c = h.cutoff.astype(np.float64)[:, None]
        amb = np.abs(surv - c) <= BAND
        elig = np.sort(surv[surv >= c])[::-1]
        t = min(h.budget, elig.size)
        if 0 < t < elig.size:
            tau = elig[t - 1]
            near_cut = amb.copy()
            amb |= np.abs(surv - tau) <= BAND
            # a position that may or may not pass its cutoff and would rank
            # inside the budget can move the budget's last pick to any request
            if np.any(near_cut & (surv >= tau - BAND)):
                amb[:] = True
    elif h.cfg.mode == "static":
        L = oracle.cut_static(h.cfg.B, h.cfg.gamma)
        amb = np.zeros_like(surv, dtype=bool)
    else:
        L = oracle.cut_budget(surv, h.budget)
        n = surv.size
        t = min(h.budget, n)
        if 0 < t < n:
            tau = np.sort(surv.ravel())[::-1][t - 1]
            amb = np.abs(surv - tau) <= BAND
        else:
            amb = np.zeros_like(surv, dtype=bool)
    cu, ptok, psrc = oracle.compact(L, h.tokens)
    return conf, surv, L, cu, ptok, psrc, int(amb.sum()), np.nonzero(amb.any(axis=1))[0]


def oracle_back(h: HostStep, front, rows: np.ndarray) -> OracleStep:
    """Oracle steps 5-6 on the packed rows the oracle itself selected."""
    conf, surv, L, cu, ptok, psrc, n_amb, amb_req = front
    amax = oracle.argmax_rows(rows)
    acc, bon = oracle.accept(cu, h.tokens, amax)
    return OracleStep(conf, surv, L, cu, ptok, psrc, amax, acc, bon, n_amb, amb_req)


def run_oracle(s) -> OracleStep:
    """The oracle's whole step on host copies of generated inputs. Only the
    packed logit rows the oracle itself selects are copied to the host."""
    h = snapshot(s)
    front = oracle_front(h)
    total = int(front[3][-1])
    return oracle_back(h, front, s.host_rows(front[5][:total]))


@dataclass
class Report:
    total: int
    ambiguous_positions: int
    flipped_requests: List[int] = field(default_factory=list)
    max_conf_err: float = 0.0
    max_surv_err: float = 0.0


def compare(g: Dict[str, np.ndarray], o: OracleStep, tokens: np.ndarray, ctx: str = "") -> Report:
    """Assert GPU outputs `g` (numpy copies) against the oracle step `o`."""
    rep = Report(total=int(o.cu[-1]), ambiguous_positions=o.ambiguous_positions)
    if "conf" in g:
        rep.max_conf_err = float(np.max(np.abs(g["conf"].astype(np.float64) - o.conf)))
        assert rep.max_conf_err <= FP_TOL, f"{ctx} conf error {rep.max_conf_err}"
    if "survival" in g:
        rep.max_surv_err = float(np.max(np.abs(g["survival"].astype(np.float64) - o.surv)))
        assert rep.max_surv_err <= FP_TOL, f"{ctx} survival error {rep.max_surv_err}"
    gL = g["lengths"]
    flips = np.nonzero(gL != o.lengths)[0]
    bad = sorted(set(flips.tolist()) - set(o.ambiguous_requests.tolist()))
    assert not bad, f"{ctx} lengths differ on unambiguous requests {bad}: " \
                    f"gpu {gL[bad].tolist()} oracle {o.lengths[bad].tolist()}"
    rep.flipped_requests = flips.tolist()
    B = gL.shape[0]
    gcu = g["cu_seqlens"]
    # cu_seqlens is the scan of the GPU's own lengths; compare it to the exact
    # scan of those lengths and to the oracle's where no flip happened
    assert gcu[0] == 0 and np.array_equal(np.diff(gcu), gL + 1), f"{ctx} cu_seqlens not a scan"
    if flips.size == 0:
        assert np.array_equal(gcu, o.cu), f"{ctx} cu_seqlens"
        total = rep.total
        for k, ov in (("packed_tokens", o.ptok), ("packed_src_row", o.psrc),
                      ("packed_argmax", None)):
            gv = g[k][:total]
            ref = ov[:total] if ov is not None else o.amax
            if not np.array_equal(gv, ref):
                i = int(np.nonzero(gv != ref)[0][0])
                raise AssertionError(f"{ctx} {k} differs at packed row {i}: gpu {gv[i]} oracle {ref[i]}")
        assert np.array_equal(g["accepted"], o.accepted), f"{ctx} accepted"
        assert np.array_equal(g["bonus"], o.bonus), f"{ctx} bonus"
    else:
        g1 = tokens.shape[1]
        for b in range(B):
            if b in flips:
                continue
            gs, os_ = int(gcu[b]), int(o.cu[b])
            n = int(o.lengths[b]) + 1
            assert np.array_equal(g["packed_tokens"][gs:gs + n], o.ptok[os_:os_ + n]), ctx
            assert np.array_equal(g["packed_src_row"][gs:gs + n], o.psrc[os_:os_ + n]), ctx
            assert np.array_equal(g["packed_argmax"][gs:gs + n], o.amax[os_:os_ + n]), ctx
            assert g["accepted"][b] == o.accepted[b] and g["bonus"][b] == o.bonus[b], ctx
        del g1
    return rep


def planted_accept_pin(h, o: OracleStep):
    """Pin from the generator's planting record (not from any argmax): with m_b
    the first unplanted draft position, a_b >= min(L_b, m_b), and a_b can only
    exceed it when the unplanted row's argmax equals the draft by chance.
    `h` is a StepInputs or a HostStep."""
    plant = h.plant
    tok = h.tokens if isinstance(h, HostStep) else h.host("tokens")
    for b in range(h.cfg.B):
        unplanted = np.nonzero(~plant[b])[0]
        m = int(unplanted[0]) if unplanted.size else h.cfg.gamma
        L = int(o.lengths[b])
        a = int(o.accepted[b])
        assert a <= L
        assert a >= min(L, m), (b, a, L, m)
        if a > min(L, m):
            assert o.amax[o.cu[b] + m] == tok[b, m + 1]
        if a < L:
            assert o.bonus[b] != tok[b, a + 1]
