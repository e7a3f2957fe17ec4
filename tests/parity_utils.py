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
    # valid verify lengths per request: [lo_b, hi_b] (lo == hi == L_b unless
    # request b holds an ambiguous position)
    len_lo: np.ndarray = None
    len_hi: np.ndarray = None
    # the batch total of lengths every valid schedule has (budget cut), or -1
    len_total: int = -1
    # the batch total no valid schedule exceeds (combined cut), or -1
    len_cap: int = -1
    # oracle argmax of every row 0..gamma of each ambiguous request
    amb_amax: Dict[int, np.ndarray] = field(default_factory=dict)


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


@dataclass
class Front:
    """Oracle steps 1-4 and the band of valid lengths around its cut."""
    conf: np.ndarray
    surv: np.ndarray
    lengths: np.ndarray
    cu: np.ndarray
    ptok: np.ndarray
    psrc: np.ndarray
    ambiguous_positions: int
    ambiguous_requests: np.ndarray
    len_lo: np.ndarray
    len_hi: np.ndarray
    len_total: int
    len_cap: int
    gamma: int

    @property
    def total(self) -> int:
        return int(self.cu[-1])

    def packed_rows(self) -> np.ndarray:
        """Dense logit rows the oracle's own schedule selects."""
        return self.psrc[: self.total]

    def ambiguous_rows(self) -> np.ndarray:
        """Every dense row (0..gamma) of each ambiguous request."""
        g1 = self.gamma + 1
        return np.concatenate([b * g1 + np.arange(g1) for b in self.ambiguous_requests]
                              + [np.zeros(0, np.int64)]).astype(np.int64)


def _above(surv: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per request: positions certainly above `ref` and possibly at or above it."""
    d = surv - ref
    return (d > BAND).sum(axis=1), (d >= -BAND).sum(axis=1)


def oracle_front(h: HostStep) -> Front:
    _, conf = oracle.confidence(h.hidden, h.w, h.bias, h.temps)
    surv = oracle.survival(conf)
    B = surv.shape[0]
    total_fixed, cap = -1, -1
    if h.cfg.mode == "threshold":
        L = oracle.cut_threshold(surv, h.cutoff)
        c = h.cutoff.astype(np.float64)[:, None]
        amb = np.abs(surv - c) <= BAND
        lo, hi = _above(surv, c)
    elif h.cfg.mode == "combined" and h.budget <= 0:
        # a budget of zero keeps no position, whatever passes its cutoff
        L = oracle.cut_combined(surv, h.cutoff, h.budget)
        cap = 0
        amb = np.zeros_like(surv, dtype=bool)
        lo = hi = L
    elif h.cfg.mode == "combined":
        L = oracle.cut_combined(surv, h.cutoff, h.budget)
        c = h.cutoff.astype(np.float64)[:, None]
        amb = np.abs(surv - c) <= BAND
        lo, hi = _above(surv, c)
        cap = int(h.budget)
        elig = np.sort(surv[surv >= c])[::-1]
        t = min(h.budget, elig.size)
        if 0 < t < elig.size:
            tau = elig[t - 1]
            near_cut = amb.copy()
            amb |= np.abs(surv - tau) <= BAND
            lo = np.minimum(lo, _above(surv, np.full_like(c, tau))[0])
            # a position that may or may not pass its cutoff and would rank
            # inside the budget can move the budget's last pick to any request
            if np.any(near_cut & (surv >= tau - BAND)):
                amb[:] = True
                lo = np.zeros_like(lo)
    elif h.cfg.mode == "static":
        L = oracle.cut_static(h.cfg.B, h.cfg.gamma)
        amb = np.zeros_like(surv, dtype=bool)
        lo = hi = L
    else:
        L = oracle.cut_budget(surv, h.budget)
        n = surv.size
        t = min(h.budget, n)
        total_fixed = t
        if 0 < t < n:
            tau = np.sort(surv.ravel())[::-1][t - 1]
            amb = np.abs(surv - tau) <= BAND
            lo, hi = _above(surv, np.full((B, 1), tau))
        else:
            amb = np.zeros_like(surv, dtype=bool)
            lo = hi = L
    amb_req = np.nonzero(amb.any(axis=1))[0]
    lo = np.where(amb.any(axis=1), lo, L).astype(np.int64)
    hi = np.where(amb.any(axis=1), hi, L).astype(np.int64)
    assert np.all(lo <= L) and np.all(L <= hi)
    cu, ptok, psrc = oracle.compact(L, h.tokens)
    return Front(conf, surv, L, cu, ptok, psrc, int(amb.sum()), amb_req, lo, hi,
                 total_fixed, cap, int(h.cfg.gamma))


def oracle_back(h: HostStep, front: Front, rows: np.ndarray,
                amb_rows: np.ndarray = None) -> OracleStep:
    """Oracle steps 5-6 on the packed rows the oracle itself selected.
    `amb_rows` ([n_ambiguous_requests * (gamma+1), V], optional) are every row
    of the ambiguous requests, in the order of `front.ambiguous_rows()`."""
    f = front
    amax = oracle.argmax_rows(rows)
    acc, bon = oracle.accept(f.cu, h.tokens, amax)
    amb_amax = {}
    if amb_rows is not None and len(f.ambiguous_requests):
        full = oracle.argmax_rows(amb_rows).reshape(len(f.ambiguous_requests), f.gamma + 1)
        amb_amax = {int(b): full[i] for i, b in enumerate(f.ambiguous_requests)}
    return OracleStep(f.conf, f.surv, f.lengths, f.cu, f.ptok, f.psrc, amax, acc, bon,
                      f.ambiguous_positions, f.ambiguous_requests, f.len_lo, f.len_hi,
                      f.len_total, f.len_cap, amb_amax)


def oracle_rows(s, front: Front):
    """Host copies of the rows the oracle reads: its packed rows, then every row
    of each ambiguous request."""
    return s.host_rows(front.packed_rows()), s.host_rows(front.ambiguous_rows())


def run_oracle(s) -> OracleStep:
    """The oracle's whole step on host copies of generated inputs. Only the
    packed logit rows the oracle itself selects (and every row of a request
    holding an ambiguous position) are copied to the host."""
    h = snapshot(s)
    front = oracle_front(h)
    return oracle_back(h, front, *oracle_rows(s, front))


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
        # A flipped length must lie in the band of valid lengths, and the batch
        # must keep the totals every valid schedule has.
        for b in flips:
            assert o.len_lo[b] <= gL[b] <= o.len_hi[b], \
                f"{ctx} request {b}: gpu length {gL[b]} outside [{o.len_lo[b]}, {o.len_hi[b]}]"
        if o.len_total >= 0:
            assert int(gL.sum()) == o.len_total, f"{ctx} budget total {gL.sum()} != {o.len_total}"
        if o.len_cap >= 0:
            assert int(gL.sum()) <= o.len_cap, f"{ctx} combined total {gL.sum()} > {o.len_cap}"
        for b in range(B):
            gs, n = int(gcu[b]), int(gL[b]) + 1
            if b in flips:
                # the rows, acceptance and bonus follow from the oracle's own
                # argmax of the request's rows, over the GPU's (valid) length
                g1 = tokens.shape[1]
                assert np.array_equal(g["packed_tokens"][gs:gs + n], tokens[b, :n]), ctx
                assert np.array_equal(g["packed_src_row"][gs:gs + n], b * g1 + np.arange(n)), ctx
                if b in o.amb_amax:
                    full = o.amb_amax[b]
                    assert np.array_equal(g["packed_argmax"][gs:gs + n], full[:n]), ctx
                    a = 0
                    while a < n - 1 and full[a] == tokens[b, a + 1]:
                        a += 1
                    assert g["accepted"][b] == a and g["bonus"][b] == full[a], \
                        f"{ctx} request {b} accept/bonus on flipped length"
                continue
            os_ = int(o.cu[b])
            assert np.array_equal(g["packed_tokens"][gs:gs + n], o.ptok[os_:os_ + n]), ctx
            assert np.array_equal(g["packed_src_row"][gs:gs + n], o.psrc[os_:os_ + n]), ctx
            assert np.array_equal(g["packed_argmax"][gs:gs + n], o.amax[os_:os_ + n]), ctx
            assert g["accepted"][b] == o.accepted[b] and g["bonus"][b] == o.bonus[b], ctx
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
