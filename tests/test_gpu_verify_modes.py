"""GPU parity of the static and cap-accept verify modes (needs an MI355X).

[P1] "DFlash to DSpark in SGLang", section "The confidence scheduler and
verify modes": static verifies the full block; cap-accept pays that verify but
commits only the cut's window, so its committed output equals compact's
exactly, and it logs the acceptance of the whole block beside it.

The oracle sees only generated inputs: it computes its own full-block argmax,
its own cut and its own cap. The GPU's cap-accept result is compared with the
oracle's, and with the GPU's own compact step (the pages' invariant).
"""
import numpy as np
import pytest
import torch

import __graft_entry__  # noqa: F401
import confidence_scheduled_ragged_amd as dspark
import oracle
from parity_utils import FP_TOL, oracle_front, snapshot
from synth import CONFIGS, make_step

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def host(t):
    return t.cpu().numpy()


def _static_step(s):
    out = dspark.dspark_step(s.hidden, s.w, s.bias, s.temps, s.tokens, s.logits, "static")
    return out


def _compact_step(s):
    return dspark.dspark_step(s.hidden, s.w, s.bias, s.temps, s.tokens, s.logits, s.cfg.mode,
                              cutoff=s.cutoff, budget=s.budget)


def _oracle_full_argmax(s):
    B, g1 = s.cfg.B, s.cfg.gamma + 1
    return oracle.argmax_rows(s.host_rows(np.arange(B * g1, dtype=np.int32)))


@pytest.mark.parametrize("name,steps", [("tiny", 3), ("mid", 2), ("mixed_threshold", 1),
                                        ("stage_path", 1)])
def test_static_step_matches_oracle(name, steps):
    # "stage_path": B > 4096 takes the stage kernels inside dspark_step
    cfg = (CONFIGS["tiny"].scaled(B=4200, gamma=2, d=64, V=64) if name == "stage_path"
           else CONFIGS[name])
    for step in range(steps):
        s = make_step(cfg, step, device=DEV)
        g = {k: host(v) for k, v in _static_step(s).items()}
        torch.cuda.synchronize()
        h = snapshot(s)
        _, conf = oracle.confidence(h.hidden, h.w, h.bias, h.temps)
        surv = oracle.survival(conf)
        B, gam = cfg.B, cfg.gamma
        am = _oracle_full_argmax(s)
        L = oracle.cut_static(B, gam)
        cu, ptok, psrc = oracle.compact(L, h.tokens)
        acc, bon = oracle.accept(cu, h.tokens, am)
        assert np.max(np.abs(g["conf"] - conf)) <= FP_TOL
        assert np.max(np.abs(g["survival"] - surv)) <= FP_TOL
        assert np.array_equal(g["lengths"], L)
        assert np.array_equal(g["cu_seqlens"], cu)
        assert np.array_equal(g["packed_tokens"], ptok)
        assert np.array_equal(g["packed_src_row"], psrc)
        assert np.array_equal(g["packed_argmax"], am)
        assert np.array_equal(g["accepted"], acc) and np.array_equal(g["bonus"], bon)


@pytest.mark.parametrize("name,steps", [("tiny", 4), ("mid", 3), ("budget", 1),
                                        ("mixed_threshold", 2), ("mixed_budget", 2)])
def test_cap_accept_matches_oracle_and_compact(name, steps):
    cfg = CONFIGS[name]
    utils = []
    for step in range(steps):
        s = make_step(cfg, step, device=DEV)
        st = _static_step(s)
        cp = _compact_step(s)
        sums = torch.full((2,), -1, dtype=torch.int64, device=DEV)
        acc, bon, full, _ = dspark.dspark_cap_accept(st["packed_argmax"], s.tokens, cp["lengths"],
                                                     sums=sums)
        torch.cuda.synchronize()
        acc, bon, full, sums = host(acc), host(bon), host(full), host(sums)
        gL = host(cp["lengths"])
        # the pages' invariant, GPU against GPU: cap-accept commits what compact commits
        assert np.array_equal(acc, host(cp["accepted"]))
        assert np.array_equal(bon, host(cp["bonus"]))
        # the static step's acceptance is the uncapped record
        assert np.array_equal(full, host(st["accepted"]))
        assert sums[0] == acc.astype(np.int64).sum() and sums[1] == full.astype(np.int64).sum()
        # against the oracle's own cut, full-block argmax and cap
        h = snapshot(s)
        front = oracle_front(h)
        oL, amb_req = front.lengths, front.ambiguous_requests
        o_acc, o_bon, o_full = oracle.cap_accept(oL, h.tokens, _oracle_full_argmax(s))
        assert np.array_equal(full, o_full)
        same = gL == oL
        assert np.all(same | np.isin(np.arange(cfg.B), amb_req)), "length flip off the band"
        assert np.all((front.len_lo <= gL) & (gL <= front.len_hi)), "length outside the band"
        assert np.array_equal(acc[same], o_acc[same]) and np.array_equal(bon[same], o_bon[same])
        utils.append(oracle.utilization(o_acc, o_full))
        if same.all():
            assert abs(oracle.utilization([sums[0]], [sums[1]]) - utils[-1]) < 1e-12
    print(f"\n[{name}] utilisation of the window against the full verify: "
          f"{', '.join(f'{u:.3f}' for u in utils)}", flush=True)


@pytest.mark.parametrize("B,g", [(1, 1), (5, 3), (130, 16), (7, 64)])
def test_cap_accept_edge_lengths(B, g):
    # hand-built full-block argmax and drafts: lengths include 0, gamma and
    # out-of-range values (clamped on the GPU; the oracle gets the clamped ones)
    rng = np.random.default_rng(B * 100 + g)
    V = 50
    am_full = rng.integers(0, V, B * (g + 1)).astype(np.int32)
    tok = rng.integers(0, V, (B, g + 1)).astype(np.int32)
    m = rng.integers(0, g + 1, B)
    for b in range(B):
        for j in range(g):
            if j < m[b]:
                tok[b, j + 1] = am_full[b * (g + 1) + j]
            elif tok[b, j + 1] == am_full[b * (g + 1) + j]:
                tok[b, j + 1] = (tok[b, j + 1] + 1) % V
    L = rng.integers(-2, g + 3, B).astype(np.int32)
    L[0] = 0
    Lc = np.clip(L, 0, g).astype(np.int32)
    t = lambda a: torch.from_numpy(a).to(DEV)
    acc, bon, full, _ = dspark.dspark_cap_accept(t(am_full), t(tok), t(L))
    o_acc, o_bon, o_full = oracle.cap_accept(Lc, tok, am_full)
    assert np.array_equal(host(full), o_full) and np.array_equal(o_full, m)
    assert np.array_equal(host(acc), o_acc) and np.array_equal(host(bon), o_bon)
