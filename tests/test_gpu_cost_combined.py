"""GPU parity of the combined cut (cutoff and budget together) and the
cost-table cutoff (needs an MI355X).

[P1] "DFlash to DSpark in SGLang", section "The confidence scheduler and
verify modes": a request's window ends at the first position whose survival is
below the per-token cost, that cost is read from a table timed per load level,
and a heavier load shrinks all windows at once; section "Zero-overhead scheduling and kernels": the
batch-wide verify-length top-k schedule. The oracle computes its own cutoffs,
cuts and steps from the generated inputs only.
"""
import numpy as np
import pytest
import torch

import __graft_entry__  # noqa: F401
import confidence_scheduled_ragged_amd as dspark
import oracle
from parity_utils import compare, oracle_back, oracle_front, oracle_rows, snapshot
from synth import CONFIGS, make_step

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _surv(rng, B, g, kind):
    if kind == "ties":
        # heavy ties: survival built from a few distinct probabilities
        p = rng.choice(np.array([0.5, 0.75, 0.875, 1.0], np.float32), (B, g))
    else:
        p = rng.uniform(0.2, 1.0, (B, g)).astype(np.float32)
    s = np.cumprod(p.astype(np.float64), axis=1)
    return s.astype(np.float32)


@pytest.mark.parametrize("B,g,kind", [(4, 8, "rand"), (256, 16, "rand"), (256, 16, "ties"),
                                      (600, 16, "rand"), (3, 64, "ties"), (1, 1, "rand")])
def test_combined_schedule_stage(B, g, kind):
    rng = np.random.default_rng(B * 7 + g)
    surv = _surv(rng, B, g, kind)
    c = rng.uniform(0.05, 0.6, B).astype(np.float32)
    c[0] = np.nan                      # NaN cutoff: nothing of request 0 is eligible
    for T in (0, 1, B, (B * g) // 3, B * g, B * g + 5):
        L = dspark.dspark_schedule(t(surv), "combined", cutoff=t(c), budget=T)
        torch.cuda.synchronize()
        want = oracle.cut_combined(surv.astype(np.float64), c, T)
        assert np.array_equal(L.cpu().numpy(), want), (T,)


def _run(cfg, steps, s_cutoff=None):
    for step in steps:
        s = make_step(cfg, step, device=DEV)
        if s_cutoff is not None:
            s.cutoff.copy_(s_cutoff(s))
        out = dspark.dspark_step(s.hidden, s.w, s.bias, s.temps, s.tokens, s.logits, cfg.mode,
                                 cutoff=s.cutoff, budget=s.budget)
        torch.cuda.synchronize()
        g = {k: v.cpu().numpy() for k, v in out.items()}
        h = snapshot(s)
        front = oracle_front(h)
        o = oracle_back(h, front, *oracle_rows(s, front))
        compare(g, o, h.tokens, ctx=f"{cfg.name} step {step}")


def test_combined_step_mixed_workload():
    cfg = CONFIGS["mixed_combined"]
    _run(cfg, range(12))


@pytest.mark.parametrize("case", ["small", "stage_path"])
def test_combined_step_edge(case):
    base = CONFIGS["mixed_combined"]
    cfg = {"small": base.scaled(B=8, d=256, V=1024),
           # B*gamma > 4096: the pick runs in the stage kernel, not in the front
           "stage_path": base.scaled(B=600, d=256, V=512)}[case]
    _run(cfg, range(3))


def test_cost_cutoff_lookup():
    table = np.array([0.05, 0.1, 0.2, 0.35, 0.5], np.float32)
    for load in (-3, 0, 2, 4, 9):
        c = dspark.dspark_cost_cutoff(t(table), t(np.array([load], np.int32)), 300)
        torch.cuda.synchronize()
        assert np.array_equal(c.cpu().numpy(), oracle.cost_cutoff(table, load, 300))


def test_cost_table_drives_the_step():
    # the cutoffs of the step come from the table on the device; the oracle
    # looks the same entry up itself. Higher load tightens every window.
    cfg = CONFIGS["mid"]
    table = np.array([0.1, 0.2, 0.3, 0.45], np.float32)
    prev = None
    for load in range(4):
        s = make_step(cfg, 0, device=DEV)
        dspark.dspark_cost_cutoff(t(table), t(np.array([load], np.int32)), cfg.B, cutoff=s.cutoff)
        out = dspark.dspark_step(s.hidden, s.w, s.bias, s.temps, s.tokens, s.logits, "threshold",
                                 cutoff=s.cutoff)
        torch.cuda.synchronize()
        g = {k: v.cpu().numpy() for k, v in out.items()}
        h = snapshot(s)
        h.cutoff = oracle.cost_cutoff(table, load, cfg.B)
        front = oracle_front(h)
        o = oracle_back(h, front, *oracle_rows(s, front))
        compare(g, o, h.tokens, ctx=f"cost table load {load}")
        if prev is not None:
            assert np.all(o.lengths <= prev)
        prev = o.lengths
