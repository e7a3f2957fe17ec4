"""The fused step's two forms (needs an MI355X).

Every cut runs the whole step in one launch from 96 requests up, in two
below; the environment variable DSPARK_STEP_LAUNCHES (1 or 2) selects a form
for any size. Threshold and static cuts take step_one_kernel as their one
launch; budget and combined cuts take step_pick_kernel (the head one hidden
row per wave, the batch-wide pick in workgroup 0) while B*gamma <= 4096 and
two launches beyond. Both forms must match the oracle, match each other bit
for bit, and leave the workspace's counters and score slots at zero, so that
calls of either form can follow each other on one workspace.
"""
import numpy as np
import pytest
import torch

import __graft_entry__  # noqa: F401
import confidence_scheduled_ragged_amd as dspark
from parity_utils import compare, oracle_back, oracle_front, oracle_rows, snapshot
from synth import CONFIGS, make_step

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CTRL_BYTES = 256       # control words at the start of the workspace
MAX_FUSED_B = 4096     # per-request counters that follow them (uint64 each)
PICK_SLOTS = 4096      # score slots of the one-launch pick, after both counter sets


def _host(out):
    return {k: v.cpu().numpy() for k, v in out.items()}


def _step(s, ws, two_launches, monkeypatch):
    monkeypatch.setenv("DSPARK_STEP_LAUNCHES", "2" if two_launches else "1")
    out = dspark.dspark_step(s.hidden, s.w, s.bias, s.temps, s.tokens, s.logits, s.cfg.mode,
                             cutoff=s.cutoff, budget=s.budget, ws=ws)
    torch.cuda.synchronize()
    monkeypatch.delenv("DSPARK_STEP_LAUNCHES", raising=False)
    return _host(out)


def _fresh_ws(cfg):
    n = dspark.dspark_workspace_bytes(cfg.B, cfg.gamma, cfg.V)
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    ws.fill_(0xA5)          # the init call must clear it
    dspark.dspark_workspace_init(ws)
    return ws


def _counters_zero(ws, B):
    head = ws[: CTRL_BYTES + 8 * min(B, MAX_FUSED_B)].cpu().numpy()
    slot0 = CTRL_BYTES + 16 * MAX_FUSED_B
    slots = ws[slot0: slot0 + 8 * PICK_SLOTS].cpu().numpy()
    return int(np.count_nonzero(head)) == 0 and int(np.count_nonzero(slots)) == 0


CASES = {
    "tiny": CONFIGS["tiny"],
    "mixed_threshold": CONFIGS["mixed_threshold"].scaled(V=32768),
    "static": CONFIGS["tiny"].scaled(mode="static"),
    "max_gamma": CONFIGS["tiny"].scaled(gamma=256, B=2, V=512, d=64),
    "odd_vocab": CONFIGS["tiny"].scaled(V=1001, d=250),
    "wide_batch": CONFIGS["tiny"].scaled(B=700, gamma=4, d=64, V=256),
    # the largest batch of the fused step: each request workgroup runs 16
    # requests, and cu_seqlens fills 32 KiB of LDS
    "max_batch": CONFIGS["tiny"].scaled(B=4096, gamma=4, d=128, V=512),
    # batch-wide picks: B*gamma = 4096 positions, the most the one-launch pick
    # takes; d = 7168 stages a 14 KiB head; odd d and V take the scalar paths;
    # a batch over 4096 positions takes two launches under either setting
    "mixed_budget": CONFIGS["mixed_budget"].scaled(V=32768),
    "budget_d7168": CONFIGS["budget"].scaled(V=16384),
    "mixed_combined": CONFIGS["mixed_combined"].scaled(V=32768),
    "tiny_budget": CONFIGS["tiny"].scaled(mode="budget", budget_per_request=2.5),
    "odd_budget": CONFIGS["tiny"].scaled(B=100, d=250, V=1001, mode="budget",
                                         budget_per_request=3.3),
    "long_block_budget": CONFIGS["tiny"].scaled(B=16, gamma=256, d=64, V=512, mode="budget",
                                                budget_per_request=40.0),
    "wide_combined": CONFIGS["tiny"].scaled(B=700, gamma=4, d=64, V=256, mode="combined",
                                            budget_per_request=1.5),
    "over_slots_budget": CONFIGS["tiny"].scaled(B=1100, gamma=4, d=64, V=256, mode="budget",
                                                budget_per_request=1.5),
    # zero hidden states: every request has the same survival curve, so the
    # budget's cut value is shared by many requests and ties decide the split
    "tied_budget": CONFIGS["mixed_budget"].scaled(V=4096, d=256),
    "tied_combined": CONFIGS["mixed_combined"].scaled(V=4096, d=256, cutoff=0.05),
}
TIED = ("tied_budget", "tied_combined")


@pytest.mark.parametrize("name", list(CASES))
def test_both_forms_match_the_oracle_and_each_other(name, monkeypatch):
    cfg = CASES[name]
    ws = _fresh_ws(cfg)
    for step in range(2):
        s = make_step(cfg, step, device=DEV)
        if name in TIED:
            s.hidden.zero_()
        one = _step(s, ws, False, monkeypatch)
        assert _counters_zero(ws, cfg.B), f"{name}: counters left set by the one-launch form"
        two = _step(s, ws, True, monkeypatch)
        assert _counters_zero(ws, cfg.B), f"{name}: counters left set by the two-launch form"
        for k in one:
            assert np.array_equal(one[k], two[k]), f"{name} step {step}: {k} differs between forms"
        if cfg.mode in ("budget", "combined"):
            # the stage kernel's select on the step's own survival must cut the
            # same lengths as the fused step's select
            L = dspark.dspark_schedule(torch.from_numpy(one["survival"]).to(DEV), cfg.mode,
                                       cutoff=s.cutoff, budget=s.budget)
            torch.cuda.synchronize()
            assert np.array_equal(L.cpu().numpy(), one["lengths"]), f"{name} step {step}"
        h = snapshot(s)
        front = oracle_front(h)
        compare(one, oracle_back(h, front, *oracle_rows(s, front)), h.tokens,
                ctx=f"{name} step {step}")


def test_forms_alternate_on_one_workspace(monkeypatch):
    # one form after the other, repeatedly, on the same workspace: each call
    # must start from the counters the previous one returned to zero
    cfg = CONFIGS["mixed_threshold"].scaled(B=64, V=16384)
    ws = _fresh_ws(cfg)
    steps = [make_step(cfg, i, device=DEV) for i in range(3)]
    steps.append(make_step(CONFIGS["mixed_budget"].scaled(B=64, V=16384), 0, device=DEV))
    ref = [_step(s, ws, False, monkeypatch) for s in steps]
    for rnd in range(4):
        for i, s in enumerate(steps):
            got = _step(s, ws, (rnd + i) % 2 == 1, monkeypatch)
            for k in got:
                assert np.array_equal(got[k], ref[i][k]), f"round {rnd} step {i}: {k}"
    assert _counters_zero(ws, cfg.B)
