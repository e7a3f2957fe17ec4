"""The fused step's two forms (needs an MI355X).

Threshold and static cuts run the whole step in one launch from 96 requests up
and in two below; budget and combined cuts run in two. dspark_step_ex's
`launches` argument (1 or 2) selects a form for any size where the cut allows
it. Both forms must match the oracle, match each other bit for bit, and leave
the workspace's counters at zero, so that calls of either form can follow each
other on one workspace. The one-launch form's bounded wait is driven to give
up from the host (a wait bound of one clock tick): the give-up must be reported
by dspark_step_status, every kernel must still finish, and the next call on
the same workspace must be exact without re-initialising it.
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


def _host(out):
    return {k: v.cpu().numpy() for k, v in out.items()}


def _step(s, ws, two_launches, wait_ticks=0):
    out = dspark.dspark_step(s.hidden, s.w, s.bias, s.temps, s.tokens, s.logits, s.cfg.mode,
                             cutoff=s.cutoff, budget=s.budget, ws=ws,
                             launches=2 if two_launches else 1, wait_ticks=wait_ticks)
    torch.cuda.synchronize()
    return _host(out)


def _status(ws):
    st = dspark.dspark_step_status(ws)
    torch.cuda.synchronize()
    return int(st.item())


def _fresh_ws(cfg):
    n = dspark.dspark_workspace_bytes(cfg.B, cfg.gamma, cfg.V)
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    ws.fill_(0xA5)          # the init call must clear it
    dspark.dspark_workspace_init(ws)
    return ws


def _counters_zero(ws, B):
    # the control words and every per-request counter (spread over the array)
    head = ws[: CTRL_BYTES + 8 * MAX_FUSED_B].cpu().numpy()
    return int(np.count_nonzero(head)) == 0


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
    # below 96 requests the two-launch stream runs half the waves, each
    # sub-chunk (here over 4096 slots) four loads deep
    "small_batch_long": CONFIGS["mixed_threshold"].scaled(B=95),
    "small_batch_static": CONFIGS["mixed_threshold"].scaled(B=64, mode="static"),
    # the full static block at full size: in two launches every sub-chunk is
    # long (about 19 000 slots), two loads deep
    "static_full": CONFIGS["mixed_threshold"].scaled(mode="static"),
    # draft slots past 2^32 (4 x 16 rows of an odd vocabulary of 70 000 001,
    # one slot per logit on the scalar path): the slot arithmetic of both forms
    # takes its wide division path
    "wide_slots": CONFIGS["tiny"].scaled(B=4, gamma=16, d=64, V=70_000_001, cutoff=0.0),
    # the same past 2^32 under a batch budget (T = 62 of 64 positions: the
    # front's pick, then 62 draft rows, 4.3e9 slots)
    "wide_slots_budget": CONFIGS["tiny"].scaled(B=4, gamma=16, d=64, V=70_000_001, mode="budget",
                                                budget_per_request=15.5),
    # batch-wide picks (two launches under either setting): B*gamma = 4096
    # positions, the most the in-kernel pick takes; d = 7168 reads a 14 KiB
    # head; odd d and V take the scalar paths; a batch over 4096 positions
    # takes the stage kernel's pick
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
def test_both_forms_match_the_oracle_and_each_other(name):
    cfg = CASES[name]
    ws = _fresh_ws(cfg)
    for step in range(2):
        s = make_step(cfg, step, device=DEV)
        if name in TIED:
            s.hidden.zero_()
        one = _step(s, ws, False)
        assert _counters_zero(ws, cfg.B), f"{name}: counters left set by the one-launch form"
        two = _step(s, ws, True)
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
    assert _status(ws) == 0, f"{name}: a wait gave up"


def test_forms_alternate_on_one_workspace():
    # one form after the other, repeatedly, on the same workspace: each call
    # must start from the counters the previous one returned to zero
    cfg = CONFIGS["mixed_threshold"].scaled(B=64, V=16384)
    ws = _fresh_ws(cfg)
    steps = [make_step(cfg, i, device=DEV) for i in range(3)]
    steps.append(make_step(CONFIGS["mixed_budget"].scaled(B=64, V=16384), 0, device=DEV))
    ref = [_step(s, ws, False) for s in steps]
    for rnd in range(4):
        for i, s in enumerate(steps):
            got = _step(s, ws, (rnd + i) % 2 == 1)
            for k in got:
                assert np.array_equal(got[k], ref[i][k]), f"round {rnd} step {i}: {k}"
    assert _counters_zero(ws, cfg.B)


def test_give_up_is_reported_and_the_next_call_is_exact():
    # B = 128 takes the one-launch form; its grid holds idle stream workgroups
    # that wait for the lengths from their first instruction, so a bound of one
    # tick of the 100 MHz clock makes them give up. Every kernel still ends:
    # the give-up path only sets the flag, leaves the go word and returns.
    cfg = CONFIGS["mixed_threshold"].scaled(B=128, V=16384)
    ws = _fresh_ws(cfg)
    steps = [make_step(cfg, i, device=DEV) for i in range(2)]
    ref = [_step(s, ws, False) for s in steps]
    assert _status(ws) == 0
    _step(steps[0], ws, False, wait_ticks=1)
    assert _status(ws) == 1, "the give-up was not reported"
    assert _status(ws) == 0, "the status read must clear the flag"
    # the next calls on the same workspace, not re-initialised, are exact
    for i, s in enumerate(steps):
        got = _step(s, ws, False)
        for k in got:
            assert np.array_equal(got[k], ref[i][k]), f"after the give-up, step {i}: {k}"
        h = snapshot(s)
        front = oracle_front(h)
        compare(got, oracle_back(h, front, *oracle_rows(s, front)), h.tokens,
                ctx=f"after the give-up, step {i}")
    assert _status(ws) == 0
    assert _counters_zero(ws, cfg.B)
    # and so is the two-launch form after another give-up
    _step(steps[1], ws, False, wait_ticks=1)
    got = _step(steps[1], ws, True)
    assert _status(ws) == 1
    for k in got:
        assert np.array_equal(got[k], ref[1][k]), f"two launches after a give-up: {k}"
