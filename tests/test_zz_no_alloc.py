"""dspark_step_noalloc against dspark_step (needs an MI355X).

The no-alloc entry point runs the same kernels as dspark_step on the library's
own per-device scratch array instead of a caller's workspace. Its outputs must
equal dspark_step's bit for bit (the integers exactly, conf and survival too,
since the arithmetic is the same) on consecutive calls that share the scratch:
a large batch in one launch, then a smaller one in two launches, then a large
one again. Each result is also checked against the oracle. The scratch's give-up
flag must read 0 after each call.
"""
import numpy as np
import pytest
import torch

import __graft_entry__  # noqa: F401
import confidence_scheduled_ragged_amd as dspark
from parity_utils import compare, run_oracle
from synth import CONFIGS, make_step

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _host(out):
    return {k: v.cpu().numpy() for k, v in out.items()}


def _both(s):
    ref = dspark.dspark_step(s.hidden, s.w, s.bias, s.temps, s.tokens, s.logits, s.cfg.mode,
                             cutoff=s.cutoff, budget=s.budget)
    torch.cuda.synchronize()
    ref = _host(ref)
    status = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    got = dspark.dspark_step_noalloc(s.hidden, s.w, s.bias, s.temps, s.tokens, s.logits,
                                     s.cfg.mode, cutoff=s.cutoff, budget=s.budget, status=status)
    torch.cuda.synchronize()
    return ref, _host(got), int(status.item())


def test_noalloc_matches_step_on_consecutive_calls():
    cases = [
        # B = 256: the one-launch form (per-request cutoff)
        ("large threshold", CONFIGS["mixed_threshold"].scaled(V=16384), 0),
        # a smaller batch next, with a batch-wide budget: two launches
        ("small budget", CONFIGS["mixed_budget"].scaled(B=40, V=8192, d=1024), 1),
        # odd sizes (scalar paths), then the large batch again on the same scratch
        ("odd combined", CONFIGS["tiny"].scaled(B=7, d=250, V=1001, mode="combined",
                                                budget_per_request=2.0), 2),
        ("large threshold again", CONFIGS["mixed_threshold"].scaled(V=16384), 3),
    ]
    for name, cfg, step in cases:
        s = make_step(cfg, step, device=DEV)
        ref, got, st = _both(s)
        assert st == 0, f"{name}: a wait gave up"
        total = int(ref["cu_seqlens"][-1])
        for k in ref:
            a, b = ref[k], got[k]
            if k in ("packed_tokens", "packed_src_row", "packed_argmax"):
                a, b = a[:total], b[:total]
            assert np.array_equal(a, b), f"{name}: {k} differs from dspark_step"
        compare(got, run_oracle(s), s.host("tokens"), ctx=name)


def test_noalloc_rejects_sizes_beyond_its_scratch():
    # B*(gamma+1) rows whose workspace exceeds the 4 MiB scratch: a clear error,
    # nothing enqueued
    cfg = CONFIGS["tiny"].scaled(B=20000, gamma=16, d=8, V=8)
    s = make_step(cfg, 0, device=DEV)
    with pytest.raises(dspark.DsparkError) as e:
        dspark.dspark_step_noalloc(s.hidden, s.w, s.bias, s.temps, s.tokens, s.logits,
                                   cfg.mode, cutoff=s.cutoff, budget=s.budget)
    assert e.value.status == 5  # DSPARK_ERR_WORKSPACE
