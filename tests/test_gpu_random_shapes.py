"""Seeded random shapes through the fused step (needs an MI355X).

Each case draws a batch size (around the one-launch threshold of 96 requests
and the 4096-position limit of the in-kernel pick), a block length, odd and
even hidden sizes and vocabularies (scalar and 16-byte paths, V = 1 included),
a cut and a budget, then runs dspark_step in both forms: the two must agree
bit for bit, and the one-launch outputs must match the oracle (integers
exactly, conf and survival within 1e-5, a length flip allowed only on a
request holding an ambiguous position).
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
N_CASES = 120


def _cases():
    rng = np.random.default_rng(20261203)
    base = CONFIGS["mixed_combined"]
    out = []
    for c in range(N_CASES):
        B = int(rng.choice([1, 2, 3, 17, 64, 95, 96, 97, 128, 255, 256, 300, 511]))
        g = int(rng.choice([1, 2, 3, 7, 8, 15, 16, 31, 64]))
        if B * g > 6000:
            g = max(1, 6000 // B)
        d = int(rng.choice([8, 64, 250, 256, 1000, 4096]))
        V = int(rng.choice([1, 7, 64, 1001, 2048, 4096]))
        mode = str(rng.choice(["threshold", "budget", "static", "combined"]))
        bpr = float(rng.choice([0.0, 0.5, 1.3, 2.9, 7.0, 100.0]))
        cut = float(rng.choice([0.05, 0.25, 0.6]))
        out.append(base.scaled(B=B, gamma=g, d=d, V=V, mode=mode, budget_per_request=bpr,
                               cutoff=cut, steps=1))
    return out


def _run(s, launches):
    out = dspark.dspark_step(s.hidden, s.w, s.bias, s.temps, s.tokens, s.logits, s.cfg.mode,
                             cutoff=s.cutoff, budget=s.budget, launches=launches)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def test_random_shapes_both_forms_match_the_oracle():
    amb = 0
    for c, cfg in enumerate(_cases()):
        s = make_step(cfg, c, device=DEV)
        one = _run(s, 1)
        two = _run(s, 2)
        tag = f"case {c}: B={cfg.B} gamma={cfg.gamma} d={cfg.d} V={cfg.V} {cfg.mode} T={s.budget}"
        for k in one:
            assert np.array_equal(one[k], two[k]), f"{tag}: {k} differs between forms"
        rep = compare(one, run_oracle(s), s.host("tokens"), ctx=tag)
        amb += rep.ambiguous_positions
    print(f"\n[random shapes] {N_CASES} cases, ambiguous positions {amb}")
