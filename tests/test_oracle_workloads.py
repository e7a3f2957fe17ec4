"""The oracle on generated workloads (CPU): invariants the definitions imply and
the planting pin from the generator's record."""
import numpy as np
import pytest

from parity_utils import planted_accept_pin, run_oracle
from synth import CONFIGS, make_step

SMALL = {
    "tiny": CONFIGS["tiny"],
    "batch1": CONFIGS["batch1"].scaled(d=512, V=4096),
    "mid": CONFIGS["mid"].scaled(B=16, d=512, V=4096),
    "budget": CONFIGS["budget"].scaled(B=32, d=512, V=2048),
    "mixed_threshold": CONFIGS["mixed_threshold"].scaled(B=32, d=512, V=2048),
    "mixed_budget": CONFIGS["mixed_budget"].scaled(B=32, d=512, V=2048),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_oracle_invariants_on_workload(name):
    cfg = SMALL[name]
    for step in range(3):
        s = make_step(cfg, step, device="cpu")
        o = run_oracle(s)
        assert np.all(np.diff(o.surv, axis=1) <= 0)
        assert np.all((o.surv >= 0) & (o.surv <= 1))
        assert np.all(o.accepted <= o.lengths)
        assert o.cu[-1] == int((o.lengths + 1).sum())
        if cfg.mode == "threshold":
            keep = o.surv.astype(np.float32) >= s.host("cutoff")[:, None]
            assert np.array_equal(o.lengths, keep.sum(axis=1))
        else:
            assert o.lengths.sum() == min(s.budget, cfg.B * cfg.gamma)
        planted_accept_pin(s, o)


def test_generator_is_deterministic():
    a = make_step(SMALL["mid"], 1, device="cpu")
    b = make_step(SMALL["mid"], 1, device="cpu")
    assert a.digest() == b.digest()
    c = make_step(SMALL["mid"], 2, device="cpu")
    assert a.digest() != c.digest()


def test_planted_rows_have_unique_argmax():
    s = make_step(SMALL["batch1"], 0, device="cpu")
    lg = s.host("logits").astype(np.uint32) << 16
    f = lg.view(np.float32)
    tok = s.host("tokens")
    for b, i in zip(*np.nonzero(s.plant)):
        row = f[b, i]
        t = tok[b, i + 1]
        assert row[t] == row.max() and np.sum(row == row.max()) == 1


def test_combined_band_with_zero_budget():
    # With T = 0 the combined cut keeps nothing, so a position lying on its
    # request's cutoff is not ambiguous: the parity bookkeeping must give every
    # request the exact length 0 (it once took the cutoff's band instead, whose
    # lower end counts the positions certainly above the cutoff).
    import oracle
    from parity_utils import oracle_front, snapshot

    cfg = CONFIGS["tiny"].scaled(mode="combined", budget_per_request=0.0)
    h = snapshot(make_step(cfg, 0))
    _, conf = oracle.confidence(h.hidden, h.w, h.bias, h.temps)
    surv = oracle.survival(conf)
    # every request's second position on its cutoff, its first well above it
    h.cutoff = surv[:, 1].astype(np.float32)
    assert np.all(surv[:, 0] > surv[:, 1] + 1e-3)
    f = oracle_front(h)
    assert h.budget == 0
    assert not f.lengths.any()
    assert f.ambiguous_positions == 0
    assert np.array_equal(f.len_lo, f.lengths) and np.array_equal(f.len_hi, f.lengths)
