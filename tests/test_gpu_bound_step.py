"""BoundStep: dspark_step with its arguments checked once (needs an MI355X).

The bound call launches the same C entry point on the same buffers, so its
outputs must equal dspark_step's bit for bit, also after the input buffers are
refilled in place with the next step's data (serving-loop use), in every form,
and on a stream given at binding.
"""
import numpy as np
import pytest
import torch

import __graft_entry__  # noqa: F401
import confidence_scheduled_ragged_amd as dspark
from synth import CONFIGS, make_step

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _host(o):
    return {k: v.cpu().numpy() for k, v in o.items()}


def _ref(cfg, s, ws, launches=0):
    return _host(dspark.dspark_step(s.hidden, s.w, s.bias, s.temps, s.tokens, s.logits,
                                    cfg.mode, cutoff=s.cutoff, budget=s.budget, ws=ws,
                                    launches=launches))


@pytest.mark.parametrize("name,B,launches", [("mid", 64, 0), ("mid", 64, 1), ("mid", 64, 2),
                                             ("mixed_budget", 96, 0), ("batch1", 1, 0)])
def test_bound_step_matches_dspark_step_across_refills(name, B, launches):
    cfg = CONFIGS[name].scaled(B=B, V=32768)
    steps = [make_step(cfg, i, device=DEV) for i in range(3)]
    ws = dspark.workspace(cfg.B, cfg.gamma, cfg.V, DEV)
    live = make_step(cfg, 0, device=DEV)  # the bound input buffers
    call = dspark.bind_step(live.hidden, live.w, live.bias, live.temps, live.tokens,
                            live.logits, cfg.mode, cutoff=live.cutoff, budget=live.budget,
                            ws=ws, launches=launches)
    for rnd in range(2):
        for i, s in enumerate(steps):
            for k in ("hidden", "temps", "tokens", "logits", "cutoff"):
                getattr(live, k).copy_(getattr(s, k))
            for v in call.out.values():
                v.fill_(-7)
            got = _host(call())
            torch.cuda.synchronize()
            ref = _ref(cfg, s, ws, launches)
            total = int(ref["cu_seqlens"][-1])
            for k in ref:
                g, r = got[k], ref[k]
                if k.startswith("packed_"):  # written up to the packed total only
                    g, r = g[:total], r[:total]
                assert np.array_equal(g, r), (rnd, i, k)


def test_bound_step_on_a_given_stream():
    cfg = CONFIGS["mid"].scaled(B=32, V=16384)
    s = make_step(cfg, 1, device=DEV)
    ws = dspark.workspace(cfg.B, cfg.gamma, cfg.V, DEV)
    ref = _ref(cfg, s, ws)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    call = dspark.bind_step(s.hidden, s.w, s.bias, s.temps, s.tokens, s.logits, cfg.mode,
                            cutoff=s.cutoff, budget=s.budget, ws=ws, stream=side.cuda_stream)
    call()
    side.synchronize()
    got = _host(call.out)
    total = int(ref["cu_seqlens"][-1])
    for k in ref:
        g, r = got[k], ref[k]
        if k.startswith("packed_"):
            g, r = g[:total], r[:total]
        assert np.array_equal(g, r), k


def test_bind_step_checks_its_arguments():
    cfg = CONFIGS["tiny"]
    s = make_step(cfg, 0, device=DEV)
    with pytest.raises(TypeError):
        dspark.bind_step(s.hidden.float(), s.w, s.bias, s.temps, s.tokens, s.logits, cfg.mode,
                         cutoff=s.cutoff)
    with pytest.raises(ValueError):
        dspark.bind_step(s.hidden, s.w, s.bias, s.temps, s.tokens[:, :-1].contiguous(),
                         s.logits, cfg.mode, cutoff=s.cutoff)
