"""Graph tiers and HIP-graph replay of the verify step (needs an MI355X).

[P1] "DFlash to DSpark in SGLang", section "Ragged verify under full CUDA
graphs": a step replays the smallest captured tier that holds its packed total.
dspark_tier_select picks the tier and pads the packed
arrays on the device; it is compared with the oracle's tier pick. Every launch
shape of the library is independent of the packed total, so one captured graph
of the whole step (plus the tier pick) replays correctly for any schedule:
each replay is checked against an eager run on the same inputs, with eager
work and synchronisations between the replays.
"""
import numpy as np
import pytest
import torch

import __graft_entry__  # noqa: F401
import confidence_scheduled_ragged_amd as dspark
import oracle
from synth import CONFIGS, make_step

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


@pytest.mark.parametrize("seed", range(6))
def test_tier_select_matches_oracle(seed):
    rng = np.random.default_rng(900 + seed)
    B = int(rng.integers(1, 300))
    g = int(rng.integers(1, 20))
    cap = B * (g + 1)
    L = rng.integers(0, g + 1, B).astype(np.int32)
    tok = rng.integers(0, 5000, (B, g + 1)).astype(np.int32)
    ladder = np.unique(rng.integers(1, cap + 64, int(rng.integers(1, 10)))).astype(np.int32)
    cu, ptok, psrc, _ = dspark.dspark_compact(t(L), t(tok))
    padded, idx = dspark.dspark_tier_select(cu, g, t(ladder), -3, ptok, psrc)
    torch.cuda.synchronize()
    o_cu, o_pt, o_ps = oracle.compact(L, tok)
    # the oracle pads the oracle's own packed arrays (initialised as the binding's: -1)
    o_pad, o_idx, o_pt2, o_ps2 = oracle.tier_select(o_cu, g, ladder, -3, o_pt, o_ps)
    assert int(padded.item()) == o_pad and int(idx.item()) == o_idx
    assert np.array_equal(ptok.cpu().numpy(), o_pt2)
    assert np.array_equal(psrc.cpu().numpy(), o_ps2)


def _copy_inputs(dst, s):
    for k in ("hidden", "temps", "tokens", "logits", "cutoff"):
        getattr(dst, k).copy_(getattr(s, k))


@pytest.mark.parametrize("name,B", [("mixed_threshold", 64), ("mixed_threshold", 128),
                                    ("mixed_budget", 64)])
def test_step_graph_replays_match_eager(name, B):
    # B = 128 with a per-request cutoff is the one-launch form: its counters and
    # go word must be back at zero for every replay
    cfg = CONFIGS[name].scaled(B=B, V=32768)
    steps = [make_step(cfg, i, device=DEV) for i in range(4)]
    static = make_step(cfg, 0, device=DEV)          # the captured input buffers
    ladder = t(np.array([B, 2 * B, 4 * B, 8 * B, B * (cfg.gamma + 1)], np.int32))
    ws = dspark.workspace(cfg.B, cfg.gamma, cfg.V, DEV)
    out = dspark.alloc_step_outputs(cfg.B, cfg.gamma, DEV)
    tier = {"padded_total": torch.empty(1, dtype=torch.int32, device=DEV),
            "tier_index": torch.empty(1, dtype=torch.int32, device=DEV)}

    def body():
        dspark.dspark_step(static.hidden, static.w, static.bias, static.temps, static.tokens,
                           static.logits, cfg.mode, cutoff=static.cutoff, budget=static.budget,
                           out=out, ws=ws)
        dspark.dspark_tier_select(out["cu_seqlens"], cfg.gamma, ladder, 0, out["packed_tokens"],
                                  out["packed_src_row"], out=tier)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        body()                                        # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        body()
    torch.cuda.synchronize()
    for rep in range(3):
        for i, s in enumerate(steps):
            _copy_inputs(static, s)
            for v in out.values():
                v.fill_(-7)
            graph.replay()
            torch.cuda.synchronize()
            got = {k: v.cpu().numpy().copy() for k, v in out.items()}
            got_tier = (int(tier["padded_total"].item()), int(tier["tier_index"].item()))
            # eager run of the same step into fresh outputs
            e = dspark.alloc_step_outputs(cfg.B, cfg.gamma, DEV)
            dspark.dspark_step(s.hidden, s.w, s.bias, s.temps, s.tokens, s.logits, cfg.mode,
                               cutoff=s.cutoff, budget=s.budget, out=e, ws=ws)
            et = dspark.dspark_tier_select(e["cu_seqlens"], cfg.gamma, ladder, 0,
                                           e["packed_tokens"], e["packed_src_row"])
            torch.cuda.synchronize()
            total = int(e["cu_seqlens"][-1].item())
            assert got_tier == (int(et[0].item()), int(et[1].item())), (rep, i)
            pad_end = min(got_tier[0], cfg.B * (cfg.gamma + 1))
            for k, v in e.items():
                ev = v.cpu().numpy()
                if k in ("packed_tokens", "packed_src_row"):
                    assert np.array_equal(got[k][:pad_end], ev[:pad_end]), (rep, i, k)
                elif k == "packed_argmax":
                    assert np.array_equal(got[k][:total], ev[:total]), (rep, i, k)
                else:
                    assert np.array_equal(got[k], ev), (rep, i, k)


@pytest.mark.parametrize("name", ["mixed_threshold", "mixed_budget"])
def test_profiled_step_matches_step_and_brackets_the_dominant_kernel(name):
    # dspark_step_ex with timing events gives dspark_step's results and records them
    # around the dominant kernel, inside the step's own event pair: the whole
    # step in one launch (per-request cutoff, B = 128), the stream kernel of
    # two launches (budget)
    cfg = CONFIGS[name].scaled(B=128, V=65536)
    s = make_step(cfg, 1, device=DEV)
    ref = dspark.dspark_step(s.hidden, s.w, s.bias, s.temps, s.tokens, s.logits, cfg.mode,
                             cutoff=s.cutoff, budget=s.budget)
    ref = {k: v.cpu().numpy() for k, v in ref.items()}
    e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    e[0].record()
    got = dspark.dspark_step_ex(s.hidden, s.w, s.bias, s.temps, s.tokens, s.logits, cfg.mode,
                                cutoff=s.cutoff, budget=s.budget, events=(e[1], e[2]))
    e[3].record()
    torch.cuda.synchronize()
    for k, v in got.items():
        assert np.array_equal(v.cpu().numpy(), ref[k]), k
    step_ms, kern_ms = e[0].elapsed_time(e[3]), e[1].elapsed_time(e[2])
    assert 0.0 < kern_ms <= step_ms
    if name == "mixed_budget":
        assert e[0].elapsed_time(e[1]) > 0.0  # the front ran before the bracket opened
