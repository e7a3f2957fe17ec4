"""GPU parity of every C-ABI entry point against the oracle (needs an MI355X).

Each stage entry point gets generated or hand-built inputs that are handed to
both sides; the fused step is compared end to end on the seeded workloads.
Integers must match exactly; conf and survival within 1e-5 of the fp64 oracle.
"""
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import __graft_entry__  # noqa: F401
import confidence_scheduled_ragged_amd as dspark
import oracle
from parity_utils import (compare, oracle_back, oracle_front, oracle_rows, planted_accept_pin,
                          snapshot)
from synth import CONFIGS, bf16_bits_to_f32, make_step, rne_bf16

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def to_bf16(a: np.ndarray) -> torch.Tensor:
    bits = rne_bf16(np.asarray(a, np.float32))
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(DEV)


def bits_tensor(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).view(torch.bfloat16).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


# ------------------------------------------------------------ confidence

@pytest.mark.parametrize("B,g,d", [(4, 8, 256), (3, 5, 1000), (2, 16, 4101), (64, 16, 4096),
                                   (5, 3, 20000), (1, 1, 8), (2, 64, 7168)])
def test_confidence_stage(B, g, d):
    rng = np.random.default_rng(B * 1000 + g * 10 + d)
    hb = rne_bf16(rng.standard_normal((B, g, d)).astype(np.float32))
    wb = rne_bf16((rng.standard_normal(d) / math.sqrt(d)).astype(np.float32))
    temps = (1 + 0.03 * np.arange(g)).astype(np.float32)
    bias = float(np.float32(0.2))
    conf, surv = dspark.dspark_confidence(bits_tensor(hb), bits_tensor(wb), bias,
                                          torch.from_numpy(temps).to(DEV))
    c2, s2 = dspark.dspark_confidence(bits_tensor(hb), bits_tensor(wb), bias,
                                      torch.from_numpy(temps).to(DEV))
    torch.cuda.synchronize()
    _, oc = oracle.confidence(hb, wb, bias, temps)
    os_ = oracle.survival(oc)
    assert np.max(np.abs(host(conf) - oc)) <= 1e-5
    assert np.max(np.abs(host(surv) - os_)) <= 1e-5
    assert np.all(np.diff(host(surv), axis=1) <= 0)
    assert torch.equal(conf, c2) and torch.equal(surv, s2)       # bit-reproducible


# -------------------------------------------------------------- schedule

def _sched_cases():
    rng = np.random.default_rng(7)
    cases = []
    for B, g in [(4, 8), (64, 16), (256, 16), (1000, 7), (3, 1), (2, 64)]:
        p = rng.uniform(0.3, 1.0, (B, g))
        s = np.cumprod(p, axis=1).astype(np.float32)
        cases.append((f"rand{B}x{g}", s))
    cases.append(("all_equal", np.full((6, 5), 0.5, np.float32)))
    cases.append(("saturated", np.ones((8, 16), np.float32)))
    q = np.cumprod(np.full((5, 8), 0.5), axis=1).astype(np.float32)
    cases.append(("repeated_rows", q))
    z = np.zeros((3, 4), np.float32)
    z[:, 0] = 0.5
    cases.append(("zeros", z))
    return cases


@pytest.mark.parametrize("name,surv", _sched_cases(), ids=[c[0] for c in _sched_cases()])
def test_schedule_stage(name, surv):
    B, g = surv.shape
    rng = np.random.default_rng(B + g)
    s_dev = torch.from_numpy(surv).to(DEV)
    # threshold: random cutoffs plus the special values
    cut = rng.uniform(0, 1, B).astype(np.float32)
    cut[: min(B, 4)] = np.array([0.0, -1.0, 1.5, np.nan], np.float32)[: min(B, 4)]
    if B > 4:
        cut[4] = surv[4, g // 2]                                      # exact tie: kept
    L = dspark.dspark_schedule(s_dev, "threshold", cutoff=torch.from_numpy(cut).to(DEV))
    ref = oracle.cut_threshold(surv.astype(np.float64), cut)
    assert np.array_equal(host(L), ref)
    # budget: edge budgets and a sweep
    N = B * g
    for T in sorted({0, 1, N // 3, N // 2, N - 1, N, N + 5, int(rng.integers(0, N + 1))}):
        L = dspark.dspark_schedule(s_dev, "budget", budget=T)
        ref = oracle.cut_budget(surv.astype(np.float64), T)
        assert np.array_equal(host(L), ref), (name, T)


# --------------------------------------------------------------- compact

# up to 4096 requests and 65536 positions one thread per position, beyond
# that one workgroup: (4096, 15) is exactly at the position limit, (5000, 2)
# and (300, 256) beyond one limit each
@pytest.mark.parametrize("B,g", [(4, 8), (256, 16), (1500, 3), (1, 1), (3, 64), (4096, 15),
                                 (5000, 2), (300, 256)])
def test_compact_stage(B, g):
    rng = np.random.default_rng(B * 31 + g)
    L = rng.integers(0, g + 1, B).astype(np.int32)
    tok = rng.integers(0, 150000, (B, g + 1)).astype(np.int32)
    cu, pt, ps, _ = dspark.dspark_compact(torch.from_numpy(L).to(DEV), torch.from_numpy(tok).to(DEV))
    ocu, opt, ops = oracle.compact(L, tok)
    assert np.array_equal(host(cu), ocu)
    total = int(ocu[-1])
    assert np.array_equal(host(pt), opt) and np.array_equal(host(ps), ops)   # incl. -1 tails
    assert total == int((L + 1).sum())


def test_compact_clamps_lengths_and_gathers_rows():
    B, g, V = 6, 4, 1000
    rng = np.random.default_rng(3)
    raw = np.array([-3, 0, 2, 4, 9, 1], np.int32)
    tok = rng.integers(0, V, (B, g + 1)).astype(np.int32)
    logits = to_bf16(rng.standard_normal((B, g + 1, V)))
    cu, pt, ps, plog = dspark.dspark_compact(torch.from_numpy(raw).to(DEV),
                                             torch.from_numpy(tok).to(DEV), logits=logits)
    ocu, opt, ops = oracle.compact(np.clip(raw, 0, g), tok)
    assert np.array_equal(host(cu), ocu) and np.array_equal(host(ps), ops)
    total = int(ocu[-1])
    dense = logits.view(-1, V)
    assert torch.equal(plog[:total], dense[torch.from_numpy(ops[:total]).long().to(DEV)])
    assert torch.all(plog[total:].view(torch.int16) == 0)


# ---------------------------------------------------------------- accept

def _accept_case(B, g, V, seed, packed=False):
    rng = np.random.default_rng(seed)
    L = rng.integers(0, g + 1, B).astype(np.int32)
    lg = rng.standard_normal((B, g + 1, V)).astype(np.float32)
    tok = rng.integers(0, V, (B, g + 1)).astype(np.int32)
    # make the drafts agree with the rows for a random prefix
    bits = rne_bf16(lg)
    f = bf16_bits_to_f32(bits)
    for b in range(B):
        m = int(rng.integers(0, g + 1))
        for j in range(min(m, g)):
            tok[b, j + 1] = int(np.argmax(f[b, j]))
    cu, pt, ps = oracle.compact(L, tok)
    return L, tok, bits, cu, ps


@pytest.mark.parametrize("B,g,V", [(4, 8, 1024), (3, 5, 1000), (2, 16, 151936), (8, 2, 37),
                                   (5, 3, 1), (1, 1, 64), (64, 16, 129280), (2, 3, 8)])
def test_accept_stage_dense_and_packed(B, g, V):
    L, tok, bits, cu, ps = _accept_case(B, g, V, seed=B + g + V)
    total = int(cu[-1])
    amax = oracle.argmax_rows(bits.reshape(-1, V), ps[:total])
    acc, bon = oracle.accept(cu, tok, amax)
    lg = bits_tensor(bits)
    tok_d = torch.from_numpy(tok).to(DEV)
    cu_d = torch.from_numpy(cu).to(DEV)
    pam, a, bo = dspark.dspark_accept(lg, torch.from_numpy(ps).to(DEV), cu_d, tok_d)
    assert np.array_equal(host(pam)[:total], amax)
    assert np.all(host(pam)[total:] == -1)
    assert np.array_equal(host(a), acc) and np.array_equal(host(bo), bon)
    # already-packed logits, no source rows
    packed = np.zeros((B * (g + 1), V), np.uint16)
    packed[:total] = bits.reshape(-1, V)[ps[:total]]
    pam2, a2, bo2 = dspark.dspark_accept(bits_tensor(packed), None, cu_d, tok_d)
    assert np.array_equal(host(pam2)[:total], amax)
    assert np.array_equal(host(a2), acc) and np.array_equal(host(bo2), bon)


def test_accept_ties_across_waves_and_signed_zero():
    # Few rows of a long vocabulary: each row is split over many waves, so the
    # lowest-index rule must hold across wave boundaries.
    B, g, V = 1, 7, 151936
    f = np.full((B, g + 1, V), -1.0, np.float32)
    f[0, 0, [100000, 5]] = 7.0            # tie far apart -> 5
    f[0, 1, [8, 9]] = 7.0                 # tie inside one 16-byte slot -> 8
    f[0, 2, [15, 16]] = 7.0               # tie across a slot boundary -> 15
    f[0, 3, :] = 2.5                      # all equal -> 0
    f[0, 4, :] = -3.0
    f[0, 4, 3] = -0.0
    f[0, 4, 70000] = 0.0                  # -0 before +0 -> 3
    f[0, 5, :] = -3.0
    f[0, 5, 11] = 0.0
    f[0, 5, 90000] = -0.0                 # +0 before -0 -> 11
    f[0, 6, V - 1] = 9.0                  # last element
    f[0, 7, V - 9: V] = 9.0               # last slot, tie -> V-9
    bits = rne_bf16(f)
    bits[0, 4, 3] = 0x8000                # make sure -0 survives rounding
    bits[0, 5, 90000] = 0x8000
    tok = np.zeros((B, g + 1), np.int32)
    want = [5, 8, 15, 0, 3, 11, V - 1, V - 9]
    tok[0, 1:] = want[:g]
    L = np.array([g], np.int32)
    cu, pt, ps = oracle.compact(L, tok)
    amax = oracle.argmax_rows(bits.reshape(-1, V), ps)
    assert list(amax) == want
    pam, a, bo = dspark.dspark_accept(bits_tensor(bits), torch.from_numpy(ps).to(DEV),
                                      torch.from_numpy(cu).to(DEV), torch.from_numpy(tok).to(DEV))
    assert list(host(pam)) == want
    assert host(a)[0] == g and host(bo)[0] == V - 9


def test_accept_out_of_range_source_rows_are_contained():
    B, g, V = 2, 2, 256
    rng = np.random.default_rng(5)
    bits = rne_bf16(rng.standard_normal((B, g + 1, V)).astype(np.float32))
    tok = rng.integers(0, V, (B, g + 1)).astype(np.int32)
    cu = np.array([0, 3, 6], np.int32)
    ps = np.array([0, 1, 2, 99, -4, 5], np.int32)    # two rows outside the dense block
    pam, a, bo = dspark.dspark_accept(bits_tensor(bits), torch.from_numpy(ps).to(DEV),
                                      torch.from_numpy(cu).to(DEV), torch.from_numpy(tok).to(DEV))
    p = host(pam)
    assert p[3] == -1 and p[4] == -1
    good = oracle.argmax_rows(bits.reshape(-1, V), ps[[0, 1, 2, 5]])
    assert list(p[[0, 1, 2, 5]]) == list(good)


# ----------------------------------------------------------- fused step

def _gpu_step(s, out=None):
    out = dspark.dspark_step(s.hidden, s.w, s.bias, s.temps, s.tokens, s.logits, s.cfg.mode,
                             cutoff=s.cutoff, budget=s.budget, out=out)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in out.items()}


def _run_workload(cfg, steps, tag):
    """GPU step and oracle step on each seeded step. The oracle runs in worker
    threads on host copies of the generated inputs; the packed rows it reads
    are the ones its own schedule selects."""
    reports = []
    futs = []
    with ThreadPoolExecutor(8) as pool:
        for step in steps:
            s = make_step(cfg, step, device=DEV)
            g = _gpu_step(s)
            h = snapshot(s)
            front = oracle_front(h)
            rows = oracle_rows(s, front)
            del s

            def job(h=h, front=front, rows=rows, g=g, step=step):
                o = oracle_back(h, front, *rows)
                rep = compare(g, o, h.tokens, ctx=f"{tag} step {step}")
                planted_accept_pin(h, o)
                return rep

            futs.append(pool.submit(job))
            if len(futs) - len(reports) > 12:
                reports.append(futs[len(reports)].result())
        for f in futs[len(reports):]:
            reports.append(f.result())
    amb = sum(r.ambiguous_positions for r in reports)
    flips = sum(len(r.flipped_requests) for r in reports)
    rows = sum(r.total for r in reports)
    print(f"\n[{tag}] steps={len(reports)} packed rows={rows} ambiguous positions={amb} "
          f"length flips={flips} max conf err={max(r.max_conf_err for r in reports):.2e} "
          f"max surv err={max(r.max_surv_err for r in reports):.2e}", flush=True)
    return reports


@pytest.mark.parametrize("name", ["tiny", "batch1", "mid", "budget"])
def test_step_workload(name):
    cfg = CONFIGS[name]
    _run_workload(cfg, range(cfg.steps), name)


@pytest.mark.parametrize("name", ["mixed_threshold", "mixed_budget"])
def test_step_mixed_workload(name):
    cfg = CONFIGS[name]
    _run_workload(cfg, range(cfg.steps), name)


@pytest.mark.parametrize("case", ["gamma1", "all_zero", "all_full", "budget0", "budget_all",
                                  "nan_cut", "odd_vocab", "tiny_vocab", "big_gamma", "max_gamma",
                                  "max_gamma_budget", "stage_path_budget", "stage_path_wide"])
def test_step_edge_cases(case):
    base = CONFIGS["tiny"]
    cfg = {
        "gamma1": base.scaled(gamma=1),
        "all_zero": base.scaled(cutoff=2.0),
        "all_full": base.scaled(cutoff=0.0),
        "budget0": CONFIGS["mixed_budget"].scaled(B=8, d=256, V=1024, budget_per_request=0.0),
        "budget_all": CONFIGS["mixed_budget"].scaled(B=8, d=256, V=1024, budget_per_request=99.0),
        "nan_cut": base.scaled(cutoff=float("nan")),
        "odd_vocab": base.scaled(V=1001, d=250),
        "tiny_vocab": base.scaled(V=3, B=7),
        "big_gamma": base.scaled(gamma=64, B=3, V=4096),
        # the largest drafted block the ABI takes (gamma = 256)
        "max_gamma": base.scaled(gamma=256, B=2, V=512, d=64),
        "max_gamma_budget": CONFIGS["mixed_budget"].scaled(gamma=256, B=12, V=512, d=64),
        # beyond the fused kernels' limits (B*gamma > 8192 in budget mode, B > 4096):
        # dspark_step runs the stage kernels
        "stage_path_budget": CONFIGS["mixed_budget"].scaled(B=600, d=256, V=512),
        "stage_path_wide": base.scaled(B=4200, gamma=2, d=64, V=64),
    }[case]
    _run_workload(cfg, range(3), case)


def test_step_repeat_is_bit_identical():
    cfg = CONFIGS["mixed_budget"].scaled(B=64, V=32768)
    s = make_step(cfg, 0, device=DEV)
    a = _gpu_step(s)
    for _ in range(5):
        b = _gpu_step(s)
        for k in a:
            assert np.array_equal(a[k], b[k]), k


def test_step_leaves_packed_tails_untouched():
    cfg = CONFIGS["tiny"]
    s = make_step(cfg, 1, device=DEV)
    out = dspark.alloc_step_outputs(cfg.B, cfg.gamma, DEV)
    for k in ("packed_tokens", "packed_src_row", "packed_argmax"):
        out[k].fill_(-7)
    g = _gpu_step(s, out=out)
    total = int(g["cu_seqlens"][-1])
    for k in ("packed_tokens", "packed_src_row", "packed_argmax"):
        assert np.all(g[k][total:] == -7)
        assert np.all(g[k][:total] != -7)


def test_accept_malformed_offsets_leave_the_next_call_correct():
    # cu_seqlens out of order and past the capacity: the outputs are
    # unspecified but every access stays in bounds, and the per-request counters
    # the call used return to zero, so a well-formed call on the same workspace
    # right after it matches the oracle.
    B, g, V = 6, 3, 512
    L, tok, bits, cu, ps = _accept_case(B, g, V, seed=77)
    lg = bits_tensor(bits)
    ws = dspark.workspace(B, g, V, DEV)
    bad_cu = torch.tensor([0, 9, 4, 30, 2, 12, 7], dtype=torch.int32, device=DEV)
    bad_src = torch.tensor(np.arange(B * (g + 1)) % (B * (g + 1)), dtype=torch.int32,
                           device=DEV)
    dspark.dspark_accept(lg, bad_src, bad_cu, torch.from_numpy(tok).to(DEV), ws=ws)
    torch.cuda.synchronize()
    total = int(cu[-1])
    pam, acc, bon = dspark.dspark_accept(lg, torch.from_numpy(ps).to(DEV),
                                         torch.from_numpy(cu).to(DEV),
                                         torch.from_numpy(tok).to(DEV), ws=ws)
    torch.cuda.synchronize()
    amax = oracle.argmax_rows(bits.reshape(-1, V), ps[:total])
    o_acc, o_bon = oracle.accept(cu, tok, amax)
    assert np.array_equal(host(pam)[:total], amax)
    assert np.array_equal(host(acc), o_acc) and np.array_equal(host(bon), o_bon)
