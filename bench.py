#!/usr/bin/env python3
"""Benchmark of the fused verify step (dspark_step) on one MI355X.

Workload: mixed traffic, B=256 requests, gamma=16 drafted tokens, drafter
hidden d=4096 (bf16), target vocabulary V=151936 (bf16 logits), half the
requests predictable and half prose-like, per-request cutoff c=0.25. The same
seeded inputs are also run under the batch budget T=742 (2.9 per request), and
the budget workload with d=7168, V=129280, T=768 is reported beside it.

A step is one dspark_step call over one batch. R distinct seeded batches
(each with its own 1.3 GB dense logit block) stay resident in HBM and are
cycled, so consecutive steps never re-read cached rows. W warm-up steps run
untimed; then K steps are timed between two device synchronisations, with a
pair of HIP events (on the stream the kernels are launched on) around each
step. One JSON line goes to stdout; progress goes to stderr.

Reported:
  value        packed verify rows per second (sum of cu_seqlens[B] over the
               K steps / elapsed time)
  roofline     the dominant kernel: its algorithmic bytes per launch / its
               mean duration, against the 8 TB/s HBM peak. With a per-request
               cutoff the step is one launch (step_one_kernel), so that kernel
               is the step, and its mean duration is the time between one pair
               of HIP events recorded on the kernels' stream around the same K
               back-to-back launches that the wall clock times, divided by K
               (no event sits between two launches; the figure includes the
               short gap between consecutive launches). The mean of HIP events
               recorded around each single launch is kept as a second field.
  step_roofline the same for the whole step, events around the call
  cpu_baseline the fp64 oracle's whole step on the host (one thread) on a
               bounded sample of the same batches, in the same unit
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_dspark_step_mixed_threshold.txt")
CSRC = os.path.join(ROOT, "confidence_scheduled_ragged_amd", "csrc")


def kernel_source_digest() -> str:
    """sha256 over the HIP sources, to tell whether recorded counters still
    describe the kernels being timed."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".hpp")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per step and per launch of the dominant kernel from the
    committed rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE scaled by the
    copy-kernel factor), or None when there is none or the kernels changed
    since it was taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != kernel_source_digest():
        return None
    try:
        return dict(step=float(kv["hbm_bytes_per_step"]),
                    kernel=float(kv["hbm_bytes_dominant_kernel"]))
    except (KeyError, ValueError):
        return None


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def step_bytes(cfg, total: int) -> int:
    """Algorithmic HBM bytes of one step: every input the method must read once
    and every output it writes, with the logits counted only at packed rows."""
    B, g, d, V = cfg.B, cfg.gamma, cfg.d, cfg.V
    reads = (2 * B * g * d            # hidden states
             + 2 * d + 4 * g          # head weight, temperatures
             + (4 * B if cfg.mode in ("threshold", "combined") else 0)   # cutoffs
             + 4 * B * (g + 1)        # verify-block tokens
             + 2 * V * total)         # packed logit rows
    writes = (8 * B * g               # conf, survival
              + 4 * B + 4 * (B + 1)   # lengths, cu_seqlens
              + 12 * total            # packed tokens, source rows, argmax
              + 8 * B)                # accepted, bonus
    return reads + writes


def dominant_kernel_bytes(cfg, total: int) -> int:
    """Algorithmic HBM bytes of the step's dominant kernel. Threshold and static
    cuts run the step in one launch: all of step_bytes. Budget and combined cuts
    take two, and the second (step_stream_kernel) dominates: the draft rows
    (packed rows other than the roots, which the first launch reads), the
    lengths and verify-block tokens it reads, and every output it writes
    (cu_seqlens, packed tokens / source rows / argmax, accepted, bonus)."""
    if cfg.mode in ("threshold", "static"):
        return step_bytes(cfg, total)
    B, g, V = cfg.B, cfg.gamma, cfg.V
    reads = 2 * V * (total - B) + 4 * B + 4 * B * (g + 1)
    writes = 4 * (B + 1) + 12 * total + 8 * B
    return reads + writes


def step_bytes_a3_a6(cfg, total: int) -> int:
    """Algorithmic HBM bytes of schedule + compact + accept given the survival
    curves: survival and cutoffs in, the packed logit rows, tokens, and every
    integer output."""
    B, g, V = cfg.B, cfg.gamma, cfg.V
    reads = (4 * B * g + (4 * B if cfg.mode in ("threshold", "combined") else 0)
             + 4 * B * (g + 1) + 2 * V * total)
    writes = 4 * B + 4 * (B + 1) + 12 * total + 8 * B
    return reads + writes


def run_arm(cfg, slots, outs, ws, steps, warmup, dspark, torch, kernel_events=False):
    """Time `steps` dspark_step calls cycling over the resident slots: the wall
    time of exactly `steps` calls between two device synchronisations, with
    nothing else on the stream but one HIP event before the first call and one
    after the last (their elapsed time over `steps` is the mean launch period
    on the GPU), then the same `steps` calls again with a HIP event pair around
    each (the per-step times; an event record adds its own gap to the stream,
    so it stays out of the first pass). With kernel_events, the event pass goes
    through dspark_step_ex, which records a second pair of events around the
    dominant kernel. Afterwards the workspace's give-up flag must read 0 (no
    bounded wait gave up)."""
    R = len(slots)
    kev = None

    def launch(i, events=None):
        s = slots[i % R]
        dspark.dspark_step(s.hidden, s.w, s.bias, s.temps, s.tokens, s.logits, cfg.mode,
                           cutoff=s.cutoff, budget=cfg.budget, out=outs[i % R], ws=ws,
                           events=events)

    # warm up by count and by time: after an idle period the clocks need a few
    # milliseconds of load before they settle
    t_w = time.perf_counter()
    i = 0
    while i < warmup or time.perf_counter() - t_w < 0.2:
        launch(i)
        i += 1
        if i % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    totals = [int(o["cu_seqlens"][-1].item()) for o in outs]
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    if kernel_events:
        kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for a, b in kev:                 # create the events before the timed region
            a.record()
            b.record()
    e_first, e_last = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_first.record()
    for i in range(steps):
        launch(i)
    e_last.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    batch_ms = e_first.elapsed_time(e_last) / steps
    for i in range(steps):
        ev[i][0].record()
        launch(i, kev[i] if kev else None)
        ev[i][1].record()
    torch.cuda.synchronize()
    step_ms = [a.elapsed_time(b) for a, b in ev]
    kernel_ms = [a.elapsed_time(b) for a, b in kev] if kev else None
    st = int(dspark.dspark_step_status(ws).item())
    if st != 0:
        raise RuntimeError(f"{cfg.name}: a bounded wait of the fused step gave up "
                           f"(dspark_step_status = {st}); the timed outputs are undefined")
    rows = sum(totals[i % R] for i in range(steps))
    nbytes = sum(step_bytes(cfg, totals[i % R]) for i in range(steps))
    mean_ms = sum(step_ms) / steps
    res = dict(wall_s=wall, rows=rows, bytes=nbytes, mean_step_ms=mean_ms,
               step_ms_sorted=sorted(step_ms), totals=totals, batch_ms=batch_ms)
    if kernel_ms:
        res["kernel_mean_ms"] = sum(kernel_ms) / steps
        res["kernel_bytes"] = sum(dominant_kernel_bytes(cfg, totals[i % R])
                                  for i in range(steps)) / steps
    return res


def run_stage_arm(cfg, slots, outs, ws, steps, dspark, torch):
    """Steps 3-6 through the stage entry points (dspark_schedule ->
    dspark_compact without a logits copy -> dspark_accept on the dense logits
    through packed_src_row), given the survival curves of a prior fused step."""
    R = len(slots)
    surv = [o["survival"].clone() for o in outs]

    def launch(i):
        s, o = slots[i % R], outs[i % R]
        dspark.dspark_schedule(surv[i % R], cfg.mode, cutoff=s.cutoff, budget=cfg.budget,
                               lengths=o["lengths"])
        dspark.dspark_compact(o["lengths"], s.tokens, out=o)
        dspark.dspark_accept(s.logits, o["packed_src_row"], o["cu_seqlens"], s.tokens, out=o, ws=ws)

    for i in range(max(8, R)):
        launch(i)
    torch.cuda.synchronize()
    totals = [int(o["cu_seqlens"][-1].item()) for o in outs]
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        launch(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    mean_ms = sum(ms) / steps
    nbytes = sum(step_bytes_a3_a6(cfg, totals[i % R]) for i in range(steps)) / steps
    return dict(event_ms_per_step=mean_ms, p50_ms=ms[steps // 2], bytes_a3_a6=nbytes,
                achieved_gbs=nbytes / (mean_ms / 1e3) / 1e9,
                frac_of_hbm_peak=nbytes / (mean_ms / 1e3) / 1e9 / HBM_PEAK_GBS)


def run_audit(cfg_t, cfg_b, slots, ws, steps, warmup, dspark, torch):
    """The static and cap-accept verify modes on the same resident batches: the
    static step's time (every row of the block verified), the cap-accept
    kernel's time, and the utilisation of the threshold and budget windows
    against the full verify (sum committed / sum a full verify accepts)."""
    dev = slots[0].hidden.device
    cfg_s = cfg_t.scaled(mode="static")
    outs_s = [dspark.alloc_step_outputs(cfg_s.B, cfg_s.gamma, dev) for _ in slots]
    r_s = run_arm(cfg_s, slots, outs_s, ws, steps, warmup, dspark, torch)
    res = dict(static_full_block=arm_summary(cfg_s, r_s, steps, cfg_s.B))
    tot = {}
    cap_ms = []
    for cfg in (cfg_t, cfg_b):
        acc_sum = full_sum = 0
        for i, s in enumerate(slots):
            o = dspark.dspark_step(s.hidden, s.w, s.bias, s.temps, s.tokens, s.logits, cfg.mode,
                                   cutoff=s.cutoff, budget=cfg.budget, ws=ws)
            sums = torch.zeros(2, dtype=torch.int64, device=dev)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            dspark.dspark_cap_accept(outs_s[i]["packed_argmax"], s.tokens, o["lengths"], sums=sums)
            e1.record()
            torch.cuda.synchronize()
            cap_ms.append(e0.elapsed_time(e1))
            a, f = (int(x) for x in sums.cpu())
            acc_sum += a
            full_sum += f
        tot[cfg.mode] = acc_sum / max(full_sum, 1)
    res["cap_accept_us"] = 1e3 * sorted(cap_ms)[len(cap_ms) // 2]
    # offline STS fit on the audit records: head logits from the logged scores
    # and the temperatures they were taken with, labels from cap-accept
    from confidence_scheduled_ragged_amd.calibrate import (fit_sts_temperatures,
                                                           head_logits_from_scores)
    import numpy as np
    zs, fulls = [], []
    for i, s in enumerate(slots):
        _, _, full, _ = dspark.dspark_cap_accept(outs_s[i]["packed_argmax"], s.tokens,
                                                 outs_s[i]["lengths"])
        zs.append(head_logits_from_scores(outs_s[i]["conf"].cpu().numpy(),
                                          s.temps.cpu().numpy()))
        fulls.append(full.cpu().numpy())
    t0 = time.perf_counter()
    fitted = fit_sts_temperatures(np.concatenate(zs), np.concatenate(fulls))
    res["sts_fit"] = dict(records=int(sum(len(f) for f in fulls)),
                          ms=(time.perf_counter() - t0) * 1e3,
                          temperatures=[round(float(x), 4) for x in fitted],
                          head_temperatures=[round(float(x), 4)
                                             for x in slots[0].temps.cpu().numpy()])
    res["utilization_threshold_window"] = tot["threshold"]
    res["utilization_budget_window"] = tot["budget"]
    return res


def run_combined_cost_table(cfg_c, slots, ws, steps, warmup, dspark, torch):
    """The cutoff from a cost table on the device (load level 3 of a five-entry
    table, 0.25 expected tokens) and the cutoff and budget together (T = 742)
    in one fused step, on the resident mixed batches."""
    dev = slots[0].hidden.device
    table = torch.tensor([0.1, 0.15, 0.2, 0.25, 0.3], dtype=torch.float32, device=dev)
    load = torch.tensor([3], dtype=torch.int32, device=dev)
    cut = torch.empty(cfg_c.B, dtype=torch.float32, device=dev)
    R = len(slots)
    outs = [dspark.alloc_step_outputs(cfg_c.B, cfg_c.gamma, dev) for _ in slots]

    def launch(i):
        s = slots[i % R]
        dspark.dspark_cost_cutoff(table, load, cfg_c.B, cutoff=cut)
        dspark.dspark_step(s.hidden, s.w, s.bias, s.temps, s.tokens, s.logits, "combined",
                           cutoff=cut, budget=cfg_c.budget, out=outs[i % R], ws=ws)

    for i in range(max(warmup, 2 * R)):
        launch(i)
    torch.cuda.synchronize()
    totals = [int(o["cu_seqlens"][-1].item()) for o in outs]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        launch(i)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    nbytes = sum(step_bytes(cfg_c, totals[i % R]) for i in range(steps)) / steps
    return dict(us_per_step=us, mean_packed_rows=sum(totals) / R, budget=cfg_c.budget,
                cutoff=0.25, achieved_gbs=nbytes / (us / 1e6) / 1e9,
                frac_of_hbm_peak=nbytes / (us / 1e6) / 1e9 / HBM_PEAK_GBS)


def run_gather(cfg, outs, steps, dspark, torch, width=7168):
    """The packed activation gather: per-position bf16 activations
    [B*(gamma+1), width] of the target moved to [total, width] through the
    packed source rows of the fused threshold steps. One distinct activation
    tensor per resident batch, so rows are not re-read from the Infinity Cache.
    Bytes: every packed row read once and written once."""
    dev = outs[0]["cu_seqlens"].device
    cap = cfg.B * (cfg.gamma + 1)
    R = len(outs)
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    acts = [torch.randn((cap, width), generator=gen, device=dev).to(torch.bfloat16)
            for _ in range(R)]
    dst = torch.empty((cap, width), dtype=torch.bfloat16, device=dev)
    totals = [int(o["cu_seqlens"][-1].item()) for o in outs]
    for i in range(R):
        dspark.dspark_gather_rows(acts[i], outs[i]["packed_src_row"], outs[i]["cu_seqlens"],
                                  out=dst)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        dspark.dspark_gather_rows(acts[i % R], outs[i % R]["packed_src_row"],
                                  outs[i % R]["cu_seqlens"], out=dst)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    nbytes = sum(2 * totals[i % R] * width * 2 for i in range(steps)) / steps
    del acts, dst
    return dict(width=width, dtype="bf16", us_per_call=us, mean_packed_rows=sum(totals) / R,
                bytes_per_call=nbytes, achieved_gbs=nbytes / (us / 1e6) / 1e9,
                frac_of_hbm_peak=nbytes / (us / 1e6) / 1e9 / HBM_PEAK_GBS)


def run_graph_latency(cfg, steps, dspark, torch, make_step, make_params, R=4, M=8):
    """Latency of the fused step at a small workload, the same kernels and
    buffers launched five ways: K eager dspark_step calls through the checked
    binding; K calls of BoundStep objects (arguments checked and marshalled
    once); K replays of HIP graphs holding one step each, captured once per
    resident batch; and K/M replays of one graph holding M consecutive steps
    (a step's cost as part of a larger captured graph, as in a serving loop
    that captures the whole decode step). The difference between the last two
    is the fixed cost of one graph launch."""
    dev = torch.device("cuda:0")
    p = make_params(cfg)
    slots = [make_step(cfg, i, device=dev, params=p) for i in range(R)]
    outs = [dspark.alloc_step_outputs(cfg.B, cfg.gamma, dev) for _ in slots]
    ws = dspark.workspace(cfg.B, cfg.gamma, cfg.V, dev)

    def body(i):
        s = slots[i]
        dspark.dspark_step(s.hidden, s.w, s.bias, s.temps, s.tokens, s.logits, cfg.mode,
                           cutoff=s.cutoff, budget=s.budget, out=outs[i], ws=ws)

    def timed(fn, n=steps, per=1):
        # wall and event time per step, and the host time to issue the calls
        # (equal to the wall time when the host, not the GPU, sets the pace)
        for i in range(2 * R):
            fn(i % R)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for i in range(n):
            fn(i % R)
        t1 = time.perf_counter()
        e1.record()
        torch.cuda.synchronize()
        issue.append((t1 - t0) * 1e6 / (n * per))
        return ((time.perf_counter() - t0) * 1e6 / (n * per),
                e0.elapsed_time(e1) * 1e3 / (n * per))

    issue = []
    eager_wall, eager_ev = timed(body)
    bound = [dspark.bind_step(s.hidden, s.w, s.bias, s.temps, s.tokens, s.logits, cfg.mode,
                              cutoff=s.cutoff, budget=s.budget, out=outs[i], ws=ws)
             for i, s in enumerate(slots)]
    bound_wall, bound_ev = timed(lambda i: bound[i]())
    totals = [int(o["cu_seqlens"][-1].item()) for o in outs]
    nbytes = sum(step_bytes(cfg, t) for t in totals) / len(totals)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(R):
            body(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for i in range(R):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            body(i)
        graphs.append(g)
    torch.cuda.synchronize()
    graph_wall, graph_ev = timed(lambda i: graphs[i].replay())
    del graphs
    gm = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gm):
        for i in range(M):
            body(i % R)
    torch.cuda.synchronize()
    gm_wall, gm_ev = timed(lambda i: gm.replay(), n=max(1, steps // M), per=M)
    del gm
    best = min(bound_ev, gm_ev)
    return dict(workload=cfg.name, B=cfg.B, eager_us_per_step=eager_wall,
                eager_event_us_per_step=eager_ev, bound_us_per_step=bound_wall,
                bound_event_us_per_step=bound_ev, graph_us_per_step=graph_wall,
                graph_event_us_per_step=graph_ev, steps_per_graph=M,
                graph_multi_us_per_step=gm_wall, graph_multi_event_us_per_step=gm_ev,
                graph_launch_cost_us=graph_ev - gm_ev,
                host_issue_us_per_step=dict(zip(("eager", "bound", "graph", "graph_multi"), issue)),
                mean_packed_rows=sum(totals) / len(totals),
                algorithmic_bytes_per_step=nbytes,
                achieved_gbs=nbytes / (best / 1e6) / 1e9,
                frac_of_hbm_peak=nbytes / (best / 1e6) / 1e9 / HBM_PEAK_GBS)


def stream_read_context(torch, dev):
    """HBM GB/s of a plain device-to-device copy of 1 GiB on the same device,
    for context (bytes read plus bytes written over the copy time)."""
    src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 5 * 2 * src.numel() / (e0.elapsed_time(e1) / 1e3) / 1e9
    del src, dst
    return dict(kernel="device-to-device copy of 1 GiB (read + write bytes)", gbs=gbs,
                frac_of_hbm_peak=gbs / HBM_PEAK_GBS)


def _oracle_worker(args):
    """One host process of the all-core oracle timing: whole oracle steps on the
    shared batches until `seconds` have passed."""
    import numpy as np
    from multiprocessing import shared_memory

    import oracle

    specs, scalars, mode, seconds, wid = args
    shms, arrs = [], []
    for batch in specs:
        a = {}
        for name, (shm_name, shape, dtype) in batch.items():
            shm = shared_memory.SharedMemory(name=shm_name)
            shms.append(shm)
            a[name] = np.ndarray(shape, dtype=dtype, buffer=shm.buf)
        arrs.append(a)
    rows = n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        h, sc = arrs[(n + wid) % len(arrs)], scalars[(n + wid) % len(arrs)]
        o = oracle.step(h["hidden"], h["w"], sc["bias"], h["temps"], h["tokens"], h["logits"],
                        mode, cutoff=h["cutoff"], budget=sc["budget"])
        rows += int(o["cu_seqlens"][-1])
        n += 1
    el = time.perf_counter() - t0
    del arrs
    for shm in shms:
        shm.close()
    return rows, n, el


def cpu_baseline_all_cores(cfg, host, seconds=10.0):
    """The same oracle in one process per host core (at most 16, the host share
    of one GPU), each on the shared batches: aggregate packed rows/s."""
    import multiprocessing as mp
    from multiprocessing import shared_memory

    import numpy as np

    cores = max(1, min(16, os.cpu_count() or 1))
    shms, specs, scalars = [], [], []
    try:
        for h in host:
            spec = {}
            for name in ("hidden", "w", "temps", "tokens", "cutoff", "logits"):
                a = np.ascontiguousarray(h[name])
                shm = shared_memory.SharedMemory(create=True, size=max(1, a.nbytes))
                shms.append(shm)
                np.ndarray(a.shape, dtype=a.dtype, buffer=shm.buf)[...] = a
                spec[name] = (shm.name, a.shape, a.dtype.str)
            specs.append(spec)
            scalars.append(dict(bias=h["bias"], budget=h["budget"]))
        ctx = mp.get_context("spawn")
        t0 = time.perf_counter()
        with ctx.Pool(cores) as pool:
            res = pool.map(_oracle_worker, [(specs, scalars, cfg.mode, seconds, i)
                                            for i in range(cores)])
        wall = time.perf_counter() - t0
    finally:
        for shm in shms:
            shm.close()
            shm.unlink()
    rows = sum(r[0] for r in res)
    steps = sum(r[1] for r in res)
    busy = max(r[2] for r in res)
    return dict(value=rows / busy, unit="packed verify rows/s", cores=cores, kind="oracle",
                sample=f"{cores} host processes x {seconds:.0f} s of whole oracle steps on the "
                       f"same {len(host)} batches: {steps} steps, {rows} packed rows "
                       f"(wall {wall:.1f} s including process start)")


def arm_summary(cfg, r, steps, B):
    """Per-arm figures. The HBM rate divides the algorithmic bytes by the mean
    launch period between one event pair around the K back-to-back steps
    (`us_per_step`, no event between steps); the per-step event times of the
    second pass (each record adds its own gap) give the distribution."""
    batch_s = r["batch_ms"] * steps / 1e3
    return dict(
        rows_per_s=r["rows"] / r["wall_s"],
        request_steps_per_s=B * steps / r["wall_s"],
        ms_per_step=r["wall_s"] * 1e3 / steps,
        us_per_step=r["batch_ms"] * 1e3,
        event_ms_per_step=r["mean_step_ms"],
        p10_ms=r["step_ms_sorted"][len(r["step_ms_sorted"]) // 10],
        p50_ms=r["step_ms_sorted"][len(r["step_ms_sorted"]) // 2],
        p90_ms=r["step_ms_sorted"][(9 * len(r["step_ms_sorted"])) // 10],
        mean_packed_rows=r["rows"] / steps,
        achieved_gbs=r["bytes"] / batch_s / 1e9,
        frac_of_hbm_peak=r["bytes"] / batch_s / 1e9 / HBM_PEAK_GBS,
    )


def cpu_baseline(cfg, slots, min_s=10.0, max_s=30.0):
    """The oracle's whole step, single-threaded, on the first batches of the
    rotation until at least `min_s` seconds of CPU work (capped at `max_s`)."""
    import numpy as np

    import oracle

    host = []
    for s in slots[:2]:
        host.append(dict(hidden=s.host("hidden"), w=s.host("w"), temps=s.host("temps"),
                         tokens=s.host("tokens"), cutoff=s.host("cutoff"),
                         logits=s.host("logits"), bias=s.bias, budget=s.budget))
    rows = 0
    n = 0
    results = []
    t0 = time.perf_counter()
    while True:
        h = host[n % len(host)]
        o = oracle.step(h["hidden"], h["w"], h["bias"], h["temps"], h["tokens"], h["logits"],
                        cfg.mode, cutoff=h["cutoff"], budget=h["budget"])
        if n < len(host):
            results.append(o)
        rows += int(o["cu_seqlens"][-1])
        n += 1
        el = time.perf_counter() - t0
        if el >= min_s or el >= max_s:
            break
    for s in slots[:2]:
        s._host.pop("logits", None)
    del np
    return dict(value=rows / el, unit="packed verify rows/s", cores=1, kind="oracle",
                sample=f"{n} whole steps (batches 0-{len(host) - 1} of the rotation, "
                       f"{rows} packed rows) of the same workload in {el:.1f} s",
                seconds=el), results, host


def check_against_oracle(results, outs, host):
    """Outputs of the GPU's own runs of the sampled batches against the oracle's
    results on those batches: conf/survival within 1e-5 of fp64; the integer
    outputs exact. A position whose fp64 survival lies within 1e-5 of its
    request's cutoff is ambiguous (fp32 and fp64 may fall on either side):
    such positions are counted, and lengths that differ only on requests
    holding one make the verdict "ambiguous" (the packing, acceptance and bonus
    of every other request must still match). Returns (verdict, count)."""
    import numpy as np

    verdict = True
    n_amb = 0
    for o, g, h in zip(results, outs, host):
        gg = {k: v.cpu().numpy() for k, v in g.items()}
        ok = bool(np.max(np.abs(gg["conf"] - o["conf"])) <= 1e-5)
        ok &= bool(np.max(np.abs(gg["survival"] - o["survival"])) <= 1e-5)
        amb = np.abs(o["survival"] - h["cutoff"].astype(np.float64)[:, None]) <= 1e-5
        n_amb += int(amb.sum())
        flips = np.nonzero(gg["lengths"] != o["lengths"])[0]
        if flips.size == 0:
            total = int(o["cu_seqlens"][-1])
            for k in ("cu_seqlens", "accepted", "bonus"):
                ok &= bool(np.array_equal(gg[k], o[k]))
            for k in ("packed_tokens", "packed_src_row", "packed_argmax"):
                ok &= bool(np.array_equal(gg[k][:total], o[k][:total]))
        else:
            ok &= bool(np.all(amb[flips].any(axis=1)))
            for b in range(len(gg["lengths"])):
                if b in flips:
                    continue
                n = int(o["lengths"][b]) + 1
                gs, os_ = int(gg["cu_seqlens"][b]), int(o["cu_seqlens"][b])
                for k in ("packed_tokens", "packed_argmax"):
                    ok &= bool(np.array_equal(gg[k][gs:gs + n], o[k][os_:os_ + n]))
                ok &= bool(gg["accepted"][b] == o["accepted"][b])
                ok &= bool(gg["bonus"][b] == o["bonus"][b])
            if ok and verdict is True:
                verdict = "ambiguous"
        if not ok:
            verdict = False
    return verdict, n_amb


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotation", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra-arms", action="store_true")
    ap.add_argument("--profile-budget", nargs="?", const="budget", default=None,
                    choices=["budget", "mixed_budget", "mixed_combined"],
                    help="time only one batch-wide-pick workload (default: the budget workload, "
                         "d=7168 V=129280 T=768; or the mixed workload's budget or combined "
                         "arm), for a kernel trace of it; prints its arm summary instead of the "
                         "JSON line")
    ap.add_argument("--latency-only", action="store_true",
                    help="time only the batch-1 and mid latency arm (eager, bound, one step per "
                         "graph, several steps per graph), for a kernel trace of it; prints the "
                         "arm's records instead of the JSON line")
    ap.add_argument("--no-all-cores", action="store_true",
                    help="skip the oracle timing on all host cores")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 1 GiB device-to-device copy (a plain copy kernel of known "
                         "size) so counter runs can scale FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the verify hot path runs on a single MI355X here "
              f"and --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch

    import confidence_scheduled_ragged_amd as dspark
    from synth import CONFIGS, make_params, make_step

    dev = torch.device("cuda:0")
    dspark.lib()
    if args.profile_budget:
        cfg4 = CONFIGS[args.profile_budget]
        p4 = make_params(cfg4)
        slots4 = [make_step(cfg4, i, device=dev, params=p4) for i in range(args.rotation)]
        outs4 = [dspark.alloc_step_outputs(cfg4.B, cfg4.gamma, dev) for _ in slots4]
        ws4 = dspark.workspace(cfg4.B, cfg4.gamma, cfg4.V, dev)
        r_4 = run_arm(cfg4, slots4, outs4, ws4, args.steps, args.warmup, dspark, torch)
        print(json.dumps(arm_summary(cfg4, r_4, args.steps, cfg4.B)), flush=True)
        return
    if args.latency_only:
        lat = [run_graph_latency(CONFIGS[n], args.steps, dspark, torch, make_step, make_params)
               for n in ("batch1", "mid")]
        print(json.dumps(lat), flush=True)
        return
    cfg_t = CONFIGS["mixed_threshold"]
    cfg_b = CONFIGS["mixed_budget"]
    params = make_params(cfg_t)
    log(f"generating {args.rotation} resident batches of B={cfg_t.B} gamma={cfg_t.gamma} "
        f"d={cfg_t.d} V={cfg_t.V}")
    slots = []
    for i in range(args.rotation):
        slots.append(make_step(cfg_t, i, device=dev, params=params))
    torch.cuda.synchronize()
    log("batches resident")
    ws = dspark.workspace(cfg_t.B, cfg_t.gamma, cfg_t.V, dev)
    outs = [dspark.alloc_step_outputs(cfg_t.B, cfg_t.gamma, dev) for _ in slots]

    # the headline pass: wall time and one event pair around the K launches; its
    # event pass also records HIP events around each launch of the dominant
    # kernel (a second field: the event records add a few us to each step)
    r_t = run_arm(cfg_t, slots, outs, ws, args.steps, args.warmup, dspark, torch,
                  kernel_events=True)
    r_k = r_t
    s_t = arm_summary(cfg_t, r_t, args.steps, cfg_t.B)
    log(f"threshold arm: {s_t['rows_per_s']:.3e} rows/s, {s_t['us_per_step']:.1f} us/step, "
        f"{s_t['achieved_gbs']:.0f} GB/s ({100 * s_t['frac_of_hbm_peak']:.1f} % of peak)")

    extra = {}
    context = None
    if not args.no_extra_arms:
        st = run_stage_arm(cfg_t, slots, outs, ws, args.steps, dspark, torch)
        extra["stages_a3_a6_threshold"] = st
        log(f"stage path a3-a6: {st['event_ms_per_step'] * 1e3:.1f} us/step, "
            f"{st['achieved_gbs']:.0f} GB/s")
        ga = run_gather(cfg_t, outs, args.steps, dspark, torch)
        extra["packed_activation_gather_7168"] = ga
        log(f"packed activation gather (7168 bf16): {ga['us_per_call']:.1f} us, "
            f"{ga['achieved_gbs']:.0f} GB/s")
        # budget arm on the same resident batches (the two arms share their seeds)
        r_b = run_arm(cfg_b, slots, outs, ws, args.steps, args.warmup, dspark, torch)
        extra["mixed_budget_T742"] = arm_summary(cfg_b, r_b, args.steps, cfg_b.B)
        log(f"budget arm: {extra['mixed_budget_T742']['rows_per_s']:.3e} rows/s")
        cc = run_combined_cost_table(CONFIGS["mixed_combined"], slots, ws, args.steps,
                                     args.warmup, dspark, torch)
        extra["combined_cost_table"] = cc
        log(f"cost table + combined cut: {cc['us_per_step']:.1f} us/step, "
            f"{cc['mean_packed_rows']:.0f} rows")
        audit = run_audit(cfg_t, cfg_b, slots, ws, args.steps, args.warmup, dspark, torch)
        extra["audit_static_cap_accept"] = audit
        log(f"audit: static {audit['static_full_block']['event_ms_per_step'] * 1e3:.1f} us/step, "
            f"utilisation thr {audit['utilization_threshold_window']:.3f} "
            f"bud {audit['utilization_budget_window']:.3f}")
        cfg4 = CONFIGS["budget"]
        p4 = make_params(cfg4)
        slots4 = [make_step(cfg4, i, device=dev, params=p4) for i in range(args.rotation)]
        outs4 = [dspark.alloc_step_outputs(cfg4.B, cfg4.gamma, dev) for _ in slots4]
        ws4 = dspark.workspace(cfg4.B, cfg4.gamma, cfg4.V, dev)
        r_4 = run_arm(cfg4, slots4, outs4, ws4, args.steps, args.warmup, dspark, torch)
        extra["budget_d7168_V129280_T768"] = arm_summary(cfg4, r_4, args.steps, cfg4.B)
        log(f"budget d=7168 arm: {extra['budget_d7168_V129280_T768']['rows_per_s']:.3e} rows/s")
        del slots4, outs4
        lat = [run_graph_latency(CONFIGS[n], args.steps, dspark, torch, make_step, make_params)
               for n in ("batch1", "mid")]
        extra["graph_replay_latency"] = lat
        for x in lat:
            log(f"graph replay, {x['workload']}: eager {x['eager_us_per_step']:.1f} us/step, "
                f"bound {x['bound_us_per_step']:.1f}, graph {x['graph_us_per_step']:.1f}, "
                f"{x['steps_per_graph']} steps per graph {x['graph_multi_us_per_step']:.1f} "
                f"(one graph launch {x['graph_launch_cost_us']:.1f} us); host issue per step "
                + ", ".join(f"{k} {v:.1f}" for k, v in x["host_issue_us_per_step"].items()))
        context = stream_read_context(torch, dev)
        log(f"plain device copy: {context['gbs']:.0f} GB/s")

    cpu = None
    cpu_all = None
    parity = None
    n_amb = None
    if not args.no_cpu_baseline:
        log("timing the oracle on the host (bounded sample)")
        cpu, results, host = cpu_baseline(cfg_t, slots)
        # the GPU outputs of the first timed batches: rerun them once more to be sure the
        # buffers hold exactly those batches' results
        for i in range(len(results)):
            s = slots[i]
            dspark.dspark_step(s.hidden, s.w, s.bias, s.temps, s.tokens, s.logits, cfg_t.mode,
                               cutoff=s.cutoff, budget=s.budget, out=outs[i], ws=ws)
        torch.cuda.synchronize()
        parity, n_amb = check_against_oracle(results, outs[: len(results)], host)
        cpu.pop("seconds", None)
        log(f"oracle: {cpu['value']:.1f} rows/s on 1 core; parity on sampled batches: {parity} "
            f"({n_amb} ambiguous positions)")
        if not args.no_all_cores:
            log("timing the oracle on all host cores (bounded sample)")
            cpu_all = cpu_baseline_all_cores(cfg_t, host)
            log(f"oracle: {cpu_all['value']:.1f} rows/s on {cpu_all['cores']} cores")
        del host

    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 3 x 1 GiB device-to-device copies done")
        del src, dst

    mean_bytes = r_t["bytes"] / args.steps
    k_gbs = r_k["kernel_bytes"] / (r_t["batch_ms"] / 1e3) / 1e9
    k_gbs_bracket = r_k["kernel_bytes"] / (r_k["kernel_mean_ms"] / 1e3) / 1e9
    traffic = recorded_traffic()
    line = {
        "metric": "packed verify rows/s + achieved HBM GB/s (frac of peak), B=256 gamma=16 V=151936",
        "value": s_t["rows_per_s"],
        "unit": "packed verify rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": s_t["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "mixed traffic: B=256 gamma=16 d=4096 V=151936, half predictable "
                               "half prose-like, per-request cutoff c=0.25, fused dspark_step",
                   "B": cfg_t.B, "gamma": cfg_t.gamma, "d": cfg_t.d, "V": cfg_t.V,
                   "mode": "threshold", "rotation": args.rotation,
                   "mean_packed_rows": s_t["mean_packed_rows"]},
        "request_steps_per_s": s_t["request_steps_per_s"],
        "achieved_gbs": s_t["achieved_gbs"],
        "step_us": {"mean": r_t["mean_step_ms"] * 1e3,
                    "p10": s_t["p10_ms"] * 1e3, "p50": s_t["p50_ms"] * 1e3,
                    "p90": s_t["p90_ms"] * 1e3},
        "roofline": {"bound": "hbm",
                     "kernel": "step_one_kernel (the whole step in one launch: confidence "
                               "GEMV, survival, cut, compaction outputs, root and draft-row "
                               "argmax, acceptance, bonus)",
                     "achieved": k_gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": k_gbs / HBM_PEAK_GBS,
                     "traffic": traffic["kernel"] if traffic else None,
                     "traffic_over_algorithmic": (traffic["kernel"] / r_k["kernel_bytes"]
                                                  if traffic else None),
                     "algorithmic_bytes_per_launch": r_k["kernel_bytes"],
                     "mean_launch_us": r_t["batch_ms"] * 1e3,
                     "timing": "one HIP event pair on the kernels' stream around the K "
                               "back-to-back launches of the wall-clock pass, elapsed / K "
                               "(includes the gap between consecutive launches)",
                     "event_bracket_us": r_k["kernel_mean_ms"] * 1e3,
                     "event_bracket_frac": k_gbs_bracket / HBM_PEAK_GBS,
                     "event_bracket_timing": "HIP events recorded right before and after "
                                             "each launch (dspark_step_ex) in a second pass; "
                                             "each record adds its own gap"},
        "step_roofline": {"bound": "hbm",
                          "kernel": "the whole dspark_step (one launch), HIP events around "
                                    "each call in the second pass",
                          "achieved": mean_bytes / (r_t["mean_step_ms"] / 1e3) / 1e9,
                          "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": mean_bytes / (r_t["mean_step_ms"] / 1e3) / 1e9 / HBM_PEAK_GBS,
                          "traffic": traffic["step"] if traffic else None,
                          "traffic_over_algorithmic": (traffic["step"] / mean_bytes
                                                       if traffic else None),
                          "algorithmic_bytes_per_launch": mean_bytes,
                          "mean_launch_us": r_t["mean_step_ms"] * 1e3},
        "cpu_baseline": cpu,
        "cpu_baseline_all_cores": cpu_all,
        "stream_read_context": context,
        "parity_on_sampled_batches": parity,
        "ambiguous_positions_sampled": n_amb,
        "arms": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
