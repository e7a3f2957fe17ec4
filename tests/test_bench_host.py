"""bench.py's host logic (CPU): the algorithmic bytes its rates divide by, its
refusal of more than one GPU, and the guard that ties the recorded HBM counters
to the kernel sources they were taken with.

The byte count is checked against the sizes of the arrays a step actually reads
and writes (the generated inputs and the oracle's outputs of the same step),
not against the formula retyped.
"""
import importlib.util
import os
import shutil
import subprocess
import sys

import pytest

from parity_utils import run_oracle
from synth import CONFIGS, make_step

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")

_spec = importlib.util.spec_from_file_location("bench_under_test", BENCH)
bench = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(bench)


def _nbytes(t):
    return t.numel() * t.element_size()


@pytest.mark.parametrize("mode", ["threshold", "budget", "static", "combined"])
def test_step_bytes_are_what_a_step_reads_and_writes(mode):
    cfg = CONFIGS["tiny"].scaled(mode=mode, budget_per_request=2.5)
    s = make_step(cfg, 3)
    o = run_oracle(s)
    total = int(o.cu[-1])
    assert total == int(o.lengths.sum()) + cfg.B
    reads = (_nbytes(s.hidden) + _nbytes(s.w) + _nbytes(s.temps) + _nbytes(s.tokens)
             + total * cfg.V * s.logits.element_size())      # only the packed logit rows
    if mode in ("threshold", "combined"):
        reads += _nbytes(s.cutoff)
    f32 = 4  # conf and survival are written in fp32; every integer output is int32
    writes = ((o.conf.size + o.surv.size) * f32
              + (o.lengths.size + o.cu.size + o.accepted.size + o.bonus.size) * 4
              + (o.ptok[:total].size + o.psrc[:total].size + o.amax[:total].size) * 4)
    assert bench.step_bytes(cfg, total) == reads + writes


@pytest.mark.parametrize("mode", ["threshold", "budget", "static", "combined"])
def test_dominant_kernel_bytes(mode):
    cfg = CONFIGS["mixed_threshold"].scaled(mode=mode, budget_per_request=2.9)
    total = cfg.B + 742
    whole = bench.step_bytes(cfg, total)
    dom = bench.dominant_kernel_bytes(cfg, total)
    if mode in ("threshold", "static"):
        # one launch: the dominant kernel is the whole step
        assert dom == whole
    else:
        # the second launch reads every draft row but no hidden state or root row
        drafts = 2 * cfg.V * (total - cfg.B)
        assert drafts < dom < whole - 2 * cfg.B * cfg.gamma * cfg.d - 2 * cfg.V * cfg.B + 1


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert r.stdout == ""
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr


def test_recorded_traffic_follows_the_sources(tmp_path, monkeypatch):
    src = tmp_path / "csrc"
    shutil.copytree(bench.CSRC, src)
    monkeypatch.setattr(bench, "CSRC", str(src))
    record = tmp_path / "traffic.txt"
    record.write_text("# counters of some build\n"
                      f"source_sha256 = {bench.kernel_source_digest()}\n"
                      "hbm_bytes_per_step = 123\n"
                      "hbm_bytes_dominant_kernel = 45\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(record))
    assert bench.recorded_traffic() == {"step": 123.0, "kernel": 45.0}
    # any change to a kernel source voids the record
    hip = sorted(p for p in src.iterdir() if p.suffix == ".hip")[0]
    hip.write_text(hip.read_text() + "\n// changed\n")
    assert bench.recorded_traffic() is None
    # and so does a missing or malformed record
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.recorded_traffic() is None
    bad = tmp_path / "bad.txt"
    bad.write_text(f"source_sha256 = {bench.kernel_source_digest()}\nhbm_bytes_per_step = x\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(bad))
    assert bench.recorded_traffic() is None
