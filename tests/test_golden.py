"""Stored cases under tests/golden/.

worked_verify_block.json is a verify step of two requests worked out by hand
from the pages' definitions (head, survival, the three cuts, packing, greedy
acceptance, bonus): the oracle must reproduce it (CPU), and so must the HIP
library through the fused step in both forms (batch-wide picks take two
launches in either) and through the stage entry points (GPU).
oracle_small_case.json holds the oracle's outputs for one seeded step, written by tests/golden/make_oracle_case.py; the oracle must
still reproduce it bit for bit, and the HIP library must match it.
"""
import json
import os

import numpy as np
import pytest

import oracle
from synth import rne_bf16

HERE = os.path.dirname(os.path.abspath(__file__))
WORKED = os.path.join(HERE, "golden", "worked_verify_block.json")
STORED = os.path.join(HERE, "golden", "oracle_small_case.json")
INT_KEYS = ("lengths", "cu_seqlens", "packed_tokens", "packed_src_row", "packed_argmax",
            "accepted", "bonus")


def _load(path):
    with open(path) as f:
        return json.load(f)


def _worked_inputs(w):
    B, g, V = w["B"], w["gamma"], w["V"]
    hidden = rne_bf16(np.array(w["hidden"], np.float32))
    wb = rne_bf16(np.array(w["w"], np.float32))
    logits = rne_bf16(np.array(w["logits"], np.float32))
    # the fixture's values are bf16-exact: rounding must not have moved any
    assert np.array_equal((hidden.astype(np.uint32) << 16).view(np.float32),
                          np.array(w["hidden"], np.float32))
    assert np.array_equal(((logits.astype(np.uint32) << 16).view(np.float32)),
                          np.array(w["logits"], np.float32))
    # -0.0 entries keep their sign bit (they test the signed-zero tie)
    assert np.count_nonzero(logits == 0x8000) == 2
    tokens = np.array(w["tokens"], np.int32)
    assert hidden.shape == (B, g, w["d"]) and logits.shape == (B, g + 1, V)
    return hidden, wb, np.array(w["temps"], np.float32), tokens, logits


def _stored_inputs(s):
    B, g, d, V = s["B"], s["gamma"], s["d"], s["V"]
    hidden = np.array(s["hidden_bits"], np.uint16).reshape(B, g, d)
    wb = np.array(s["w_bits"], np.uint16)
    logits = np.array(s["logits_bits"], np.uint16).reshape(B, g + 1, V)
    return hidden, wb, np.array(s["temps"], np.float32), np.array(s["tokens"], np.int32), logits


def _cutoff(doc, case):
    if case["mode"] in ("threshold", "combined"):
        c = case.get("cutoff") or doc["cutoff"]
        return np.array(c, np.float32)
    return None


def _check_ints(got, case):
    total = case["cu_seqlens"][-1]
    for k in INT_KEYS:
        exp = np.array(case[k])
        g = np.asarray(got[k])
        if k.startswith("packed_"):
            g = g[:total]
        assert np.array_equal(g, exp), (case["name"], k, g.tolist(), exp.tolist())


# ------------------------------------------------------------------ CPU pins

def test_worked_block_oracle():
    w = _load(WORKED)
    hidden, wb, temps, tokens, logits = _worked_inputs(w)
    z, conf = oracle.confidence(hidden, wb, w["bias"], temps)
    assert np.allclose(z, np.array(w["worked_head_logits"]["z"]), rtol=0, atol=1e-15)
    assert np.allclose(conf, np.array(w["conf"]), rtol=0, atol=1e-15)
    surv = oracle.survival(conf)
    assert np.allclose(surv, np.array(w["survival"]), rtol=0, atol=1e-15)
    am = oracle.argmax_rows(logits.reshape(-1, w["V"]))
    assert am.tolist() == w["worked_row_argmax"]["argmax"]
    for case in w["cases"]:
        o = oracle.step(hidden, wb, w["bias"], temps, tokens, logits, case["mode"],
                        cutoff=_cutoff(w, case), budget=case["budget"])
        assert np.allclose(o["conf"], np.array(w["conf"]), rtol=0, atol=1e-15)
        assert np.allclose(o["survival"], np.array(w["survival"]), rtol=0, atol=1e-15)
        _check_ints(o, case)


def test_stored_case_oracle():
    s = _load(STORED)
    hidden, wb, temps, tokens, logits = _stored_inputs(s)
    assert len(s["cases"]) == 4
    for case in s["cases"]:
        o = oracle.step(hidden, wb, s["bias"], temps, tokens, logits, case["mode"],
                        cutoff=_cutoff(s, case), budget=case["budget"])
        assert np.array_equal(o["conf"], np.array(case["conf"])), case["name"]
        assert np.array_equal(o["survival"], np.array(case["survival"])), case["name"]
        _check_ints(o, case)


def test_stored_case_is_what_its_script_writes(tmp_path, monkeypatch):
    # the committed script, run again, must write the committed file
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "make_oracle_case", os.path.join(HERE, "golden", "make_oracle_case.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    out = tmp_path / "case.json"
    monkeypatch.setattr(mod, "OUT", str(out))
    mod.main()
    assert _load(str(out)) == _load(STORED)


# ------------------------------------------------------------------ GPU parity

def _gpu_step(doc, inputs, case, launches, monkeypatch):
    import torch

    import confidence_scheduled_ragged_amd as dspark

    hidden, wb, temps, tokens, logits = inputs
    dev = "cuda:0"

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16).copy()).view(
            torch.bfloat16).to(dev)

    c = _cutoff(doc, case)
    out = dspark.dspark_step(bf(hidden), bf(wb), doc["bias"], torch.from_numpy(temps).to(dev),
                             torch.from_numpy(tokens).to(dev), bf(logits), case["mode"],
                             cutoff=None if c is None else torch.from_numpy(c).to(dev),
                             budget=case["budget"], launches=launches)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


@pytest.mark.gpu
@pytest.mark.parametrize("launches", [1, 2])
def test_worked_block_gpu_step(launches, monkeypatch):
    w = _load(WORKED)
    inputs = _worked_inputs(w)
    for case in w["cases"]:
        g = _gpu_step(w, inputs, case, launches, monkeypatch)
        assert np.max(np.abs(g["conf"] - np.array(w["conf"]))) <= 1e-5
        assert np.max(np.abs(g["survival"] - np.array(w["survival"]))) <= 1e-5
        _check_ints(g, case)


@pytest.mark.gpu
def test_worked_block_gpu_stages():
    import torch

    import confidence_scheduled_ragged_amd as dspark

    w = _load(WORKED)
    hidden, wb, temps, tokens, logits = _worked_inputs(w)
    dev = "cuda:0"

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16).copy()).view(
            torch.bfloat16).to(dev)

    conf, surv = dspark.dspark_confidence(bf(hidden), bf(wb), w["bias"],
                                          torch.from_numpy(temps).to(dev))
    tok = torch.from_numpy(tokens).to(dev)
    lg = bf(logits)
    for case in w["cases"]:
        c = _cutoff(w, case)
        L = dspark.dspark_schedule(surv, case["mode"],
                                   cutoff=None if c is None else torch.from_numpy(c).to(dev),
                                   budget=case["budget"])
        cu, ptok, psrc, _ = dspark.dspark_compact(L, tok)
        pam, acc, bon = dspark.dspark_accept(lg.view(-1, w["V"]), psrc, cu, tok)
        torch.cuda.synchronize()
        got = dict(lengths=L, cu_seqlens=cu, packed_tokens=ptok, packed_src_row=psrc,
                   packed_argmax=pam, accepted=acc, bonus=bon)
        _check_ints({k: v.cpu().numpy() for k, v in got.items()}, case)
    torch.cuda.synchronize()
    assert np.max(np.abs(conf.cpu().numpy() - np.array(w["conf"]))) <= 1e-5
    assert np.max(np.abs(surv.cpu().numpy() - np.array(w["survival"]))) <= 1e-5


@pytest.mark.gpu
@pytest.mark.parametrize("launches", [1, 2])
def test_stored_case_gpu_step(launches, monkeypatch):
    s = _load(STORED)
    inputs = _stored_inputs(s)
    for case in s["cases"]:
        g = _gpu_step(s, inputs, case, launches, monkeypatch)
        assert np.max(np.abs(g["conf"] - np.array(case["conf"]))) <= 1e-5
        assert np.max(np.abs(g["survival"] - np.array(case["survival"]))) <= 1e-5
        _check_ints(g, case)
