"""Write ``oracle_small_case.json``: one small seeded verify step and the
oracle's outputs for it under every cut.

The inputs are drawn here with numpy (seeded, no arithmetic of the method);
every expected value comes from ``oracle.step`` and nothing else. The file is
a stored regression case: the CPU tests check that the oracle still
reproduces it, the GPU tests that the HIP library does.

Run from the repository root:  python tests/golden/make_oracle_case.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from synth import rne_bf16  # noqa: E402

OUT = os.path.join(HERE, "oracle_small_case.json")

B, GAMMA, D, V = 5, 6, 40, 64
SEED = 20261202


def draw():
    rng = np.random.default_rng(SEED)
    w = rne_bf16((rng.standard_normal(D) / np.sqrt(D)).astype(np.float32))
    hidden = rne_bf16(rng.standard_normal((B, GAMMA, D)).astype(np.float32) * 1.5)
    temps = (1.0 + 0.05 * np.arange(GAMMA)).astype(np.float32)
    bias = float(np.float32(0.75))
    logits = rng.standard_normal((B, GAMMA + 1, V)).astype(np.float32)
    tokens = rng.integers(0, V, (B, GAMMA + 1)).astype(np.int32)
    # drafts of request b agree with the row maxima for a seeded number of
    # positions: the draft's id is given the row's largest value plus 4
    agree = rng.integers(0, GAMMA + 1, B)
    for b in range(B):
        for i in range(int(agree[b])):
            logits[b, i, tokens[b, i + 1]] = logits[b, i].max() + 4.0
    logits_bits = rne_bf16(logits)
    cutoff = rng.uniform(0.1, 0.5, B).astype(np.float32)
    return dict(w=w, hidden=hidden, temps=temps, bias=bias, logits=logits_bits, tokens=tokens,
                cutoff=cutoff)


CUTS = [
    ("threshold", "threshold", True, 0),
    ("budget_T11", "budget", False, 11),
    ("static", "static", False, 0),
    ("combined_T6", "combined", True, 6),
]


def margin(surv, mode, cutoff, T):
    """Smallest distance of a survival value from the value that decides the
    cut (the request's cutoff, or the T-th largest value for a budget)."""
    s = np.asarray(surv)
    gaps = []
    if mode in ("threshold", "combined"):
        gaps.append(np.min(np.abs(s - np.asarray(cutoff, np.float64)[:, None])))
    if mode in ("budget", "combined"):
        v = s.reshape(-1)
        if mode == "combined":
            v = v[(s >= np.asarray(cutoff, np.float64)[:, None]).reshape(-1)]
        v = np.sort(v)[::-1]
        if 0 < T < v.size:
            gaps.append(v[T - 1] - v[T])
    return min(gaps) if gaps else np.inf


def main():
    x = draw()
    cases = []
    for name, mode, with_cut, T in CUTS:
        o = oracle.step(x["hidden"], x["w"], x["bias"], x["temps"], x["tokens"], x["logits"], mode,
                        cutoff=x["cutoff"] if with_cut else None, budget=T)
        # the stored case must not hinge on a rounding-level difference
        assert margin(o["survival"], mode, x["cutoff"], T) > 1e-4, name
        total = int(o["cu_seqlens"][-1])
        cases.append(dict(
            name=name, mode=mode, budget=T, uses_cutoff=with_cut,
            conf=[[float(v) for v in r] for r in o["conf"]],
            survival=[[float(v) for v in r] for r in o["survival"]],
            lengths=o["lengths"].tolist(), cu_seqlens=o["cu_seqlens"].tolist(),
            packed_tokens=o["packed_tokens"][:total].tolist(),
            packed_src_row=o["packed_src_row"][:total].tolist(),
            packed_argmax=o["packed_argmax"][:total].tolist(),
            accepted=o["accepted"].tolist(), bonus=o["bonus"].tolist()))
    doc = dict(
        about="Stored oracle outputs for one seeded step; written by make_oracle_case.py, "
              "which calls only the oracle. Not a value printed on the pages: a regression "
              "case for the oracle and a stored parity case for the HIP library.",
        B=B, gamma=GAMMA, d=D, V=V, seed=SEED, bias=x["bias"],
        temps=x["temps"].tolist(), cutoff=[float(v) for v in x["cutoff"]],
        w_bits=x["w"].tolist(), hidden_bits=x["hidden"].reshape(-1).tolist(),
        logits_bits=x["logits"].reshape(-1).tolist(), tokens=x["tokens"].tolist(),
        cases=cases)
    with open(OUT, "w") as f:
        json.dump(doc, f, separators=(",", ":"))
        f.write("\n")
    print(f"wrote {OUT}")


if __name__ == "__main__":
    main()
