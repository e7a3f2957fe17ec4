"""The oracle's pins catch plausible mistakes: each case plants one mistake in
a copy of the oracle's C source (on the CPU, in a temporary directory),
builds it, points the oracle at it and runs the pins that should catch it.
Every planted mistake must make at least one of those pins fail. The verify
block worked by hand under tests/golden/ must also catch, on its own, every
planted mistake in the parts it exercises (head, survival, cuts without exact
ties, packing, argmax ties, acceptance, bonus). The real oracle is untouched
and reloaded afterwards."""
import os
import subprocess

import pytest

import oracle
import test_golden as golden
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "dspark_oracle.c")

# (name, original text, mistaken text, pins expected to catch it)
MUTATIONS = [
    ("temperature_on_dot_only",
     "double p = 1.0 / (1.0 + exp(-z / (double)temps[i]));",
     "double p = 1.0 / (1.0 + exp(-(dot / (double)temps[i] + (double)bias)));",
     ["test_confidence_zero_weight_closed_form"]),
    ("sign_flip_in_sigmoid",
     "double p = 1.0 / (1.0 + exp(-z / (double)temps[i]));",
     "double p = 1.0 / (1.0 + exp(z / (double)temps[i]));",
     ["test_confidence_zero_weight_closed_form", "test_confidence_symmetry"]),
    ("wrong_hidden_stride",
     "const uint16_t *h = hidden + ((size_t)b * gamma + i) * (size_t)d;",
     "const uint16_t *h = hidden + ((size_t)i * B + b) * (size_t)d;",
     ["test_confidence_one_hot_picks_the_right_entry"]),
    ("survival_shifted_by_one",
     "            s = s * p;\n            surv[(size_t)b * gamma + (k - 1)] = s;",
     "            surv[(size_t)b * gamma + (k - 1)] = s;\n            s = s * p;",
     ["test_survival_constant_closed_form"]),
    ("threshold_strict",
     "            if (s >= c)\n",
     "            if (s > c)\n",
     ["test_threshold_special_cases", "test_threshold_constant_closed_form"]),
    ("budget_ties_to_higher_request",
     "    if (a->flat < b->flat) return -1;\n    if (a->flat > b->flat) return 1;",
     "    if (a->flat < b->flat) return 1;\n    if (a->flat > b->flat) return -1;",
     ["test_budget_all_equal_ties_go_to_lower_requests"]),
    ("budget_ascending",
     "    if (a->s > b->s) return -1;\n    if (a->s < b->s) return 1;",
     "    if (a->s > b->s) return 1;\n    if (a->s < b->s) return -1;",
     ["test_budget_hand_examples"]),
    ("compact_drops_root_row",
     "        cu += (int64_t)L + 1;",
     "        cu += (int64_t)L;",
     ["test_compact_against_library_scan"]),
    ("argmax_last_of_ties",
     "            if (x > best) {",
     "            if (x >= best) {",
     ["test_argmax_matches_library_first_occurrence"]),
    ("accept_without_cap",
     "        while (a < L && amax[start + a] == tokens[(size_t)b * (gamma + 1) + a + 1])",
     "        while (a < gamma && amax[start + a] == tokens[(size_t)b * (gamma + 1) + a + 1])",
     ["test_accept_known_planted_prefix"]),
    ("bonus_from_next_row",
     "        bonus[b] = amax[start + a];",
     "        bonus[b] = amax[start + a + (a < L ? 1 : 0)];",
     ["test_accept_known_planted_prefix"]),
    ("cap_accept_commits_full",
     "        int32_t a = a_full < L ? a_full : L;",
     "        int32_t a = a_full;",
     ["test_cap_accept_known_planted_prefix"]),
    ("combined_ignores_cutoff",
     "        if (s >= (double)cutoff[f / gamma]) {",
     "        if (s >= 0.0) {",
     ["test_combined_brute_force", "test_combined_reduces_to_its_parts"]),
    ("gather_off_by_one_row",
     "            dst[r * row_bytes + k] = src[s * row_bytes + k];",
     "            dst[r * row_bytes + k] = src[(s + (s + 1 < cap ? 1 : 0)) * row_bytes + k];",
     ["test_gather_rows_against_fancy_indexing"]),
    ("tier_rounds_down",
     "    while (t < ntiers && tiers[t] < total)",
     "    while (t < ntiers && tiers[t] <= total)",
     ["test_tier_select_hand_examples"]),
]


# planted mistakes the hand-worked verify block alone must catch
WORKED_CATCHES = ["temperature_on_dot_only", "sign_flip_in_sigmoid", "wrong_hidden_stride",
                  "survival_shifted_by_one", "budget_ascending", "compact_drops_root_row",
                  "argmax_last_of_ties", "accept_without_cap", "bonus_from_next_row"]


def _pin_callables(names):
    out = []
    for n in names:
        f = getattr(pins, n)
        marks = getattr(f, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if params:
            argname, values = params[0].args[0], params[0].args[1]
            for v in values:
                if "," in argname:
                    out.append((f, dict(zip([a.strip() for a in argname.split(",")], v))))
                else:
                    out.append((f, {argname: v}))
        else:
            out.append((f, {}))
    return out


@pytest.fixture
def restore_oracle():
    lib_path = oracle.LIB
    yield
    oracle._lib = None
    oracle.LIB = lib_path


def _load_mutant(name, orig, bad, tmp_path):
    src = open(SRC).read()
    assert src.count(orig) == 1, f"mutation anchor for {name} not unique in the oracle"
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(src.replace(orig, bad))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                    "-fno-fast-math", "-o", str(lib), str(mutated), "-lm"], check=True)
    oracle._lib = None
    oracle.LIB = str(lib)


@pytest.mark.parametrize("name,orig,bad,catchers", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(name, orig, bad, catchers, tmp_path, restore_oracle):
    _load_mutant(name, orig, bad, tmp_path)
    caught = []
    for f, kw in _pin_callables(catchers):
        try:
            f(**kw)
        except (AssertionError, oracle.OracleError) as e:
            caught.append((f.__name__, type(e).__name__))
    assert caught, f"no pin caught the planted mistake {name}"


@pytest.mark.parametrize("name", WORKED_CATCHES)
def test_worked_block_catches_planted_mistake(name, tmp_path, restore_oracle):
    orig, bad = next((m[1], m[2]) for m in MUTATIONS if m[0] == name)
    _load_mutant(name, orig, bad, tmp_path)
    with pytest.raises((AssertionError, oracle.OracleError)):
        golden.test_worked_block_oracle()
