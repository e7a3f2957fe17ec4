"""Pins of the fp64 oracle against facts fixed by mathematics, not by itself.

The pages print no worked numbers, so every pin is a closed form, a hand
derivation, a brute-force enumeration, an independent library routine or an
invariant that the definitions imply. Each block names the mistake it would
catch.
"""
import itertools
import math

import numpy as np
import pytest

import oracle
from synth import bf16_bits_to_f32, rne_bf16


def bf(x):
    return rne_bf16(np.asarray(x, dtype=np.float32))


def exact_bf(x):
    b = bf(x)
    assert np.array_equal(bf16_bits_to_f32(b), np.asarray(x, np.float32)), "value not bf16-exact"
    return b


# ----------------------------------------------------------------- confidence

def test_confidence_zero_weight_closed_form():
    # w = 0 gives z = bias and p_i = sigma(bias / T_i). With bias = ln 9 and
    # T = (1, 2, 4): sigma(ln x) = x / (1 + x) gives 9/10, 3/4, sqrt3/(1+sqrt3).
    # Catches: temperature applied to w.h only (bias undivided), sign flip,
    # dropped bias.
    g, d = 3, 5
    bias = np.float32(math.log(9.0))
    h = bf(np.random.default_rng(1).standard_normal((2, g, d)))
    w = exact_bf(np.zeros(d))
    temps = np.array([1.0, 2.0, 4.0], np.float32)
    z, p = oracle.confidence(h, w, bias, temps)
    xb = math.exp(float(bias))                     # 9 up to the fp32 rounding of ln 9
    want = [xb / (1 + xb), math.sqrt(xb) / (1 + math.sqrt(xb)), xb ** 0.25 / (1 + xb ** 0.25)]
    for b in range(2):
        assert np.allclose(p[b], want, rtol=0, atol=1e-14)
        assert np.all(z[b] == float(bias))
    assert abs(want[0] - 0.9) < 1e-7 and abs(want[1] - 0.75) < 1e-7


def test_confidence_one_hot_picks_the_right_entry():
    # h[b,i,:] = 2 * e_{k(b,i)} with distinct k per (b, i): z must equal
    # 2 * w[k(b,i)] + bias exactly. Catches transposed or mis-strided hidden
    # indexing and reading the wrong weight entry.
    B, g, d = 3, 4, 16
    rng = np.random.default_rng(2)
    w_val = bf16_bits_to_f32(bf(rng.standard_normal(d)))
    w = exact_bf(w_val)
    hv = np.zeros((B, g, d), np.float32)
    assert B * g <= d
    for idx, (b, i) in enumerate(itertools.product(range(B), range(g))):
        hv[b, i, (idx * 5) % d] = 2.0             # 5 is coprime to 16: distinct entries
    h = exact_bf(hv)
    bias = np.float32(-0.25)
    temps = (1 + 0.5 * np.arange(g)).astype(np.float32)
    z, p = oracle.confidence(h, w, bias, temps)
    for b in range(B):
        for i in range(g):
            k = int(np.nonzero(hv[b, i])[0][0])
            assert z[b, i] == 2.0 * float(w_val[k]) + float(bias)
            # logit (inverse sigmoid) of p, times T_i, recovers z
            assert abs(math.log(p[b, i] / (1 - p[b, i])) * temps[i] - z[b, i]) < 1e-12


def test_confidence_matches_library_dot():
    # numpy's float64 matmul is an independent dot product.
    rng = np.random.default_rng(3)
    B, g, d = 5, 7, 333
    h = bf(rng.standard_normal((B, g, d)))
    w = bf(rng.standard_normal(d) / math.sqrt(d))
    bias = np.float32(0.125)
    temps = (1 + 0.05 * np.arange(g)).astype(np.float32)
    z, p = oracle.confidence(h, w, bias, temps)
    zl = bf16_bits_to_f32(h).astype(np.float64) @ bf16_bits_to_f32(w).astype(np.float64) + 0.125
    assert np.allclose(z, zl, rtol=0, atol=1e-12)
    # log-odds identity, independent of how p was formed
    assert np.allclose(np.log(p / (1 - p)) * temps[None, :], zl, rtol=0, atol=1e-9)


def test_confidence_symmetry():
    # With bias 0, negating h negates z, so p(h) + p(-h) = 1.
    rng = np.random.default_rng(4)
    hv = bf16_bits_to_f32(bf(rng.standard_normal((2, 6, 64))))
    w = bf(rng.standard_normal(64) / 8)
    temps = (1 + 0.1 * np.arange(6)).astype(np.float32)
    _, p1 = oracle.confidence(exact_bf(hv), w, 0.0, temps)
    _, p2 = oracle.confidence(exact_bf(-hv), w, 0.0, temps)
    assert np.allclose(p1 + p2, 1.0, rtol=0, atol=1e-15)


def test_confidence_rejects_bad_temperature():
    h = bf(np.ones((1, 2, 4)))
    w = bf(np.ones(4))
    with pytest.raises(oracle.OracleError):
        oracle.confidence(h, w, 0.0, np.array([1.0, 0.0], np.float32))


# ------------------------------------------------------------------- survival

def test_survival_constant_closed_form():
    # constant p = 1/2 gives S_k = 2^-k exactly; catches an S_0 = 1 shift
    # (which would give 2^-(k-1)).
    s = oracle.survival(np.full((3, 10), 0.5))
    assert np.array_equal(s, np.broadcast_to(0.5 ** np.arange(1, 11), (3, 10)))


def test_survival_hand_example():
    # p = (0.5, 0.25, 1, 0.8): S = (0.5, 0.125, 0.125, 0.1), by hand.
    s = oracle.survival(np.array([[0.5, 0.25, 1.0, 0.8]]))
    assert np.allclose(s, [[0.5, 0.125, 0.125, 0.1]], rtol=0, atol=1e-16)


def test_survival_invariants_and_log_identity():
    rng = np.random.default_rng(5)
    p = rng.uniform(0, 1, (20, 16))
    s = oracle.survival(p)
    assert np.all(np.diff(s, axis=1) <= 0) and np.all(s >= 0) and np.all(s <= 1)
    assert np.allclose(np.log(s), np.cumsum(np.log(p), axis=1), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- threshold

def test_threshold_constant_closed_form():
    # S_k = p^k: L = max{k <= gamma : p^k >= c} = min(gamma, floor(ln c / ln p)),
    # with (p, c) chosen away from the boundary.
    g = 16
    for p, c in [(0.9, 0.5), (0.5, 0.3), (0.99, 0.01), (0.7, 0.69), (0.2, 0.3)]:
        s = oracle.survival(np.full((1, g), p))
        L = oracle.cut_threshold(s, np.array([c], np.float32))
        want = min(g, math.floor(math.log(float(np.float32(c))) / math.log(p)))
        assert L[0] == want, (p, c, L[0], want)


def test_threshold_special_cases():
    s = oracle.survival(np.array([[0.5, 0.5, 0.5]]))    # S = 0.5, 0.25, 0.125
    cut = lambda c: int(oracle.cut_threshold(s, np.array([c], np.float32))[0])
    assert cut(0.0) == 3 and cut(-1.0) == 3             # c <= 0 keeps everything
    assert cut(1.5) == 0                                 # c > 1 keeps nothing
    assert cut(float("nan")) == 0                        # NaN keeps nothing
    assert cut(0.25) == 2                                # a tie is kept (>=)
    assert cut(0.2500001) == 1


def test_threshold_is_prefix_count():
    rng = np.random.default_rng(6)
    s = oracle.survival(rng.uniform(0.3, 1, (50, 16)))
    c = rng.uniform(0, 1, 50).astype(np.float32)
    L = oracle.cut_threshold(s, c)
    for b in range(50):
        keep = s[b] >= float(c[b])
        assert L[b] == keep.sum()
        assert np.all(keep[: L[b]]) and not np.any(keep[L[b]:])


# ------------------------------------------------------------------- budget

def _brute_force_budget(s, T):
    B, g = s.shape
    t_eff = min(T, B * g)
    best, arg, nbest = -1.0, None, 0
    for L in itertools.product(range(g + 1), repeat=B):
        if sum(L) != t_eff:
            continue
        val = sum(s[b, :L[b]].sum() for b in range(B))
        if val > best + 1e-12:
            best, arg, nbest = val, L, 1
        elif abs(val - best) <= 1e-12:
            nbest += 1
    return best, arg, nbest


@pytest.mark.parametrize("seed", range(12))
def test_budget_brute_force(seed):
    # The top-T pick maximises the expected verified-and-surviving mass
    # sum_b sum_{k<=L_b} S_k over all length vectors of total T (S is
    # non-increasing, so prefix sums are concave). Enumerate every vector.
    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(1, 5))
    g = int(rng.integers(1, 9 if B <= 3 else 7))
    s = oracle.survival(rng.uniform(0.2, 1.0, (B, g)))
    for T in sorted({0, 1, int(rng.integers(0, B * g + 1)), B * g // 2, B * g, B * g + 3}):
        L = oracle.cut_budget(s, T)
        best, arg, nbest = _brute_force_budget(s, T)
        got = sum(s[b, :L[b]].sum() for b in range(B))
        assert abs(got - best) <= 1e-12
        assert L.sum() == min(T, B * g)
        if nbest == 1:
            assert tuple(L) == arg


def test_budget_all_equal_ties_go_to_lower_requests():
    s = np.full((3, 4), 0.5)
    assert list(oracle.cut_budget(s, 6)) == [4, 2, 0]
    assert list(oracle.cut_budget(s, 0)) == [0, 0, 0]
    assert list(oracle.cut_budget(s, 12)) == [4, 4, 4]
    assert list(oracle.cut_budget(s, 99)) == [4, 4, 4]


def test_budget_hand_examples():
    # S rows (0.9, 0.5) and (0.9, 0.6): ranking (0.9,b0), (0.9,b1), (0.6,b1), (0.5,b0)
    s = np.array([[0.9, 0.5], [0.9, 0.6]])
    assert list(oracle.cut_budget(s, 1)) == [1, 0]
    assert list(oracle.cut_budget(s, 2)) == [1, 1]
    assert list(oracle.cut_budget(s, 3)) == [1, 2]
    s = np.array([[0.9, 0.6], [0.9, 0.6]])
    assert list(oracle.cut_budget(s, 3)) == [2, 1]


def test_cut_compares_double_values_as_they_are():
    # The cut compares and ranks the double survival values themselves: values
    # 1e-12 apart are distinct, so one is kept and one is not against a cutoff
    # lying between them, and the larger wins a budget of one whatever its
    # request. A cut rounded to any coarser precision would keep or tie both.
    c = np.float32(0.3)
    s = np.array([[float(c) + 1e-12, float(c) - 1e-12]])
    assert oracle.cut_threshold(s, np.array([c]))[0] == 1
    s2 = np.array([[float(c) - 1e-12], [float(c) + 1e-12]])
    assert list(oracle.cut_budget(s2, 1)) == [0, 1]
    s3 = np.array([[float(c)], [float(c)]])
    assert list(oracle.cut_budget(s3, 1)) == [1, 0]        # exact tie -> lower request
    assert list(oracle.cut_combined(s2, np.array([c, c]), 1)) == [0, 1]


def test_budget_rejects_negative():
    with pytest.raises(oracle.OracleError):
        oracle.cut_budget(np.full((1, 2), 0.5), -1)


# ------------------------------------------------------------------ compact

def test_compact_against_library_scan():
    rng = np.random.default_rng(7)
    B, g = 37, 9
    L = rng.integers(0, g + 1, B).astype(np.int32)
    tok = rng.integers(0, 50000, (B, g + 1)).astype(np.int32)
    cu, pt, ps = oracle.compact(L, tok)
    assert np.array_equal(cu, np.concatenate([[0], np.cumsum(L + 1)]))
    total = int((L + 1).sum())
    assert np.array_equal(pt[:total], np.concatenate([tok[b, :L[b] + 1] for b in range(B)]))
    dense = np.concatenate([b * (g + 1) + np.arange(L[b] + 1) for b in range(B)])
    assert np.array_equal(ps[:total], dense)
    assert np.all(np.diff(ps[:total]) > 0)
    assert np.all(pt[total:] == -1) and np.all(ps[total:] == -1)   # tail untouched


def test_compact_rejects_bad_length():
    with pytest.raises(oracle.OracleError):
        oracle.compact(np.array([3], np.int32), np.zeros((1, 3), np.int32))


# ------------------------------------------------------------------- argmax

def test_argmax_matches_library_first_occurrence():
    rng = np.random.default_rng(8)
    rows = bf(rng.standard_normal((40, 777)) * 2)
    rows[5, 100] = rows[5, 3] = bf([50.0])[0]          # exact tie: lowest index wins
    rows[6, :] = bf(1.0)                          # all equal -> index 0
    am = oracle.argmax_rows(rows)
    assert np.array_equal(am, np.argmax(bf16_bits_to_f32(rows), axis=1))
    assert am[5] == 3 and am[6] == 0


def test_argmax_signed_zero_and_negatives():
    rows = np.stack([exact_bf([-0.0, 0.0, -1.0]), exact_bf([-3.0, -0.0, 0.0]),
                     exact_bf([-5.0, -2.0, -2.0])])
    assert list(oracle.argmax_rows(rows)) == [0, 1, 1]


def test_argmax_src_rows_and_nonfinite():
    rng = np.random.default_rng(9)
    rows = bf(rng.standard_normal((10, 64)))
    src = np.array([7, 2, 2, 9], np.int32)
    assert np.array_equal(oracle.argmax_rows(rows, src), oracle.argmax_rows(rows)[src])
    rows[3, 5] = 0x7FC0                            # NaN is rejected
    with pytest.raises(oracle.OracleError):
        oracle.argmax_rows(rows, np.array([3], np.int32))


# ------------------------------------------------------------- accept/bonus

@pytest.mark.parametrize("seed", range(6))
def test_accept_known_planted_prefix(seed):
    # Every row's argmax is known by construction (one entry at +50 in a row
    # of values in [-2, 2]); drafts agree with the rows for exactly m_b
    # positions. Then a_b = min(L_b, m_b) and bonus_b = the known argmax of
    # row a_b. Catches off-by-one between rows and drafts and a missing cap.
    rng = np.random.default_rng(200 + seed)
    B, g, V = 6, 7, 300
    L = rng.integers(0, g + 1, B).astype(np.int32)
    m = rng.integers(0, g + 1, B)
    top = rng.integers(0, V, (B, g + 1))                 # argmax of dense row (b, j)
    logits = rng.uniform(-2, 2, (B, g + 1, V)).astype(np.float32)
    for b in range(B):
        for j in range(g + 1):
            logits[b, j, top[b, j]] = 50.0
    tok = np.zeros((B, g + 1), np.int32)
    tok[:, 0] = rng.integers(0, V, B)
    for b in range(B):
        for j in range(g):
            tok[b, j + 1] = top[b, j] if j < m[b] else (top[b, j] + 1 + rng.integers(0, V - 1)) % V
    lg = bf(logits)
    cu, pt, ps = oracle.compact(L, tok)
    am = oracle.argmax_rows(lg.reshape(-1, V), ps[: cu[-1]])
    acc, bon = oracle.accept(cu, tok, am)
    for b in range(B):
        a = min(int(L[b]), int(m[b]))
        assert acc[b] == a
        assert bon[b] == top[b, a]
        if a < L[b]:
            assert bon[b] != tok[b, a + 1]


# ---------------------------------------------------------- packed row gather

@pytest.mark.parametrize("dtype,row", [(np.uint8, (13,)), (np.int32, (3, 5)), (np.uint16, (64,))])
def test_gather_rows_against_fancy_indexing(dtype, row):
    # Row r < cu[B] is row packed_src_row[r] of src, byte for byte; the rest
    # of the destination keeps its contents. Catches an off-by-one row, a
    # wrong row width and writes past the packed total.
    rng = np.random.default_rng(7)
    B, g = 6, 4
    cap = B * (g + 1)
    src = rng.integers(0, 200, (cap,) + row).astype(dtype)
    L = rng.integers(0, g + 1, B).astype(np.int32)
    cu, pt, ps = oracle.compact(L, np.zeros((B, g + 1), np.int32))
    total = int(cu[-1])
    sentinel = np.full((cap,) + row, 77, dtype)
    out = oracle.gather_rows(src, ps, cu, dst=sentinel)
    assert np.array_equal(out[:total], src[ps[:total]])
    assert np.all(out[total:] == 77)
    # the rows gathered are request b's rows 0..L_b in order
    for b in range(B):
        for j in range(L[b] + 1):
            assert np.array_equal(out[cu[b] + j], src[b * (g + 1) + j])


def test_gather_rows_rejects_bad_source_row():
    cu = np.array([0, 2], np.int32)
    ps = np.array([0, 9], np.int32)
    with pytest.raises(oracle.OracleError):
        oracle.gather_rows(np.zeros((2, 4), np.uint8), ps, cu)


# ------------------------------------------- combined cut and cost-table cutoff

def _distinct_survival(rng, B, g):
    p = rng.uniform(0.3, 0.99, (B, g))
    return np.cumprod(p, axis=1)


@pytest.mark.parametrize("seed", range(8))
def test_combined_brute_force(seed):
    # Among every selection that keeps a prefix of each request's eligible
    # drafts (L_b <= threshold length) with min(T, #eligible) drafts in total,
    # the pick must be the one of largest kept survival mass (values distinct,
    # so the maximiser is unique). Catches a budget that ignores the cutoff,
    # ranking ineligible positions, and a wrong total.
    rng = np.random.default_rng(500 + seed)
    B, g = 3, 4
    surv = _distinct_survival(rng, B, g)
    c = rng.uniform(0.2, 0.8, B).astype(np.float32)
    T = int(rng.integers(0, B * g + 2))
    Lthr = oracle.cut_threshold(surv, c)
    want_total = min(T, int(Lthr.sum()))
    best, best_mass = None, -1.0
    for Ls in itertools.product(*[range(int(x) + 1) for x in Lthr]):
        if sum(Ls) != want_total:
            continue
        mass = sum(surv[b, :Ls[b]].sum() for b in range(B))
        if mass > best_mass:
            best, best_mass = Ls, mass
    L = oracle.cut_combined(surv, c, T)
    assert tuple(L.tolist()) == best


def test_combined_reduces_to_its_parts():
    rng = np.random.default_rng(21)
    B, g = 7, 6
    surv = _distinct_survival(rng, B, g)
    c = rng.uniform(0.1, 0.7, B).astype(np.float32)
    Lthr = oracle.cut_threshold(surv, c)
    # a budget that never binds leaves the threshold cut
    assert np.array_equal(oracle.cut_combined(surv, c, int(Lthr.sum())), Lthr)
    assert np.array_equal(oracle.cut_combined(surv, c, 10 ** 6), Lthr)
    # cutoffs that pass everything leave the budget cut
    zero = np.zeros(B, np.float32)
    for T in (0, 5, 17, B * g):
        assert np.array_equal(oracle.cut_combined(surv, zero, T), oracle.cut_budget(surv, T))
    # cutoffs above 1 pass nothing; each window never exceeds its threshold window
    assert np.all(oracle.cut_combined(surv, np.full(B, 2.0, np.float32), 30) == 0)
    for T in range(0, B * g + 1, 5):
        L = oracle.cut_combined(surv, c, T)
        assert np.all(L <= Lthr) and L.sum() == min(T, Lthr.sum())


def test_cost_cutoff_hand_example_and_tightening():
    table = np.array([0.1, 0.2, 0.3], np.float32)
    for load, want in ((-1, 0.1), (0, 0.1), (1, 0.2), (2, 0.3), (7, 0.3)):
        c = oracle.cost_cutoff(table, load, 4)
        assert c.dtype == np.float32 and np.all(c == np.float32(want))
    # a cost that rises with load tightens every window together
    rng = np.random.default_rng(3)
    surv = _distinct_survival(rng, 9, 8)
    prev = None
    for load in range(3):
        L = oracle.cut_threshold(surv, oracle.cost_cutoff(table, load, 9))
        if prev is not None:
            assert np.all(L <= prev)
        prev = L


# ----------------------------------------------------------------- graph tiers

def test_tier_select_hand_examples():
    # tiers 64/128/256 over a capacity of 4*(63+1) = 256 rows
    tiers = [64, 128, 256]
    B, g = 4, 63
    for total, want_pad, want_idx in ((100, 128, 1), (128, 128, 1), (0, 64, 0), (1, 64, 0),
                                      (256, 256, 2), (129, 256, 2)):
        cu = np.array([0, total, total, total, total], np.int32)
        pt = np.full(B * (g + 1), 5, np.int32)
        ps = np.full(B * (g + 1), 6, np.int32)
        padded, idx, pt2, ps2 = oracle.tier_select(cu, g, tiers, -9, pt, ps)
        assert (padded, idx) == (want_pad, want_idx)
        assert np.all(pt2[total:want_pad] == -9) and np.all(ps2[total:want_pad] == -1)
        assert np.all(pt2[:total] == 5) and np.all(pt2[want_pad:] == 5)
        assert np.all(ps2[want_pad:] == 6)


def test_tier_select_beyond_the_largest_tier_and_library_search():
    # no captured tier holds the batch: index ntiers, nothing padded; and on
    # random ladders the index is numpy's left insertion point
    padded, idx, pt, _ = oracle.tier_select(np.array([0, 40], np.int32), 63, [8, 16, 32], 0,
                                            np.zeros(64, np.int32))
    assert (padded, idx) == (40, 3) and np.all(pt == 0)
    rng = np.random.default_rng(5)
    for _ in range(50):
        tiers = np.unique(rng.integers(1, 300, rng.integers(1, 8))).astype(np.int32)
        total = int(rng.integers(0, 300))
        B = 5
        g = 59
        cu = np.array([0] + [total] * B, np.int32)
        padded, idx, _, _ = oracle.tier_select(cu, g, tiers, 0)
        assert idx == int(np.searchsorted(tiers, total, side="left"))
        assert padded == (int(tiers[idx]) if idx < len(tiers) else total)


def test_tier_select_rejects_unsorted_tiers():
    with pytest.raises(oracle.OracleError):
        oracle.tier_select(np.array([0, 3], np.int32), 3, [8, 8], 0)


# ------------------------------------------------ static and cap-accept modes

def _planted_block(rng, B, g, V):
    """Dense logits whose every row has a known argmax (+50 in values within
    [-2, 2]) and drafts agreeing with the rows for exactly m_b positions."""
    m = rng.integers(0, g + 1, B)
    top = rng.integers(0, V, (B, g + 1))
    logits = rng.uniform(-2, 2, (B, g + 1, V)).astype(np.float32)
    for b in range(B):
        for j in range(g + 1):
            logits[b, j, top[b, j]] = 50.0
    tok = np.zeros((B, g + 1), np.int32)
    tok[:, 0] = rng.integers(0, V, B)
    for b in range(B):
        for j in range(g):
            tok[b, j + 1] = top[b, j] if j < m[b] else (top[b, j] + 1 + rng.integers(0, V - 1)) % V
    return bf(logits), tok, top, m


@pytest.mark.parametrize("seed", range(6))
def test_cap_accept_known_planted_prefix(seed):
    # The full block is verified (static packing), the window is L_b: the
    # uncapped acceptance is the planted agreement m_b, the committed count is
    # min(L_b, m_b) and the bonus is the known argmax of that row. Catches a
    # missing cap, capping the record instead of the commit, and a bonus taken
    # from the wrong row.
    rng = np.random.default_rng(300 + seed)
    B, g, V = 7, 6, 257
    lg, tok, top, m = _planted_block(rng, B, g, V)
    L = rng.integers(0, g + 1, B).astype(np.int32)
    am_full = oracle.argmax_rows(lg.reshape(-1, V))
    acc, bon, full = oracle.cap_accept(L, tok, am_full)
    for b in range(B):
        assert full[b] == m[b]
        a = min(int(L[b]), int(m[b]))
        assert acc[b] == a and bon[b] == top[b, a]


@pytest.mark.parametrize("seed", range(4))
def test_cap_accept_output_equals_compact(seed):
    # The pages' invariant of the audit arm: cap-accept pays the full verify
    # but its committed output equals compact's exactly. The two sides take
    # different routes (argmax of packed rows after compaction, against argmax
    # of every row then a cap), so an index slip in either shows here.
    rng = np.random.default_rng(400 + seed)
    B, g, V = 11, 5, 190
    lg, tok, top, m = _planted_block(rng, B, g, V)
    # unplanted noise rows too: overwrite some requests' rows with plain noise
    noise = bf(rng.standard_normal((B, g + 1, V)))
    pick = rng.random(B) < 0.4
    lg = np.where(pick[:, None, None], noise, lg)
    L = rng.integers(0, g + 1, B).astype(np.int32)
    cu, pt, ps = oracle.compact(L, tok)
    am = oracle.argmax_rows(lg.reshape(-1, V), ps[: cu[-1]])
    acc_c, bon_c = oracle.accept(cu, tok, am)
    acc, bon, full = oracle.cap_accept(L, tok, oracle.argmax_rows(lg.reshape(-1, V)))
    assert np.array_equal(acc, acc_c) and np.array_equal(bon, bon_c)
    assert np.all(full >= acc) and np.all(acc <= L)
    # where the window is not binding, the record equals the commit
    loose = full <= L
    assert np.array_equal(full[loose], acc[loose])


def test_static_mode_is_the_full_window():
    # Static verify: every length is gamma, cu_seqlens is b*(gamma+1), and the
    # accepted counts are cap-accept's uncapped record. Catches a static mode
    # that still applies a cut, and a packing that is not the identity.
    rng = np.random.default_rng(12)
    B, g, d, V = 5, 4, 32, 150
    h = bf(rng.standard_normal((B, g, d)))
    w = bf(rng.standard_normal(d) / math.sqrt(d))
    temps = (1 + 0.05 * np.arange(g)).astype(np.float32)
    lg, tok, top, m = _planted_block(rng, B, g, V)
    o = oracle.step(h, w, 0.0, temps, tok, lg, "static")
    assert np.all(o["lengths"] == g)
    assert np.array_equal(o["cu_seqlens"], np.arange(B + 1) * (g + 1))
    assert np.array_equal(o["packed_src_row"], np.arange(B * (g + 1)))
    _, _, full = oracle.cap_accept(np.full(B, g, np.int32), tok, o["packed_argmax"])
    assert np.array_equal(o["accepted"], full) and np.array_equal(full, m)
    assert np.array_equal(oracle.cut_static(B, g), np.full(B, g))


def test_utilization_hand_example():
    # committed 2 + 0 + 3 = 5 of a full-verify 4 + 1 + 3 = 8: 5/8; a window that
    # never binds gives 1; nothing acceptable counts as full use.
    assert oracle.utilization([2, 0, 3], [4, 1, 3]) == 5 / 8
    assert oracle.utilization([1, 2], [1, 2]) == 1.0
    assert oracle.utilization([0, 0], [0, 0]) == 1.0


def test_cap_accept_rejects_bad_length():
    with pytest.raises(oracle.OracleError):
        oracle.cap_accept(np.array([3], np.int32), np.zeros((1, 3), np.int32),
                          np.zeros(3, np.int32))


# --------------------------------------------------------------- whole step

def test_step_equals_stage_chain_and_invariants():
    rng = np.random.default_rng(10)
    B, g, d, V = 9, 6, 48, 200
    h = bf(rng.standard_normal((B, g, d)))
    w = bf(rng.standard_normal(d) / math.sqrt(d))
    temps = (1 + 0.05 * np.arange(g)).astype(np.float32)
    tok = rng.integers(0, V, (B, g + 1)).astype(np.int32)
    lg = bf(rng.standard_normal((B, g + 1, V)))
    c = rng.uniform(0.05, 0.6, B).astype(np.float32)
    for mode in ("threshold", "budget"):
        o = oracle.step(h, w, 0.3, temps, tok, lg, mode, cutoff=c, budget=17)
        z, p = oracle.confidence(h, w, 0.3, temps)
        s = oracle.survival(p)
        L = oracle.cut_threshold(s, c) if mode == "threshold" else oracle.cut_budget(s, 17)
        cu, pt, ps = oracle.compact(L, tok)
        am = oracle.argmax_rows(lg.reshape(-1, V), ps[: cu[-1]])
        acc, bon = oracle.accept(cu, tok, am)
        assert np.array_equal(o["lengths"], L) and np.array_equal(o["cu_seqlens"], cu)
        assert np.array_equal(o["packed_argmax"][: cu[-1]], am)
        assert np.array_equal(o["accepted"], acc) and np.array_equal(o["bonus"], bon)
        assert np.all(acc <= L) and cu[-1] == (L + 1).sum()
        if mode == "budget":
            assert L.sum() == 17
