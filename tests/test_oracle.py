"""Pins for the CPU oracle: each test ties a part of it to something other than itself.

The oracle exists twice, written apart: the plain C++ implementation (oracle/routed_attention.cpp,
through oracle/cpp.py) and the numpy one (oracle/routed_attention.py).  Every pin of the method's
steps runs against both (the ``impl`` fixture), and a cross-check compares the two on seeded
problems (summaries and selections bit for bit, outputs within 1e-12).

Kinds of pin used: exact arithmetic (Python integers / fractions), a library routine that is
independent of the oracle's code (torch's bf16 conversion, torch's scaled-dot-product attention
in float64), brute force on tiny inputs (rank counting instead of sorting), closed forms
(uniform weights over a bit-coded value table), and the complexity claim printed in the
release post's "Key idea" section (tests/golden/complexity_claim.json).
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
import oracle.cpp as CPP

HERE = os.path.dirname(os.path.abspath(__file__))

IMPLS = {"numpy": O, "cpp": CPP}


@pytest.fixture(params=sorted(IMPLS))
def impl(request):
    """One oracle implementation: the numpy module or the C++ library's Python face."""
    return IMPLS[request.param]


def bf16_bits(a):
    """float32 -> bf16 bit patterns (uint16) by torch's conversion (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(
        np.uint16)


def torch_widen(bits_or_f32):
    """Exact float64 values of stored inputs by torch's own conversions (independent of the
    oracle's widening): bf16 bit patterns through torch.bfloat16, float32 through torch."""
    a = np.ascontiguousarray(bits_or_f32)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    return torch.from_numpy(a).to(torch.float64).numpy()


# ------------------------------------------------------------------------------------------ kappa
def test_round_to_bf16_matches_torch_conversion(impl):
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        (rng.standard_normal(2000) * 1e-30).astype(np.float32),
                        (rng.standard_normal(2000) * 1e30).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, -3.5, 2.0 ** -126, 2.0 ** -130], dtype=np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(impl.round_to_bf16(x), ref)


def test_round_to_bf16_ties_to_even(impl):
    one = 1.0
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7 (odd significand) -> 1
    assert impl.round_to_bf16(np.float32(one + 2.0 ** -8)) == np.float32(1.0)
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even) -> 1 + 2^-6
    assert impl.round_to_bf16(np.float32(one + 3 * 2.0 ** -8)) == np.float32(1 + 2.0 ** -6)
    # just above the halfway point rounds up
    assert impl.round_to_bf16(np.float32(one + 2.0 ** -8 + 2.0 ** -20)) == np.float32(1 + 2.0 ** -7)


def test_widen_matches_torch_on_every_bf16_pattern(impl):
    """All 65,536 bf16 bit patterns widen to torch's bf16 -> float value (NaN patterns to NaN),
    through the float64 widening and, for the numpy oracle, the float32 one."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 * 127  # exponent all ones, significand non-zero, either sign
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns raise the flag when widened
        got = impl.widen(bits, True)
    assert got.dtype == np.float64
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))  # -0 stays -0
    if impl is O:
        g32 = O.widen_f32(bits, True)
        assert g32.dtype == np.float32
        assert np.array_equal(np.isnan(g32), nan)
        assert np.array_equal(g32[~nan].astype(np.float64), ref[~nan])
        # float32 inputs pass through unchanged
        x = np.array([1.5, -0.0, 3e-45, 3.4e38], dtype=np.float32)
        assert np.array_equal(O.widen_f32(x, False).view(np.uint32), x.view(np.uint32))
    x = np.array([1.5, -0.0, 3e-45, 3.4e38, -7.25], dtype=np.float32)
    assert np.array_equal(impl.widen(x, False), torch.from_numpy(x).to(torch.float64).numpy())


def test_score_abs_bound_equals_exact_rational_evaluation():
    """gamma_d * max_j sum_e |q_e kappa(mean_j)_e| over j < r, evaluated with fractions.

    Inputs: signed small integers (so that a missing absolute value changes the sum), the largest
    term in a middle span (not the first or last), a huge span past r (must be ignored), and
    means that kappa rounds (1 + 2^-9 -> 1) so that the bf16 and fp32 bounds differ."""
    d = 8
    u = Fraction(1, 2 ** 24)
    gamma = Fraction(d) * u / (1 - Fraction(d) * u)
    q = np.array([3, -2, 1, 0, -4, 5, -1, 2], dtype=np.float64)
    means = np.array([[1, 1, -1, 0, 0, 0, 0, 0],
                      [-2, 3, 1, 7, -1, 2, 0, -3],      # the largest sum of |q_e m_e|
                      [1 + 2.0 ** -9, 0, 0, 0, 0, 0, 0, 0],
                      [1000, 1000, 1000, 1000, 1000, 1000, 1000, 1000]], dtype=np.float32)
    r = 3

    def exact(kappa):
        best = Fraction(0)
        for j in range(r):
            row = [Fraction(float(kappa(means[j, e]))) for e in range(d)]
            best = max(best, sum(abs(Fraction(float(q[e])) * row[e]) for e in range(d)))
        return gamma * best

    ident = lambda x: x
    to_bf16 = lambda x: torch.tensor(float(x), dtype=torch.float32).to(torch.bfloat16).to(torch.float64).item()
    for is_bf16, kappa in ((False, ident), (True, to_bf16)):
        got = O.score_abs_bound(q, means, r, is_bf16)
        want = exact(kappa)
        assert abs(Fraction(got) - want) <= want * Fraction(1, 2 ** 50), (is_bf16, got, float(want))
    assert O.score_abs_bound(q, means, 0, True) == 0.0
    # kappa changes the bound when the rounded span is the largest one
    q2 = np.array([1, 0, 0, 0, 0, 0, 0, 0], dtype=np.float64)
    m2 = np.array([[1 + 2.0 ** -9, 0, 0, 0, 0, 0, 0, 0]], dtype=np.float32)
    close = lambda got, want: abs(Fraction(got) - want) <= want * Fraction(1, 2 ** 50)
    assert close(O.score_abs_bound(q2, m2, 1, True), gamma)
    assert close(O.score_abs_bound(q2, m2, 1, False), gamma * (1 + Fraction(1, 2 ** 9)))


@pytest.mark.parametrize("bf16", [False, True])
def test_cpp_and_numpy_oracles_agree(bf16):
    """The two oracles on seeded problems: summaries (one-shot and appended in pieces) and
    selections bit for bit, scores and outputs within 1e-12, weights summing to 1."""
    rng = np.random.default_rng(21 + bf16)
    for (L, S, W, k, d, hkv, hq) in [(700, 16, 20, 4, 32, 2, 4), (1200, 32, 32, 6, 64, 1, 3), (90, 8, 1, 64, 16, 2, 2)]:
        keys = rng.standard_normal((hkv, L, d)).astype(np.float32)
        keys[:, : L // 2] += rng.standard_normal((hkv, 1, d)).astype(np.float32)
        vals = rng.standard_normal((hkv, L, d)).astype(np.float32)
        qs = rng.standard_normal((40, hq, d)).astype(np.float32)
        if bf16:
            keys, vals, qs = bf16_bits(keys), bf16_bits(vals), bf16_bits(qs)
        pn = O.Problem(keys, vals, L, hq, S, k, W, bf16)
        pc = CPP.Problem(keys, vals, L, hq, S, k, W, bf16)
        assert np.array_equal(pn.means.view(np.uint32), pc.means.view(np.uint32))
        # appended in uneven pieces
        m = np.zeros_like(pc.means)
        run = np.zeros((hkv, d), dtype=np.float32)
        cuts = sorted(set([0, L] + rng.integers(0, L, 6).tolist()))
        for a, b in zip(cuts[:-1], cuts[1:]):
            CPP.summary_update(keys, m, run, a, b, S)
        _, run_n = O.summaries(O.widen_f32(keys, bf16), L, S)
        assert np.array_equal(m.view(np.uint32), pn.means.view(np.uint32))
        assert np.array_equal(run.view(np.uint32), run_n.view(np.uint32))
        pos = np.concatenate([[0, 1, L - 1], rng.integers(0, L, 37)])
        res = pc.rows(qs, pos, scores=True)
        for i, t in enumerate(pos):
            for h in range(hq):
                a = pn.row(qs[i, h], h, int(t))
                assert np.array_equal(a["sel"], res["sel"][i, h]), (L, i, h)
                assert a["n_attended"] == res["n_attended"][i, h]
                assert np.abs(a["out"] - res["out"][i, h]).max() <= 1e-12
                if len(a["scores"]):
                    assert np.abs(a["scores"] - res["scores"][i][h]).max() <= 1e-12 * np.abs(a["scores"]).max()
                assert abs(res["weight_sum"][i, h] - 1.0) <= 1e-12
        dn = pc.rows(qs[:5], pos[:5], dense=True)
        for i in range(5):
            for h in range(hq):
                assert np.abs(dn["out"][i, h] - pn.dense_row(qs[i, h], h, int(pos[i]))).max() <= 1e-12


def test_cpp_oracle_skips_repeated_and_unroutable_entries_of_a_given_selection():
    """A given selection with repeats, -1 and ids >= r attends the distinct routable spans once."""
    rng = np.random.default_rng(31)
    L, S, W, k, d = 900, 16, 16, 8, 16
    keys = rng.standard_normal((1, L, d)).astype(np.float32)
    vals = rng.standard_normal((1, L, d)).astype(np.float32)
    pc = CPP.Problem(keys, vals, L, 1, S, k, W, False)
    pn = O.Problem(keys, vals, L, 1, S, k, W, False)
    q = rng.standard_normal(d).astype(np.float32)
    t = 700
    r = O.num_routable(t, S, W)
    given = np.array([5, 9, 5, -1, r, r + 3, 9, 2], dtype=np.int64)
    a = pc.row(q, 0, t, sel=given)
    b = pn.row(q, 0, t, sel=np.array([2, 5, 9]))
    assert a["n_attended"] == b["n_attended"] == 3 * S + (t - O.window_start(t, S, W) + 1)
    assert np.abs(a["out"] - b["out"]).max() <= 1e-12


# ---------------------------------------------------------------------------------- summaries
def test_summary_of_constant_span_is_that_constant(impl):
    S, d = 16, 8
    for c in [0.375, -2.5, 1.0 / 1024]:  # dyadic constants: every partial sum is exact in fp32
        keys = np.full((2, 5 * S, d), c, dtype=np.float32)
        means, run = impl.summaries(keys, 5 * S, S)
        assert np.all(means == np.float32(c))
        assert np.all(run == 0)


def test_summary_integer_keys_exact_mean(impl):
    """Small-integer keys sum exactly in fp32; the mean must be the exact rational sum/S."""
    rng = np.random.default_rng(2)
    S, d, L = 8, 6, 8 * 7 + 3
    ints = rng.integers(-50, 51, size=(3, L, d))
    keys = ints.astype(np.float32)
    means, run = impl.summaries(keys, L, S)
    assert means.shape == (3, L // S, d)
    for h in range(3):
        for j in range(L // S):
            for e in range(d):
                exact = Fraction(int(ints[h, j * S:(j + 1) * S, e].sum()), S)
                assert Fraction(float(means[h, j, e])) == exact
        # open span: running sum of the 3 tail tokens, exact
        for e in range(d):
            assert run[h, e] == float(ints[h, (L // S) * S:, e].sum())


def test_summary_sums_in_token_order_in_fp32(impl):
    """1 followed by S-1 copies of 2^-24: each fp32 addition 1 + 2^-24 ties to even -> 1."""
    S = 4
    keys = np.array([[[1.0], [2.0 ** -24], [2.0 ** -24], [2.0 ** -24]]], dtype=np.float32)
    means, _ = impl.summaries(keys, S, S)
    assert means[0, 0, 0] == np.float32(0.25)
    # the exactly rounded mean would differ: the order-of-addition reading is what is pinned
    assert np.float32((1 + 3 * 2.0 ** -24) / 4) != np.float32(0.25)


@pytest.mark.parametrize("chunk", [1, 7, 16, 100])
def test_summary_incremental_equals_one_shot(impl, chunk):
    rng = np.random.default_rng(3)
    S, d, L = 16, 8, 16 * 9 + 5
    keys = rng.standard_normal((2, L, d)).astype(np.float32)
    m1, r1 = impl.summaries(keys, L, S)
    means = np.zeros((2, L // S, d), dtype=np.float32)
    run = np.zeros((2, d), dtype=np.float32)
    p = 0
    while p < L:
        q = min(L, p + chunk)
        impl.summary_update(keys, means, run, p, q, S)
        p = q
    assert np.array_equal(means, m1) and np.array_equal(run, r1)


def test_summary_close_to_exact_mean(impl):
    rng = np.random.default_rng(4)
    S, d, L = 64, 16, 64 * 6
    keys = rng.standard_normal((1, L, d)).astype(np.float32)
    means, _ = impl.summaries(keys, L, S)
    exact = keys.astype(np.float64).reshape(1, 6, S, d).mean(axis=2)
    bound = S * 2.0 ** -24 * np.abs(keys.astype(np.float64)).reshape(1, 6, S, d).mean(axis=2) * 1.01 + 1e-30
    assert np.all(np.abs(means - exact) <= bound)


# ------------------------------------------------------------------------------ window / spans
def test_window_and_routable_closed_forms(impl):
    S, W = 64, 64
    assert impl.window_start(0, S, W) == 0 and impl.num_routable(0, S, W) == 0
    assert impl.num_routable(126, S, W) == 0
    assert impl.num_routable(127, S, W) == 1 and impl.window_start(127, S, W) == 64
    for t in range(0, 2000):
        w0 = impl.window_start(t, S, W)
        assert w0 % S == 0 and w0 <= max(0, t - W + 1)
        size = t - w0 + 1
        assert size <= W + S - 1
        assert t < W - 1 or size >= W
    # W = 3S: window holds 3S .. 4S-1 tokens once t is large
    for t in range(1000, 1200):
        assert 3 * 16 <= t - impl.window_start(t, 16, 48) + 1 <= 4 * 16 - 1


def test_every_past_token_is_routable_or_in_window(impl):
    for S, W in [(8, 8), (8, 1), (8, 20), (5, 13)]:
        for t in range(0, 200):
            r = impl.num_routable(t, S, W)
            covered = set(range(0, r * S)) | set(range(impl.window_start(t, S, W), t + 1))
            assert covered == set(range(t + 1)), (S, W, t)


# ------------------------------------------------------------------------------------ scores
def test_scores_exact_on_integers_and_unscaled(impl):
    rng = np.random.default_rng(5)
    d, r = 32, 20
    q = rng.integers(-4, 5, size=d).astype(np.float32)
    means = rng.integers(-3, 4, size=(r + 3, d)).astype(np.float32)
    s = impl.route_scores(q, means, r, is_bf16=True)  # small integers are bf16-exact
    for j in range(r):
        assert s[j] == sum(int(q[e]) * int(means[j, e]) for e in range(d))
    assert len(s) == r


def test_scores_round_mean_to_bf16_for_bf16_inputs(impl):
    means = np.array([[1.0 + 2.0 ** -9, 0.0]], dtype=np.float32)
    q = np.array([1.0, 0.0], dtype=np.float32)
    assert impl.route_scores(q, means, 1, is_bf16=True)[0] == 1.0
    assert impl.route_scores(q, means, 1, is_bf16=False)[0] == 1.0 + 2.0 ** -9


# --------------------------------------------------------------------------------- selection
def _brute_selection(scores, k):
    """j is kept iff fewer than m spans beat it: rank counting, no sorting."""
    r = len(scores)
    m = min(k, r)
    keep = [j for j in range(r)
            if sum(1 for i in range(r) if scores[i] > scores[j] or (scores[i] == scores[j] and i < j)) < m]
    return keep + [-1] * (k - len(keep))


def test_selection_matches_rank_counting_with_ties(impl):
    rng = np.random.default_rng(6)
    for trial in range(300):
        r = int(rng.integers(0, 25))
        k = int(rng.integers(1, 10))
        scores = rng.integers(-3, 4, size=r).astype(np.float64) * 0.5  # many exact ties
        assert list(impl.select_spans(scores, k)) == _brute_selection(list(scores), k)


def test_selection_matches_exhaustive_subset_search(impl):
    """The kept set maximises the score sum; among maximisers, it is lexicographically smallest."""
    rng = np.random.default_rng(7)
    for _ in range(60):
        r = int(rng.integers(1, 11))
        k = int(rng.integers(1, 6))
        scores = rng.standard_normal(r)
        m = min(k, r)
        best = max(itertools.combinations(range(r), m), key=lambda c: (sum(scores[j] for j in c), [-j for j in c]))
        assert list(impl.select_spans(scores, k)[:m]) == sorted(best)


def test_selection_special_cases(impl):
    assert list(impl.select_spans(np.zeros(10), 4)) == [0, 1, 2, 3]          # q = 0: lowest indices win
    assert list(impl.select_spans(np.array([1.0, 2.0]), 4)) == [0, 1, -1, -1]  # k > r: all spans
    assert list(impl.select_spans(np.array([]), 3)) == [-1, -1, -1]           # r = 0: window only
    s = np.array([0.1, 5.0, 3.0, 5.0, 3.0])                               # duplicates: lower index wins
    assert list(impl.select_spans(s, 3)) == [1, 2, 3]


# ------------------------------------------------------------------------- attended set / softmax
def _count_bit_set(a, b, e):
    """How many integers in [a, b] have bit e set (closed form)."""
    def upto(n):  # integers in [0, n)
        block = 1 << (e + 1)
        return (n // block) * (1 << e) + max(0, n % block - (1 << e))
    return upto(b + 1) - upto(a)


def _bitcoded_problem(L, S, k, W, d, hkv=1, hq=1, bf16=False):
    pos = np.arange(L)
    vals = ((pos[:, None] >> np.arange(d)[None, :]) & 1).astype(np.float32)
    values = np.broadcast_to(vals, (hkv, L, d)).copy()
    rng = np.random.default_rng(8)
    keys = rng.standard_normal((hkv, L, d)).astype(np.float32)
    return keys, values


def test_zero_query_gives_uniform_average_over_exact_token_set(impl):
    L, S, k, W, d = 1500, 16, 5, 24, 12
    keys, values = _bitcoded_problem(L, S, k, W, d)
    prob = impl.Problem(keys, values, L, 1, S, k, W, is_bf16=False)
    q = np.zeros(d, dtype=np.float32)
    for t in [0, 5, 38, 39, 40, 100, 777, 1499]:
        res = prob.row(q, 0, t)
        r = impl.num_routable(t, S, W)
        m = min(k, r)
        w0 = impl.window_start(t, S, W)
        ranges = [(j * S, j * S + S - 1) for j in range(m)] + [(w0, t)]  # q = 0 -> spans 0..m-1
        n = sum(b - a + 1 for a, b in ranges)
        assert res["n_attended"] == n
        for e in range(d):
            frac = Fraction(sum(_count_bit_set(a, b, e) for a, b in ranges), n)
            assert abs(res["out"][e] - float(frac)) < 1e-12, (t, e)
        assert abs(res["weight_sum"] - 1.0) < 1e-12


def test_constant_values_give_constant_output_and_weights_sum_to_one(impl):
    rng = np.random.default_rng(9)
    L, S, k, W, d = 900, 8, 3, 8, 16
    keys = (rng.standard_normal((2, L, d)) * 3).astype(np.float32)
    values = np.ones((2, L, d), dtype=np.float32)
    prob = impl.Problem(keys, values, L, 4, S, k, W, is_bf16=False)
    for t in [3, 64, 899]:
        q = (rng.standard_normal(d) * 4).astype(np.float32)
        for hq in range(4):
            res = prob.row(q, hq, t)
            assert np.allclose(res["out"], 1.0, atol=1e-13, rtol=0)
            assert abs(res["weight_sum"] - 1.0) < 1e-12


def test_dominant_key_wins(impl):
    L, S, k, W, d = 256, 8, 2, 8, 4
    keys = np.zeros((1, L, d), dtype=np.float32)
    values = np.random.default_rng(10).standard_normal((1, L, d)).astype(np.float32)
    keys[0, 37] = [100.0, 0, 0, 0]
    # span 4 (positions 32..39) holds the only large key; its mean dominates routing
    prob = impl.Problem(keys, values, L, 1, S, k, W, is_bf16=False)
    res = prob.row(np.array([10.0, 0, 0, 0], dtype=np.float32), 0, 255)
    assert 4 in res["sel"]
    assert np.allclose(res["out"], values[0, 37], atol=1e-12)


# ------------------------------------------------------------------- whole path vs a library routine
def _sdpa_f64(q, keys, values, mask):
    """torch scaled_dot_product_attention in float64 (independent of the oracle's code)."""
    qt = torch.from_numpy(np.asarray(q, dtype=np.float64))[None, None, None, :]
    kt = torch.from_numpy(keys.astype(np.float64))[None, None]
    vt = torch.from_numpy(values.astype(np.float64))[None, None]
    mt = torch.from_numpy(mask)[None, None, None, :]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mt)[0, 0, 0].numpy()


@pytest.mark.parametrize("bf16", [False, True])
def test_k_all_spans_equals_dense_causal_attention(impl, bf16):
    rng = np.random.default_rng(11)
    L, S, W, d, hkv, hq = 333, 8, 8, 16, 2, 4
    keys = rng.standard_normal((hkv, L, d)).astype(np.float32)
    values = rng.standard_normal((hkv, L, d)).astype(np.float32)
    qs = rng.standard_normal((L, hq, d)).astype(np.float32)
    if bf16:
        keys, values, qs = bf16_bits(keys), bf16_bits(values), bf16_bits(qs)
    k_all = L // S + 1
    prob = impl.Problem(keys, values, L, hq, S, k_all, W, is_bf16=bf16)
    kd, vd, qd = torch_widen(keys), torch_widen(values), torch_widen(qs)
    for t in list(range(0, 40)) + list(range(300, L)):
        for h in range(hq):
            res = prob.row(qs[t, h], h, t)
            mask = np.arange(L) <= t
            ref = _sdpa_f64(qd[t, h], kd[h // 2], vd[h // 2], mask)
            assert np.abs(res["out"] - ref).max() < 1e-12, (t, h)


def test_routed_equals_masked_attention_over_selected_tokens(impl):
    rng = np.random.default_rng(12)
    L, S, W, k, d = 640, 16, 20, 3, 8
    keys = rng.standard_normal((1, L, d)).astype(np.float32)
    values = rng.standard_normal((1, L, d)).astype(np.float32)
    prob = impl.Problem(keys, values, L, 1, S, k, W, is_bf16=False)
    for t in [100, 333, 639]:
        q = rng.standard_normal(d).astype(np.float32)
        res = prob.row(q, 0, t)
        mask = np.zeros(L, dtype=bool)
        for j in res["sel"]:
            if j >= 0:
                mask[j * S:(j + 1) * S] = True
        mask[impl.window_start(t, S, W):t + 1] = True
        assert not mask[t + 1:].any()
        ref = _sdpa_f64(q, keys[0], values[0], mask)
        assert np.abs(res["out"] - ref).max() < 1e-12


def test_planted_needle_is_routed(impl):
    rng = np.random.default_rng(13)
    L, S, W, k, d = 4096, 64, 64, 2, 32
    keys = rng.standard_normal((1, L, d)).astype(np.float32)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    keys[0, 17 * S:18 * S] += (4 * u).astype(np.float32)  # span 17 carries a strong direction
    values = rng.standard_normal((1, L, d)).astype(np.float32)
    prob = impl.Problem(keys, values, L, 1, S, k, W, is_bf16=False)
    res = prob.row((8 * u).astype(np.float32), 0, L - 1)
    assert 17 in res["sel"]


# --------------------------------------------------------------------------------- comparator
def test_comparator_rejects_non_finite_outputs():
    """A NaN or infinite output element is an infinite error (and max() keeps it)."""
    ref = np.array([0.5, -1.0, 2.0])
    for bad in (np.nan, np.inf, -np.inf):
        got = ref.copy()
        got[1] = bad
        ma, rel = O.output_errors(got, ref)
        assert ma == np.inf and rel == np.inf
        assert max(0.0, ma) == np.inf
        assert not O.output_ok(got, ref, True)[0] and not O.output_ok(got, ref, False)[0]
    assert O.output_errors(ref, ref) == (0.0, 0.0)


def test_comparator_accepts_near_ties_and_rejects_real_swaps():
    scores = np.array([1.0, 0.5, 0.5000001, 0.2, -1.0])
    oracle_sel = O.select_spans(scores, 2)
    assert list(oracle_sel) == [0, 2]
    assert O.selection_verdict(oracle_sel, oracle_sel, scores, 2, 0.0) == "exact"
    assert O.selection_verdict(np.array([0, 1]), oracle_sel, scores, 2, 0.0) == "near_tie"
    assert O.selection_verdict(np.array([0, 3]), oracle_sel, scores, 2, 0.0).startswith("fail")
    assert O.selection_verdict(np.array([1, 2]), oracle_sel, scores, 2, 0.0).startswith("fail")
    assert O.selection_verdict(np.array([2, 0]), oracle_sel, scores, 2, 0.0).startswith("fail")
    assert O.selection_verdict(np.array([0, -1]), oracle_sel, scores, 2, 0.0).startswith("fail")
    assert O.selection_verdict(np.array([0, 7]), oracle_sel, scores, 2, 0.0).startswith("fail")


# ------------------------------------------------------------------------- the page's claim
def test_search_budget_grows_like_sqrt_of_context():
    with open(os.path.join(HERE, "golden", "complexity_claim.json")) as f:
        claim = json.load(f)
    ratio_ctx = claim["context_growth"]
    budget = []
    for L in [2 ** 20, 2 ** 20 * ratio_ctx]:
        S = int(round(math.sqrt(L)))
        t = L - 1
        budget.append(O.num_routable(t, S, S) + 1)  # spans scored by the last query (+ its window span)
    assert abs(budget[1] / budget[0] - claim["search_budget_growth"]) <= claim["tolerance"]


# ------------------------------------------------------------------------------ 8-bit cache
def test_e4m3_decode_follows_the_format_and_torch():
    """Every E4M3 bit pattern decodes as the format defines (bias 7, subnormals 2^-6 f/8, one NaN
    pattern per sign, no infinity), and as torch's float8_e4m3fn does."""
    Q = O.kv_fp8
    assert Q.e4m3_decode(np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x3C, 0x7E, 0x80, 0xFE], np.uint8)).tolist() == [
        0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 1.5, 448.0, -0.0, -448.0]
    assert np.isnan(Q.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()
    codes = np.arange(256, dtype=np.uint8)
    ours = Q.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[~np.isnan(ours)], ref[~np.isnan(ref)])


def test_e4m3_encode_rounds_to_nearest_even():
    Q = O.kv_fp8
    cases = {1.0625: 0x38, 1.1875: 0x3A, 2.0 ** -10: 0x00, 3 * 2.0 ** -11: 0x01, 1.5 * 2.0 ** -9: 0x02,
             448.0: 0x7E, 440.0: 0x7E, 432.0: 0x7E, 431.9: 0x7D, -1.0: 0xB8, 2.0 ** -6: 0x08}
    for x, c in cases.items():
        assert int(Q.e4m3_encode(np.array([x]))[0]) == c, (x, c)
    # every value back to itself, and a dense sweep against torch (its conversion rounds the same
    # way inside the clamped range)
    vals = Q.e4m3_decode(np.arange(256, dtype=np.uint8))
    ok = ~np.isnan(vals)
    assert np.array_equal(Q.e4m3_decode(Q.e4m3_encode(vals[ok])), vals[ok])
    x = np.concatenate([np.linspace(-448, 448, 100001), np.ldexp(np.linspace(-1, 1, 2001), -5)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(Q.e4m3_encode(x), ref)


def test_row_quantisation_error_and_special_rows():
    """Each element lands within half an E4M3 step (times the row scale) of its value, the row
    maximum maps to +-448, and an all-zero row gets codes 0 and scale 1."""
    Q = O.kv_fp8
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((64, 128)) * np.exp(rng.uniform(-6, 6, (64, 1)))).astype(np.float32)
    x[3] = 0.0
    codes, s = Q.quantize_rows(x)
    assert codes.dtype == np.uint8 and s.dtype == np.float32
    assert np.all(codes[3] == 0) and s[3] == 1.0
    back = Q.dequantize_rows(codes, s).astype(np.float64)
    q = x.astype(np.float64) / s[:, None].astype(np.float64)
    _, u = np.frexp(q)
    step = np.ldexp(1.0, np.maximum(u - 4, -9))
    err = np.abs(back - x) / s[:, None]
    assert np.all(err <= 0.5 * step * (1 + 1e-6) + 1e-6)
    nz = np.arange(64) != 3
    assert np.all(np.abs(Q.e4m3_decode(codes[nz])).max(axis=1) == 448.0)


def test_fp8_problem_reads_the_dequantised_cache():
    """With values that E4M3 and their scale represent exactly, the 8-bit problem equals the
    float32 problem of the same values (routing on bf16-rounded means, bf16 queries)."""
    Q = O.kv_fp8
    rng = np.random.default_rng(6)
    Hkv, L, d, S, W, k = 2, 96, 64, 16, 16, 3
    vals = Q.e4m3_decode(np.arange(0, 0x7E, dtype=np.uint8))
    kq = rng.choice(vals, size=(Hkv, L, d)) * rng.choice([-1, 1], size=(Hkv, L, d))
    vq = rng.choice(vals, size=(Hkv, L, d)) * rng.choice([-1, 1], size=(Hkv, L, d))
    kq[..., 0] = 448.0
    vq[..., 0] = -448.0  # row maxima 448: scale 1, codes = values
    kc, ks = Q.quantize_rows(kq.astype(np.float32))
    vc, vs = Q.quantize_rows(vq.astype(np.float32))
    assert np.all(ks == 1.0) and np.all(vs == 1.0)
    prob8 = Q.Fp8Problem(kc, ks, vc, vs, L, 4, S, k, W)
    qb = (rng.standard_normal((4, d)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    probf = O.Problem(kq.astype(np.float32), vq.astype(np.float32), L, 4, S, k, W, False)
    for h in range(4):
        for t in (40, 95):
            a = prob8.row(qb[h], h, t)
            qf = O.widen(qb[h], True).astype(np.float32)
            b = probf.row(qf, h, t)
            assert np.array_equal(a["out"], b["out"])
            # routing: bf16-rounded means (kappa), as the bf16 path
            assert np.array_equal(a["scores"], O.route_scores(O.widen(qb[h], True), probf.means[h // 2],
                                                              len(a["scores"]), True))



def test_numpy_rows_and_tasks_match_the_cpp_oracle():
    """The numpy oracle's batch interface (used by the 8-bit cache oracle) gives the C++
    oracle's results, including a given selection with repeats and unroutable ids."""
    rng = np.random.default_rng(41)
    L, S, W, k, d, hkv, hq = 500, 16, 16, 4, 16, 2, 4
    keys = bf16_bits(rng.standard_normal((hkv, L, d)).astype(np.float32))
    vals = bf16_bits(rng.standard_normal((hkv, L, d)).astype(np.float32))
    qs = bf16_bits(rng.standard_normal((6, hq, d)).astype(np.float32))
    pos = np.array([0, 40, 200, 333, 450, 499])
    pn, pc = O.Problem(keys, vals, L, hq, S, k, W, True), CPP.Problem(keys, vals, L, hq, S, k, W, True)
    a, b = pn.rows(qs, pos, scores=True), pc.rows(qs, pos, scores=True)
    assert np.array_equal(a["sel"], b["sel"]) and np.array_equal(a["n_attended"], b["n_attended"])
    assert np.abs(a["out"] - b["out"]).max() <= 1e-12
    given = np.tile(np.array([3, 3, -1, 99, 1, 0, 3, 2])[:k], (6, hq, 1))
    a, b = pn.rows(qs, pos, sel=given), pc.rows(qs, pos, sel=given)
    assert np.array_equal(a["n_attended"], b["n_attended"])
    assert np.abs(a["out"] - b["out"]).max() <= 1e-12
    d1, d2 = pn.rows(qs, pos, dense=True), pc.rows(qs, pos, dense=True)
    assert np.abs(d1["out"] - d2["out"]).max() <= 1e-12
