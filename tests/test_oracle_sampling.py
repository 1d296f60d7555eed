"""Pins of the sampling oracle against what the pages and the mathematics fix.

Closed forms: with a stratified set of draws u_j = (j + 1/2) / N, the
frequencies of the sampled tokens equal the probabilities of the filtered,
renormalised softmax within 1/N per token (an inverse CDF over a partition of
[0, 1)); those probabilities are computed here independently with math.exp in
Python loops.  Brute force: top-k and top-p sets by exhaustive search on small
vocabularies.  Worked rule: the repetition penalty of "02 GPT 架构" §8.4.  A
mutation test plants plausible mistakes in the oracle and checks that these
pins catch every one.
"""
import itertools
import math

import numpy as np
import pytest

from oracle import sampling_oracle as S

N = 20000
U = (np.arange(N) + 0.5) / N


def _freq(z, seen, t, k, p, a, n=N):
    u = (np.arange(n) + 0.5) / n
    toks = [S.sample_row(z, seen, t, k, p, a, float(x)) for x in u]
    return np.bincount(toks, minlength=len(z)) / n


def _softmax_py(vals):
    m = max(vals)
    e = [math.exp(v - m) for v in vals]
    s = sum(e)
    return [x / s for x in e]


def _check_freq(z, seen, t, k, p, a, expect):
    f = _freq(z, seen, t, k, p, a)
    assert np.all(np.abs(f - np.asarray(expect)) <= 2.0 / N + 1e-12), (f, expect)


# --------------------------------------------------------------------------
# Temperature ("预训练一个 Mini GPT" 第7步; "02 GPT 架构" §8.1; "GPT-1学习笔记" §6.2)
# --------------------------------------------------------------------------
Z7 = np.array([1.5, -0.5, 0.25, 2.0, 0.0, -1.25, 0.75], dtype=np.float32)


@pytest.mark.parametrize("t", [1.0, 0.5, 1.5, 0.8])
def test_temperature_frequencies_match_softmax(t):
    expect = _softmax_py([float(v) / t for v in Z7])
    _check_freq(Z7, None, t, 0, 1.0, 1.0, expect)


def test_temperature_zero_is_greedy_lowest_index():
    z = np.array([0.5, 2.0, -1.0, 2.0], dtype=np.float32)
    for u in (0.0, 0.3, 0.999):
        assert S.sample_row(z, None, 0.0, 0, 1.0, 1.0, u) == 1
    # low temperature concentrates on the maximum
    f = _freq(Z7, None, 0.05, 0, 1.0, 1.0, n=2000)
    assert f[3] > 0.99


# --------------------------------------------------------------------------
# Top-k ("02 GPT 架构" §8.2; "GPT-1学习笔记" §6.2; "第 25 章" §25.7)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("k", [1, 2, 3, 6])
def test_top_k_renormalises_the_k_largest(k):
    t = 0.9
    vals = [float(v) / t for v in Z7]
    top = sorted(range(len(vals)), key=lambda i: (-vals[i], i))[:k]
    pk = _softmax_py([vals[i] for i in top])
    expect = [0.0] * len(vals)
    for i, q in zip(top, pk):
        expect[i] = q
    _check_freq(Z7, None, t, k, 1.0, 1.0, expect)


def test_top_k_ties_keep_lowest_indices():
    z = np.array([1.0, 3.0, 3.0, 0.0, 3.0], dtype=np.float32)
    cand, _ = S.filtered(z, None, 1.0, 2, 1.0)
    assert list(cand) == [1, 2]
    cand, _ = S.filtered(z, None, 1.0, 4, 1.0)
    assert list(cand) == [1, 2, 4, 0]


def test_top_k_brute_force_small_vocab():
    rng = np.random.default_rng(3)
    for _ in range(20):
        z = rng.integers(-3, 4, 6).astype(np.float32)   # many ties
        for k in range(1, 6):
            cand, _ = S.filtered(z, None, 1.0, k, 1.0)
            # every kept token is at least as large as every dropped one, and
            # among equal values the kept ones have lower indices
            kept = set(int(i) for i in cand)
            assert len(kept) == k
            for i, j in itertools.product(kept, set(range(6)) - kept):
                assert z[i] > z[j] or (z[i] == z[j] and i < j)


# --------------------------------------------------------------------------
# Top-p ("02 GPT 架构" §8.3; "GPT-1学习笔记" §6.2)
# --------------------------------------------------------------------------
def test_top_p_worked_probabilities():
    probs = [0.5, 0.3, 0.15, 0.05]
    z = np.log(np.array(probs)).astype(np.float32)
    # 0.5 < 0.75 <= 0.8: the two most probable tokens, renormalised
    _check_freq(z, None, 1.0, 0, 0.75, 1.0, [0.5 / 0.8, 0.3 / 0.8, 0.0, 0.0])
    # 0.8 < 0.9 <= 0.95: three tokens
    _check_freq(z, None, 1.0, 0, 0.9, 1.0, [0.5 / 0.95, 0.3 / 0.95, 0.15 / 0.95, 0.0])
    # a tiny p keeps the most probable token only
    for u in (0.0, 0.5, 0.99):
        assert S.sample_row(z, None, 1.0, 0, 1e-9, 1.0, u) == 0
    # equal logits give exactly equal masses: with p = 1/2 the nucleus of four
    # is the first two (a prefix that reaches p exactly is enough)
    _check_freq(np.zeros(4, np.float32), None, 1.0, 0, 0.5, 1.0, [0.5, 0.5, 0.0, 0.0])


def test_top_p_brute_force_smallest_set():
    rng = np.random.default_rng(5)
    for _ in range(30):
        z = rng.normal(0, 1.5, 6).astype(np.float32)
        p = float(rng.uniform(0.05, 0.99))
        cand, w = S.filtered(z, None, 1.0, 0, p)
        probs = _softmax_py([float(v) for v in z])
        # the smallest number of tokens whose total probability can reach p
        best = min(n for n in range(1, 7)
                   if any(sum(probs[i] for i in c) >= p - 1e-12 for c in itertools.combinations(range(6), n)))
        assert len(cand) == best
        assert sum(probs[i] for i in cand) >= p - 1e-12
        # the kept mass, float64 weights against Python math.exp sums
        assert abs(w.sum() / sum(math.exp(float(v) - float(z.max())) for v in z) - sum(probs[i] for i in cand)) < 1e-12


def test_top_p_applies_to_the_top_k_distribution():
    probs = [0.4, 0.3, 0.2, 0.1]
    z = np.log(np.array(probs)).astype(np.float32)
    # after top-k = 3 the masses are 4/9, 3/9, 2/9: p = 0.75 is reached by
    # 4/9 + 3/9 = 7/9 (on the whole distribution it would take three tokens,
    # 0.4 + 0.3 < 0.75)
    _check_freq(z, None, 1.0, 3, 0.75, 1.0, [4 / 7, 3 / 7, 0.0, 0.0])


# --------------------------------------------------------------------------
# Repetition penalty ("02 GPT 架构" §8.4)
# --------------------------------------------------------------------------
def test_repetition_penalty_rule():
    z = np.array([2.0, -2.0, 1.0, 0.0, -1.0], dtype=np.float32)
    seen = np.array([True, True, False, True, False])
    np.testing.assert_array_equal(S.penalize(z, seen, 2.0), np.array([1.0, -4.0, 1.0, 0.0, -1.0], np.float32))
    np.testing.assert_array_equal(S.penalize(z, seen, 1.0), z)


def test_repetition_penalty_frequencies():
    seen = np.array([False, False, False, True, False, True, False])
    a = 1.3
    pen = [float(v) / a if (s and v > 0) else (float(v) * a if (s and v < 0) else float(v)) for v, s in zip(Z7, seen)]
    _check_freq(Z7, seen, 1.0, 0, 1.0, a, _softmax_py(pen))
    # the greedy choice sees the penalised logits too: 2.0 / 1.3 > 1.5 > 2.0 / 1.5
    assert S.sample_row(Z7, seen, 0.0, 0, 1.0, a, 0.5) == 3
    assert S.sample_row(Z7, seen, 0.0, 0, 1.0, 1.5, 0.5) == 0


def test_draw_is_inverse_cdf_in_candidate_order():
    z = np.array([0.0, 1.0, 1.0, -1.0], dtype=np.float32)   # candidate order 1, 2, 0, 3
    e = [math.exp(v - 1.0) for v in (1.0, 1.0, 0.0, -1.0)]
    c = np.cumsum(e) / sum(e)
    assert S.sample_row(z, None, 1.0, 0, 1.0, 1.0, 0.0) == 1
    assert S.sample_row(z, None, 1.0, 0, 1.0, 1.0, float(c[0]) + 1e-6) == 2
    assert S.sample_row(z, None, 1.0, 0, 1.0, 1.0, float(c[1]) + 1e-6) == 0
    assert S.sample_row(z, None, 1.0, 0, 1.0, 1.0, 0.999999) == 3


# --------------------------------------------------------------------------
# Planted mistakes
# --------------------------------------------------------------------------
_PINS = [lambda: test_temperature_frequencies_match_softmax(0.5), test_temperature_zero_is_greedy_lowest_index,
         lambda: test_top_k_renormalises_the_k_largest(3), test_top_k_ties_keep_lowest_indices,
         test_top_p_worked_probabilities, test_top_p_brute_force_smallest_set,
         test_top_p_applies_to_the_top_k_distribution, test_repetition_penalty_rule,
         test_repetition_penalty_frequencies, test_draw_is_inverse_cdf_in_candidate_order]


def _pins_pass():
    for c in _PINS:
        try:
            c()
        except (AssertionError, ValueError, IndexError):
            return False
    return True


def test_pins_catch_planted_mistakes(monkeypatch):
    assert _pins_pass()
    orig_filtered = S.filtered

    def penalty_sign_flipped(z, seen, alpha):
        z = np.asarray(z, dtype=np.float64)
        if seen is None or alpha == 1.0:
            return z.copy()
        return np.where(seen, z / alpha, z)   # negatives divided too

    def order_ties_by_descending_index(w):
        return np.lexsort((-np.arange(w.size), -w.astype(np.float64)))

    def top_p_one_too_many(z, seen, t, k, p, alpha=1.0):
        cand, w = orig_filtered(z, seen, t, k, 1.0, alpha)
        if p < 1.0:
            cum = np.cumsum(w)
            n = int(np.searchsorted(cum, p * cum[-1], side="right")) + 1   # first prefix with mass > p Z
            cand, w = cand[:n], w[:n]
        return cand, w

    def top_p_drops_the_crossing_token(z, seen, t, k, p, alpha=1.0):
        cand, w = orig_filtered(z, seen, t, k, 1.0, alpha)
        if p < 1.0:
            cum = np.cumsum(w)
            n = max(1, int(np.searchsorted(cum, p * cum[-1], side="left")))
            cand, w = cand[:n], w[:n]
        return cand, w

    def top_p_before_top_k(z, seen, t, k, p, alpha=1.0):
        cand, w = orig_filtered(z, seen, t, 0, p, alpha)
        return (cand[:k], w[:k]) if 0 < k < len(cand) else (cand, w)

    def temperature_multiplied(z, seen, t, k, p, alpha=1.0):
        return orig_filtered(z, seen, 1.0 / t if t > 0 else t, k, p, alpha)

    mutants = [("penalize", penalty_sign_flipped), ("candidate_order", order_ties_by_descending_index),
               ("filtered", top_p_one_too_many), ("filtered", top_p_drops_the_crossing_token),
               ("filtered", top_p_before_top_k),
               ("filtered", temperature_multiplied)]
    for name, fn in mutants:
        with monkeypatch.context() as m:
            m.setattr(S, name, fn)
            assert not _pins_pass(), f"planted mistake in {name} ({fn.__name__}) went unnoticed"
