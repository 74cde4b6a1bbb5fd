"""Pins of the greedy-verify oracle.

Greedy verification is the temperature -> 0 limit of the verify step on the
page "Speculative Decoding للمحترف" (section "المفهوم بالتقريب"): pinned against
the separately pinned stochastic oracle at a tiny temperature on logits whose
maxima are well separated, against brute-force selection for the top-k of
the LogitSpec page (section 2), and on hand-made tie cases.
"""

import numpy as np

import oracle
from oracle.greedy import argmax_lowest, greedy_verify, top_k_after_first


def test_ties_go_to_the_lower_id():
    assert argmax_lowest([1.0, 3.0, 3.0, 2.0]) == 1
    assert argmax_lowest([-np.inf, -1.0, -1.0]) == 1
    assert list(top_k_after_first([5.0, 5.0, 2.0, 5.0, 7.0], 3)) == [0, 1, 3]
    assert list(top_k_after_first([1.0, 2.0], 4)) == [0, -1, -1, -1]


def test_top_k_matches_repeated_selection():
    # brute force: pick the max (lowest id among ties) k+1 times, removing it
    rng = np.random.default_rng(5)
    for _ in range(20):
        l = np.round(rng.normal(0, 2, size=300) * 4) / 4   # many ties
        k = int(rng.integers(1, 70))
        rest = list(range(l.size))
        picks = []
        for _ in range(min(k + 1, l.size)):
            best = min(rest, key=lambda i: (-l[i], i))
            picks.append(best)
            rest.remove(best)
        want = (picks[1:] + [-1] * k)[:k]
        assert list(top_k_after_first(l, k)) == want


def test_greedy_is_the_cold_limit_of_the_verify_step():
    # at T = 1e-3 with maxima at least 0.5 apart both softmaxes put all but
    # ~e^-500 of their mass on their argmax, and a draft sampled from the
    # draft's softmax is its argmax: the stochastic oracle's accept scan and
    # emitted tokens must equal the greedy ones
    rng = np.random.default_rng(6)
    B, K, V = 40, 4, 50
    t = rng.normal(0, 1, size=(B, K + 1, V))
    d = rng.normal(0, 1, size=(B, K, V))
    am = rng.integers(0, V, size=(B, K + 1))
    ad = np.where(rng.random((B, K)) < 0.7, am[:, :K], rng.integers(0, V, size=(B, K)))
    for b in range(B):
        for j in range(K + 1):
            t[b, j, am[b, j]] = t[b, j].max() + 0.5 + rng.random()
        for j in range(K):
            d[b, j, ad[b, j]] = d[b, j].max() + 0.5 + rng.random()
    x = ad
    g = greedy_verify(t, x, None, 3)
    s = oracle.verify(t, d, x, None, 1e-3, 1.0, seed=3)
    assert np.array_equal(g.n_accepted, s.n_accepted)
    assert np.array_equal(g.tokens, s.tokens)
    assert 0 < np.mean(g.n_accepted) < K


def test_invalid_rows_and_lengths():
    rng = np.random.default_rng(7)
    t = rng.normal(size=(4, 3, 20))
    x = rng.integers(0, 20, size=(4, 2))
    x[1, 0] = 25
    t[2, 1, 3] = np.nan
    t[3, 2, 0] = np.nan   # beyond L = 1 for row 3: not read
    g = greedy_verify(t, x, [2, 2, 2, 1], 5)
    assert list(g.n_accepted[[1, 2]]) == [-1, -1]
    assert np.all(g.topk[[1, 2]] == -1)
    assert g.n_accepted[3] >= 0 and g.n_accepted[0] >= 0
