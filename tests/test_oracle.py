"""Pins of the float64 oracle to facts fixed outside the oracle itself.

Each test names what pins it: a worked example derived by hand from the
equations on the page "Speculative Decoding للمحترف: ضاعف سرعة Llama 70B لـ 2.4x
بدون فقد token واحد" (section "التعريف الرياضي من Leviathan et al."), closed
forms that follow from those equations, brute-force enumeration on tiny
vocabularies of the exactness claim made in the same section, special cases
that reduce to textbook routines, and statistics.
"""

import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle
from oracle.verify import decide_row, inverse_cdf, nucleus, ratio, residual_weights, softmax

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *rest = line.split()
            vals[key] = np.array([float(Fraction(r)) for r in rest])
    return vals


# --------------------------------------------------------------------------
# Hand-derived worked example (tests/golden/hand_v3.txt)
# --------------------------------------------------------------------------

def test_golden_hand_example():
    g = _golden("hand_v3.txt")
    lp, lq = np.log(g["p_target"]), np.log(g["p_draft"])
    p, _, _ = softmax(lp, 1.0)
    q, _, _ = softmax(lq, 1.0)
    np.testing.assert_allclose(p, g["p_target"], rtol=1e-15)
    np.testing.assert_allclose(q, g["p_draft"], rtol=1e-15)
    alpha = np.array([min(1.0, ratio(p[x], q[x])) for x in range(3)])
    np.testing.assert_allclose(alpha, g["alpha"], rtol=1e-14)
    assert abs(np.sum(np.minimum(p, q)) - g["beta"][0]) < 1e-15
    w = residual_weights(p, q)
    np.testing.assert_allclose(w / w.sum(), g["residual"], atol=1e-15)
    assert abs(w.sum() - g["Z"][0]) < 1e-15
    pf, kept, _ = nucleus(p, 0.8)
    np.testing.assert_allclose(pf, g["topp_0.8_target"], atol=1e-15)
    assert abs(kept - g["topp_0.8_kept"][0]) < 1e-15


def test_golden_hand_example_accept_thresholds():
    # alpha(1) = 2/3: u just below accepts, u just above rejects (u < alpha).
    g = _golden("hand_v3.txt")
    p, q = g["p_target"], g["p_draft"]
    r = ratio(p[1], q[1])
    assert oracle.accept(2 / 3 - 1e-9, r)
    assert not oracle.accept(2 / 3 + 1e-9, r)
    # token 0 has alpha 1: accepted for every u in [0, 1)
    assert oracle.accept(1 - 2 ** -24, ratio(p[0], q[0]))


# --------------------------------------------------------------------------
# Library routine and closed forms
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T", [0.3, 0.7, 1.0, 2.5])
def test_softmax_matches_scipy(T):
    rng = np.random.default_rng(1)
    l = rng.normal(0, 3, size=5000)
    p, m, s = softmax(l, T)
    np.testing.assert_allclose(p, scipy.special.softmax(l / T), rtol=1e-13, atol=1e-300)
    assert m == l.max()
    np.testing.assert_allclose(s, np.sum(np.exp((l - l.max()) / T)), rtol=1e-15)


def test_softmax_masked_vocab():
    l = np.array([0.0, -np.inf, 1.0, -np.inf])
    p, _, _ = softmax(l, 0.7)
    assert p[1] == 0.0 and p[3] == 0.0
    np.testing.assert_allclose(p[[0, 2]], scipy.special.softmax(np.array([0.0, 1.0]) / 0.7), rtol=1e-15)


def _rand_dist(rng, V, scale=2.0):
    return softmax(rng.normal(0, scale, size=V), 1.0)[0]


@pytest.mark.parametrize("seed", range(5))
def test_residual_mass_is_total_variation(seed):
    # Z = sum max(0, p - q) = 1 - sum min(p, q) = 1/2 |p - q|_1, and the
    # normalised residual sums to one.
    rng = np.random.default_rng(seed)
    p, q = _rand_dist(rng, 50), _rand_dist(rng, 50)
    w = residual_weights(p, q)
    z = w.sum()
    assert abs(z - (1 - np.minimum(p, q).sum())) < 1e-14
    assert abs(z - 0.5 * np.abs(p - q).sum()) < 1e-14
    assert abs((w / z).sum() - 1.0) < 1e-14


# --------------------------------------------------------------------------
# Brute force: the exactness claim, on tiny vocabularies
# --------------------------------------------------------------------------

GRID = 2 ** 14


def _acc_vec(u, r):
    return float(np.mean(np.array([oracle.accept(float(ui), r) for ui in u])))


def _sample_law(w):
    """Law of the oracle's inverse_cdf under a uniform u grid."""
    u = (np.arange(GRID) + 0.5) / GRID
    ys = np.array([inverse_cdf(w, float(ui))[0] for ui in u])
    return np.bincount(ys, minlength=len(w)) / GRID


@pytest.mark.parametrize("V,topp,seed", [(3, 1.0, 0), (5, 1.0, 1), (6, 1.0, 2), (5, 0.8, 3), (6, 0.6, 4)])
def test_bruteforce_emitted_token_law_equals_target(V, topp, seed):
    """P(token emitted at a position = v | the position is reached) = p(v).

    Enumerates the drafted id x under q and sweeps both uniforms over a grid,
    calling the oracle's own accept and resample steps.  The claim that this
    equals the target's law is the section "التعريف الرياضي" exactness claim.
    """
    rng = np.random.default_rng(seed)
    p = _rand_dist(rng, V)
    q = _rand_dist(rng, V)
    if topp < 1.0:
        p = nucleus(p, topp)[0]
        q = nucleus(q, topp)[0]
    law = np.zeros(V)
    w = residual_weights(p, q)
    res_law = _sample_law(w) if w.sum() > 0 else np.zeros(V)
    u = (np.arange(GRID) + 0.5) / GRID
    for x in range(V):
        if q[x] == 0.0:
            continue
        a = _acc_vec(u, ratio(p[x], q[x]))
        law[x] += q[x] * a
        law += q[x] * (1 - a) * res_law
    np.testing.assert_allclose(law, p, atol=4 * V / GRID)


def test_bruteforce_analytic_identity():
    # With the exact accept probability min(1, r) and the exact residual law
    # w/Z the identity holds to rounding: min(q, p) + (1 - beta) w/Z = p.
    rng = np.random.default_rng(7)
    for V in (2, 4, 6):
        for _ in range(20):
            p, q = _rand_dist(rng, V, 3.0), _rand_dist(rng, V, 3.0)
            w = residual_weights(p, q)
            beta = sum(q[x] * min(1.0, ratio(p[x], q[x])) for x in range(V))
            law = np.array([q[v] * min(1.0, ratio(p[v], q[v])) for v in range(V)]) + (1 - beta) * w / w.sum()
            np.testing.assert_allclose(law, p, atol=1e-14)


def test_row_acceptance_count_law():
    """P(n = m) = prod_{i<m} beta_i * (1 - beta_m) and P(n = L) = prod beta_i,
    with beta_j = sum_x min(p_j, q_j) (closed form from the section
    "التعريف الرياضي" equation for alpha).  Monte Carlo over drafted ids x_j ~ q_j
    and independent uniforms, through the full-row scan of decide_row."""
    rng = np.random.default_rng(11)
    V, L = 4, 3
    p = [_rand_dist(rng, V) for _ in range(L + 1)]
    q = [_rand_dist(rng, V) for _ in range(L)]
    beta = [float(np.minimum(p[j], q[j]).sum()) for j in range(L)]
    N = 20000
    counts = np.zeros(L + 1)
    for _ in range(N):
        x = [int(rng.choice(V, p=q[j])) for j in range(L)]
        d = decide_row(p, q, x, rng.random(L + 1), rng.random(L + 1))
        counts[d.n] += 1
        assert d.tokens[: d.n] == x[: d.n] and len(d.tokens) == d.n + 1
    expect = []
    reach = 1.0
    for m in range(L):
        expect.append(reach * (1 - beta[m]))
        reach *= beta[m]
    expect.append(reach)
    assert scipy.stats.chisquare(counts, N * np.array(expect)).pvalue > 1e-3


# --------------------------------------------------------------------------
# Special cases
# --------------------------------------------------------------------------

def _row(tl, dl, x, T=1.0, top_p=1.0, seed=0, L=None):
    tl = np.asarray(tl, float)[None]
    dl = np.asarray(dl, float)[None]
    x = np.asarray(x, np.int64)[None]
    dlen = None if L is None else np.array([L])
    return oracle.verify(tl, dl, x, dlen, T, top_p, seed)


def test_identical_models_accept_everything():
    rng = np.random.default_rng(3)
    K, V = 4, 30
    tl = rng.normal(0, 3, size=(K + 1, V))
    for seed in range(50):
        x = rng.integers(0, V, size=K)
        r = _row(tl, tl[:K], x, T=0.7, seed=seed)
        assert r.n_accepted[0] == K
        assert list(r.tokens[0, :K]) == list(x)


def test_no_drafts_is_textbook_inverse_cdf():
    # L = 0: the row reduces to one inverse-CDF draw from the target softmax:
    # the token is the smallest v with F(v) > u (F the running sum).
    rng = np.random.default_rng(5)
    V = 40
    tl = rng.normal(0, 2, size=(3, V))
    dl = rng.normal(0, 2, size=(2, V))
    p = scipy.special.softmax(tl[0] / 0.9)
    for seed in range(40):
        r = _row(tl, dl, [0, 0], T=0.9, seed=seed, L=0)
        u = oracle.uniforms(seed, 0, 0)[1]
        F, v = 0.0, 0
        while True:
            F += p[v]
            if F > u * p.sum():
                break
            v += 1
        assert r.n_accepted[0] == 0
        assert r.tokens[0, 0] == v


def test_disjoint_supports_reject_first():
    V = 10
    tl = np.full((3, V), -np.inf)
    dl = np.full((2, V), -np.inf)
    tl[:, :5] = np.random.default_rng(0).normal(size=(3, 5))
    dl[:, 5:] = np.random.default_rng(1).normal(size=(2, 5))
    for seed in range(30):
        r = _row(tl, dl, [7, 8], seed=seed)
        assert r.n_accepted[0] == 0
        assert 0 <= r.tokens[0, 0] < 5


def test_one_hot_target_emits_argmax():
    V = 20
    tl = np.zeros((3, V))
    tl[:, 13] = 250.0
    dl = np.zeros((2, V))
    for seed in range(30):
        r = _row(tl, dl, [4, 5], seed=seed)
        assert r.n_accepted[0] == 0
        assert r.tokens[0, 0] == 13


def test_bonus_comes_from_last_target_position():
    V = 12
    rng = np.random.default_rng(2)
    tl = rng.normal(size=(4, V))
    tl[3] = -50.0
    tl[3, 9] = 50.0  # one-hot at position L = 3
    for seed in range(20):
        r = _row(tl, tl[:3], [1, 2, 3], seed=seed)
        assert r.n_accepted[0] == 3
        assert list(r.tokens[0]) == [1, 2, 3, 9]


def test_invalid_rows():
    V = 8
    tl = np.zeros((2, 3, V))
    dl = np.zeros((2, 2, V))
    x = np.zeros((2, 2), np.int64)
    # NaN in a needed row, and +inf
    t1 = tl.copy(); t1[0, 1, 3] = np.nan; t1[1, 0, 0] = np.inf
    r = oracle.verify(t1, dl, x, None, 1.0, 1.0, 0)
    assert list(r.n_accepted) == [-1, -1] and np.all(r.tokens == -1)
    # NaN in a position past L is never read
    t2 = tl.copy(); t2[0, 2, :] = np.nan
    d2 = dl.copy(); d2[0, 1, :] = np.nan
    r = oracle.verify(t2, d2, x, np.array([1, 2]), 1.0, 1.0, 0)
    assert r.n_accepted[0] >= 0 and r.n_accepted[1] >= 0
    # all -inf, bad length, bad id
    t3 = tl.copy(); t3[0, 0, :] = -np.inf
    r = oracle.verify(t3, dl, x, np.array([0, 3]), 1.0, 1.0, 0)
    assert list(r.n_accepted) == [-1, -1]
    x4 = x.copy(); x4[1, 1] = V
    r = oracle.verify(tl, dl, x4, np.array([2, 2]), 1.0, 1.0, 0)
    assert r.n_accepted[0] >= 0 and r.n_accepted[1] == -1
    r = oracle.verify(tl, dl, x4, np.array([2, 1]), 1.0, 1.0, 0)
    assert r.n_accepted[1] >= 0  # the bad id sits past L


# --------------------------------------------------------------------------
# Nucleus: the sorting definition against two other formulations
# --------------------------------------------------------------------------

def _nucleus_greedy(p, top_p):
    """Repeatedly take the most probable remaining token (lowest id on ties)
    until the taken mass reaches top_p."""
    left = list(range(len(p)))
    taken, mass = [], 0.0
    while left and mass < top_p:
        best = max(left, key=lambda i: (p[i], -i))
        left.remove(best)
        taken.append(best)
        mass += p[best]
    return sorted(taken)


def _nucleus_threshold(l, p, top_p):
    """Value threshold on the logit plus ties kept by lowest id."""
    order_vals = np.unique(l)[::-1]
    above = 0.0
    for tau in order_vals:
        tied = np.nonzero(l == tau)[0]
        pt = p[tied[0]]
        if above + len(tied) * pt >= top_p or tau == order_vals[-1]:
            r = 0
            acc = above
            while r < len(tied) and acc < top_p:
                acc += pt
                r += 1
            keep = np.nonzero(l > tau)[0].tolist() + tied[: max(r, 1)].tolist()
            return sorted(keep)
        above += len(tied) * pt
    return list(range(len(l)))


@pytest.mark.parametrize("seed", range(12))
def test_nucleus_formulations_agree(seed):
    rng = np.random.default_rng(seed)
    V = 60
    # bf16-like coarse logits so that ties are common
    l = np.round(rng.normal(0, 2, size=V) * 4) / 4
    top_p = float(np.float32(rng.uniform(0.3, 0.97)))
    p = softmax(l, 0.7)[0]
    pf, kept, _ = nucleus(p, top_p)
    ids = sorted(np.nonzero(pf > 0)[0].tolist())
    assert ids == _nucleus_greedy(p, top_p)
    assert ids == _nucleus_threshold(l, p, top_p)
    assert abs(pf.sum() - 1) < 1e-14
    assert abs(kept - p[ids].sum()) < 1e-14


def test_nucleus_tie_group_split_by_id():
    # four equal tokens of mass 1/4: top_p 0.5 keeps exactly ids 0 and 1
    p = np.full(4, 0.25)
    pf, kept, margin = nucleus(p, 0.5)
    assert list(np.nonzero(pf)[0]) == [0, 1]
    assert kept == 0.5 and margin == 0.0


# --------------------------------------------------------------------------
# Statistics over Philox seeds (P(first token) = p_0; mean acceptance)
# --------------------------------------------------------------------------

@pytest.mark.slow
def test_statistics_first_token_and_acceptance():
    rng = np.random.default_rng(21)
    V, K, T = 8, 3, 0.8
    tl = rng.normal(0, 1.5, size=(K + 1, V))
    dl = tl[:K] + rng.normal(0, 1.0, size=(K, V))
    p = [scipy.special.softmax(tl[j] / T) for j in range(K + 1)]
    q = [scipy.special.softmax(dl[j] / T) for j in range(K)]
    beta = [np.minimum(p[j], q[j]).sum() for j in range(K)]
    N = 6000
    first = np.zeros(V)
    acc0 = 0
    n_sum = 0
    xr = np.random.default_rng(99)
    for s in range(N):
        x = [xr.choice(V, p=q[j]) for j in range(K)]
        r = _row(tl, dl, x, T=T, seed=0xABCD00000000 + s)
        first[r.tokens[0, 0]] += 1
        acc0 += r.n_accepted[0] >= 1
        n_sum += r.n_accepted[0]
    chi2 = scipy.stats.chisquare(first, N * p[0])
    assert chi2.pvalue > 1e-3
    sd = np.sqrt(beta[0] * (1 - beta[0]) / N)
    assert abs(acc0 / N - beta[0]) < 4 * sd
    en = sum(np.prod(beta[:m]) for m in range(1, K + 1))
    assert abs(n_sum / N - en) < 0.06


def test_probe_values():
    rng = np.random.default_rng(4)
    V, K, T = 100, 2, 0.7
    tl = rng.normal(0, 3, size=(1, K + 1, V))
    dl = tl[:, :K] + rng.normal(0, 1, size=(1, K, V))
    x = np.array([[3, 4]])
    r = oracle.verify(tl, dl, x, None, T, 1.0, 77)
    T32 = float(np.float32(T))
    for j in range(r.n_accepted[0] + 1 if r.n_accepted[0] < K else K):
        m = tl[0, j].max()
        assert r.probe_pos[0, j, 0] == m
        np.testing.assert_allclose(r.probe_pos[0, j, 1], np.exp((tl[0, j] - m) / T32).sum(), rtol=1e-15)
    assert r.probe_row[0, 3] == r.n_accepted[0]


def test_inverse_cdf_boundaries_are_strict():
    # smallest id with C[id] > t: a t sitting exactly on a running sum belongs
    # to the next token, and zero-weight ids are never drawn
    assert inverse_cdf(np.array([0.0, 0.5, 0.5]), 0.0)[0] == 1
    assert inverse_cdf(np.array([0.25, 0.25, 0.5]), 0.25)[0] == 1
    assert inverse_cdf(np.array([0.25, 0.25, 0.5]), 0.5)[0] == 2
    assert inverse_cdf(np.array([0.5, 0.0, 0.5]), 0.5)[0] == 2
    assert inverse_cdf(np.array([0.5, 0.5, 0.0]), 1 - 2 ** -24)[0] == 1


@pytest.mark.parametrize("seed", range(4))
def test_nucleus_large_tie_groups(seed):
    # few distinct logit values over many ids: the cut lands inside a tie
    # group and must keep its lowest ids (what a stable sort keeps)
    rng = np.random.default_rng(100 + seed)
    V = 3000
    l = rng.integers(0, 6, size=V).astype(float)
    p = softmax(l, 1.0)[0]
    top_p = float(np.float32(rng.uniform(0.2, 0.9)))
    pf, _, _ = nucleus(p, top_p)
    ids = sorted(np.nonzero(pf > 0)[0].tolist())
    assert ids == _nucleus_threshold(l, p, top_p)
