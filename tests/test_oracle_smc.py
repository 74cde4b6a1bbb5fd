"""Pins of the SMC-SD step oracle to facts fixed outside the oracle itself.

The step follows the page "Faster LLM Inference via Sequential Monte Carlo",
section 2: importance weights from the ratio of target to draft
probabilities, a bonus token per particle, and resampling when the effective
sample size falls low.  Pinned here by brute-force enumeration (the weights
make the draft-sampled estimator of any target expectation exact), by the
verify oracle (which has its own pins) for the bonus draw, by closed forms
of the effective sample size and by the defining count property and the
unbiasedness of systematic resampling.
"""

import itertools

import numpy as np
import scipy.special

import oracle
from oracle.smc import ess, log_weight_increment, smc_step, systematic


def _rng(s):
    return np.random.default_rng(1000 + s)


# --------------------------------------------------------------------------
# The importance weights
# --------------------------------------------------------------------------

def test_weights_make_draft_sampling_exact_by_enumeration():
    # For K drafted tokens x ~ prod_j q_j, E_q[exp(increment) f(x)] must equal
    # E_p[f(x)] for every f: enumerate all V^K sequences of a tiny
    # vocabulary, with q and p from scipy's softmax (not the oracle's).
    rng = _rng(1)
    V, K, T = 4, 3, 0.8
    lt = rng.normal(0, 2, size=(K, V))
    ld = lt + rng.normal(0, 1, size=(K, V))
    p = [scipy.special.softmax(lt[j] / T) for j in range(K)]
    q = [scipy.special.softmax(ld[j] / T) for j in range(K)]
    po = [oracle.softmax(lt[j], T)[0] for j in range(K)]
    qo = [oracle.softmax(ld[j], T)[0] for j in range(K)]
    f = rng.normal(size=(V,) * K)
    e_q, e_p, total = 0.0, 0.0, 0.0
    for x in itertools.product(range(V), repeat=K):
        qx = np.prod([q[j][x[j]] for j in range(K)])
        px = np.prod([p[j][x[j]] for j in range(K)])
        w = np.exp(log_weight_increment(po, qo, list(x)))
        total += qx * w
        e_q += qx * w * f[x]
        e_p += px * f[x]
    assert abs(total - 1.0) < 1e-12
    assert abs(e_q - e_p) < 1e-12


def test_identical_models_give_zero_increment_and_the_verify_bonus():
    # draft == target: every ratio is 1, so the increment is exactly 0, the
    # ESS stays N and the bonus equals the verify step's bonus (every draft
    # accepted, the same Philox counter at position K).
    rng = _rng(2)
    N, K, V, T = 6, 3, 50, 0.7
    t = rng.normal(0, 3, size=(N, K + 1, V)).astype(np.float32)
    d = t[:, :K].copy()
    x = rng.integers(0, V, size=(N, K))
    r = smc_step(t, d, x, np.zeros(N), T, 0.5, seed=77)
    assert np.all(r.increment == 0.0)
    assert r.ess == N and not r.resampled
    assert np.array_equal(r.ancestors, np.arange(N))
    v = oracle.verify(t, d, x, None, T, 1.0, seed=77)
    assert np.all(v.n_accepted == K)
    assert np.array_equal(r.bonus, v.tokens[:, K])


def test_increment_sign_and_scale():
    # one position, two tokens: log p(x) - log q(x) by hand
    lt = np.array([[0.0, np.log(3.0)], [0.0, 0.0]])  # p = (1/4, 3/4) at position 0
    ld = np.array([[np.log(3.0), 0.0]])               # q = (3/4, 1/4)
    r = smc_step(lt[None], ld[None], np.array([[1]]), np.zeros(1), 1.0, 0.0, seed=1)
    assert abs(r.increment[0] - np.log(3.0)) < 1e-15   # log(3/4) - log(1/4)
    r = smc_step(lt[None], ld[None], np.array([[0]]), np.array([0.5]), 1.0, 0.0, seed=1)
    assert abs(r.increment[0] + np.log(3.0)) < 1e-15
    assert abs(r.logw[0] - (0.5 - np.log(3.0))) < 1e-15


# --------------------------------------------------------------------------
# Effective sample size
# --------------------------------------------------------------------------

def test_ess_closed_forms():
    assert ess(np.zeros(7)) == 7.0
    assert ess(np.array([3.0, -np.inf, -np.inf])) == 1.0
    a, b = 0.2, 1.7
    want = (a + b) ** 2 / (a * a + b * b)
    assert abs(ess(np.log([a, b])) - want) < 1e-14
    lw = _rng(3).normal(size=20)
    assert abs(ess(lw) - ess(lw + 123.0)) < 1e-12
    assert ess(np.full(4, -np.inf)) == 0.0


# --------------------------------------------------------------------------
# Systematic resampling
# --------------------------------------------------------------------------

def test_systematic_count_property():
    # each particle is copied floor(N w_i) or ceil(N w_i) times; ancestors
    # are non-decreasing; zero-weight particles are never copied
    rng = _rng(4)
    N = 50
    lw = rng.normal(0, 1.5, size=N)
    lw[[3, 17]] = -np.inf
    w = np.exp(lw - lw.max())
    w /= w.sum()
    for u0 in (0.0, 0.123, 0.5, 0.999):
        a, _ = systematic(lw, u0)
        cnt = np.bincount(a, minlength=N)
        assert cnt.sum() == N
        assert np.all(cnt >= np.floor(N * w) - 0) and np.all(cnt <= np.ceil(N * w))
        assert np.all(np.diff(a) >= 0)
        assert cnt[3] == 0 and cnt[17] == 0


def test_systematic_equal_weights_is_identity():
    for u0 in (0.0, 0.3, 0.9999):
        a, _ = systematic(np.zeros(9), u0)
        assert np.array_equal(a, np.arange(9))


def test_systematic_is_unbiased_over_u0():
    # averaged over u0 uniform on [0, 1), particle i is copied N w_i times
    rng = _rng(5)
    N, M = 12, 4000
    lw = rng.normal(0, 1, size=N)
    w = np.exp(lw - lw.max())
    w /= w.sum()
    mean = np.zeros(N)
    for u0 in (np.arange(M) + 0.5) / M:
        a, _ = systematic(lw, u0)
        mean += np.bincount(a, minlength=N)
    mean /= M
    assert np.max(np.abs(mean - N * w)) < 2.0 / M


# --------------------------------------------------------------------------
# The step
# --------------------------------------------------------------------------

def _inputs(N, K, V, s):
    rng = _rng(s)
    t = rng.normal(0, 3, size=(N, K + 1, V)).astype(np.float32)
    d = (t[:, :K] + rng.normal(0, 1.5, size=(N, K, V))).astype(np.float32)
    x = rng.integers(0, V, size=(N, K))
    return t, d, x


def test_step_resampling_threshold():
    N, K, V = 16, 3, 40
    t, d, x = _inputs(N, K, V, 6)
    lw0 = _rng(7).normal(0, 0.5, size=N)
    keep = smc_step(t, d, x, lw0, 0.9, 0.0, seed=5)
    assert not keep.resampled and np.array_equal(keep.ancestors, np.arange(N))
    np.testing.assert_allclose(keep.logw, lw0 + keep.increment, rtol=0, atol=1e-15)
    assert 1.0 <= keep.ess <= N
    full = smc_step(t, d, x, lw0, 0.9, 1.0, seed=5)
    assert full.resampled and np.all(full.logw == 0.0)
    assert abs(full.ess - keep.ess) < 1e-12
    # the copies follow the weights the step computed
    a, _ = systematic(keep.logw, oracle.systematic_uniform(5))
    assert np.array_equal(full.ancestors, a)
    np.testing.assert_array_equal(full.bonus, keep.bonus)


def test_step_invalid_particles():
    N, K, V = 6, 2, 30
    t, d, x = _inputs(N, K, V, 8)
    x[1, 0] = V            # drafted id out of range
    t[2, 1, 5] = np.nan    # NaN in a needed target row
    d[3, 0, :] = -np.inf   # an all -inf draft row
    lw = np.zeros(N)
    lw[4] = np.nan         # unusable input weight
    r = smc_step(t, d, x, lw, 1.0, 1.0, seed=9)
    bad = [1, 2, 3, 4]
    assert np.all(r.bonus[bad] == -1)
    assert r.resampled
    assert not np.any(np.isin(r.ancestors, bad))
    none = smc_step(t, d, np.full((N, K), V), np.zeros(N), 1.0, 1.0, seed=9)
    assert none.ess == 0.0 and not none.resampled
    assert np.all(none.logw == -np.inf) and np.array_equal(none.ancestors, np.arange(N))
