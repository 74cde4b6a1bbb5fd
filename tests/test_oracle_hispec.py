"""Pins of the two-stage (hierarchical) verify oracle.

The page "HiSpec: Hierarchical Speculative Decoding for LLMs" (section 2)
claims the two-stage check draft -> intermediate -> final layer is lossless:
the output follows the final layer exactly.  Pinned here by that claim
(chi-square over many seeds on a tiny vocabulary, against the final layer's
softmax computed by scipy), and by the special cases where a layer pair is
identical and a stage must accept everything.
"""

import numpy as np
import scipy.special
import scipy.stats

import oracle
from oracle.hispec import hispec_verify


def _layers(B, K, V, s, scale=2.0):
    rng = np.random.default_rng(2000 + s)
    f = rng.normal(0, scale, size=(B, K + 2, V))
    i = f[:, : K + 1] + rng.normal(0, 1.0, size=(B, K + 1, V))
    d = i[:, :K] + rng.normal(0, 1.0, size=(B, K, V))
    x = rng.integers(0, V, size=(B, K))
    return f, i, d, x


def test_identical_intermediate_and_final_layers_accept_stage_one_output():
    f, i, d, x = _layers(6, 3, 40, 1)
    f[:, : 3 + 1] = i
    r = hispec_verify(f, i, d, x, None, 0.9, 1.0, seed=11)
    n1 = r.n_stage1
    assert np.all(r.n_accepted == n1 + 1)
    for b in range(6):
        assert list(r.tokens[b, : n1[b] + 1]) == list(r.stage1.tokens[b, : n1[b] + 1])


def test_identical_draft_and_intermediate_layers_pass_every_draft():
    f, i, d, x = _layers(6, 3, 40, 2)
    d[:] = i[:, :3]
    r = hispec_verify(f, i, d, x, None, 0.9, 1.0, seed=12)
    assert np.all(r.n_stage1 == 3)
    assert np.array_equal(r.stage1.tokens[:, :3], x)


def test_stage_two_uses_its_own_uniforms():
    # the two stages draw from different Philox streams
    assert oracle.uniforms(5, 3, 1, 0) != oracle.uniforms(5, 3, 1, 1)


def test_first_output_token_follows_the_final_layer():
    # [HS] section 2: lossless.  Drafts sampled from the draft layer, one
    # oracle call per seed; the first emitted token's frequencies must match
    # softmax(final layer, position 0 / T).
    V, K, T, runs = 4, 2, 1.0, 6000
    rng = np.random.default_rng(77)
    f = rng.normal(0, 1.5, size=(1, K + 2, V))
    i = f[:, : K + 1] + rng.normal(0, 1.0, size=(1, K + 1, V))
    d = i[:, :K] + rng.normal(0, 1.0, size=(1, K, V))
    qd = [scipy.special.softmax(d[0, j] / T) for j in range(K)]
    counts = np.zeros(V)
    for s in range(runs):
        x = np.array([[rng.choice(V, p=qd[j]) for j in range(K)]])
        r = hispec_verify(f, i, d, x, None, T, 1.0, seed=0x1000 + s)
        counts[r.tokens[0, 0]] += 1
    want = scipy.special.softmax(f[0, 0] / T) * runs
    chi2, p = scipy.stats.chisquare(counts, want)
    assert p > 1e-4, (counts, want, p)
