"""Pins of the oracle's forced branches, which the GPU parity check follows
when the library decides a near-boundary test or nucleus cut the other way
(finite-precision reading of the exactness claim on the page "Speculative
Decoding للمحترف: ضاعف سرعة Llama 70B لـ 2.4x بدون فقد token واحد", section
"التعريف الرياضي من Leviathan et al.").

Checked against facts outside the forced code path: forcing every decision
to the outcome it has anyway changes nothing; a nucleus prefix of a given
count is that many tokens in (probability descending, id ascending) order,
found here by a plain sort of (-p, id) pairs; a forced rejection emits a
token of positive residual weight whose interval, in scipy's softmax,
holds u * Z (from p' itself when the filtered rows leave no residual).
"""

import numpy as np
import pytest
import scipy.special

import oracle
from oracle.philox import uniforms
from oracle.verify import nucleus, nucleus_neighbours
from rejection_sampling_verifier_amd import workloads as W


def _prefix_by_sort(p, k):
    order = sorted(range(len(p)), key=lambda i: (-p[i], i))
    return order[:k]


@pytest.mark.parametrize("seed", range(5))
def test_nucleus_keep_counts_match_a_plain_sort(seed):
    rng = np.random.default_rng(seed)
    p = scipy.special.softmax(np.round(rng.standard_normal(40) * 2, 1))  # ties from the rounding
    _, kept0, _ = nucleus(p, 0.7)
    k, (prev, mid, nxt) = nucleus_neighbours(p, 0.7)
    assert mid == kept0
    # the defined cut: the shortest prefix of the sorted order reaching top_p
    srt = sorted(p, reverse=True)
    assert sum(srt[:k]) >= 0.7 - 1e-12 and sum(srt[:k - 1]) < 0.7 + 1e-12
    for count, kept_ref in ((k - 1, prev), (k, mid), (k + 1, nxt)):
        if not 1 <= count <= p.size:
            assert np.isnan(kept_ref)  # no such prefix
            continue
        out, kept, _ = nucleus(p, 0.7, keep=count)
        ids = _prefix_by_sort(p, count)
        assert set(np.nonzero(out)[0]) == set(ids)
        assert kept == pytest.approx(sum(p[i] for i in ids), rel=1e-14)
        assert kept == pytest.approx(kept_ref, rel=1e-14)
        assert out.sum() == pytest.approx(1.0, rel=1e-14)


def _inputs():
    return W.synthetic(12, 4, 60, dtype="f32", temperature=0.8, top_p=0.8, sigma=1.5, seed=9, gen_seed=9)


def _run(inp, **kw):
    return oracle.verify(inp.target, inp.draft, inp.draft_tokens, inp.draft_len, inp.temperature, inp.top_p,
                         inp.seed, **kw)


def test_forcing_natural_outcomes_changes_nothing():
    inp = _inputs()
    res = _run(inp)
    forced, cuts = {}, {}
    for b in range(inp.B):
        forced[b] = {j: bool(u < r) for j, (u, r) in enumerate(res.accepts[b])}
        cuts[b] = {key: k for key, (k, _) in res.cuts.get(b, {}).items()}
    alt = _run(inp, forced=forced, forced_cuts=cuts)
    assert np.array_equal(alt.tokens, res.tokens)
    assert np.array_equal(alt.n_accepted, res.n_accepted)


def test_forced_rejection_emits_a_residual_draw():
    inp = _inputs()
    res = _run(inp)
    T, tp = float(np.float32(inp.temperature)), float(np.float32(inp.top_p))
    checked = 0
    for b in range(inp.B):
        n = int(res.n_accepted[b])
        if n < 1:
            continue
        j = n - 1  # accepted by the unforced run: force it rejected
        alt = _run(inp, rows=[b], forced={b: {j: False}})
        assert alt.n_accepted[b] == j
        assert np.array_equal(alt.tokens[b, :j], res.tokens[b, :j])
        assert np.all(alt.tokens[b, j + 1:] == -1)
        # the residual at j from scipy's softmax and a plain sort's nucleus
        def filt(l):
            p = scipy.special.softmax(np.asarray(l, np.float64) / T)
            ids = _prefix_by_sort(p, int(np.searchsorted(np.cumsum(np.sort(p)[::-1]), tp) + 1))
            out = np.zeros_like(p)
            out[ids] = p[ids]
            return out / out.sum()
        pt = filt(inp.target[b, j])
        w = np.maximum(pt - filt(inp.draft[b, j]), 0.0)
        if not w.sum() > 0:
            w = pt  # no residual mass (equal filtered rows): the draw is from p'
        u = uniforms(inp.seed, b, j)[1]
        c = np.cumsum(w)
        y = int(alt.tokens[b, j])
        lo = c[y - 1] if y else 0.0
        assert w[y] > 0
        assert lo - 1e-12 * c[-1] <= u * c[-1] <= c[y] + 1e-12 * c[-1]
        checked += 1
    assert checked >= 3
