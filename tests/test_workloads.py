"""The seeded input generator: shapes, dtype rounding, seeds, structure."""

import numpy as np
import pytest
import torch

import oracle
from rejection_sampling_verifier_amd import workloads as W


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(0, 3, 100000), rng.normal(0, 1e-30, 1000), rng.normal(0, 1e30, 1000),
                        [0.0, -0.0, np.inf, -np.inf, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]]).astype(np.float32)
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(W.bf16_bits_to_f32(ours), torch.from_numpy(ours.view(np.int16)).view(
        torch.bfloat16).float().numpy())


def test_small_configs_reproducible():
    a = W.make_inputs(0, 3)
    b = W.make_inputs(0, 3)
    c = W.make_inputs(0, 4)
    np.testing.assert_array_equal(a.target, b.target)
    np.testing.assert_array_equal(a.draft_tokens, b.draft_tokens)
    assert not np.array_equal(a.target, c.target)
    assert a.seed == 3 and c.seed == 4
    assert a.target.shape == (1, 6, 1000) and a.draft.shape == (1, 5, 1000)
    assert a.logical_bytes() == 11 * 1000 * 4 == 44000
    assert a.positions() == 5


def test_shrunk_ragged_structure():
    x = W.make_inputs(3, 1, B=16, V=4000)
    L = x.draft_len
    assert L.min() >= 1 and L.max() <= 8
    for b in range(16):
        t = W.bf16_bits_to_f32(x.target[b])
        d = W.bf16_bits_to_f32(x.draft[b])
        assert np.all(np.isnan(t[L[b] + 1:])) and not np.any(np.isnan(t[: L[b] + 1]))
        assert np.all(np.isnan(d[L[b]:])) and not np.any(np.isnan(d[: L[b]]))
        assert np.all(x.draft_tokens[b, L[b]:] == -1)
        assert np.all((x.draft_tokens[b, : L[b]] >= 0) & (x.draft_tokens[b, : L[b]] < 4000))
        # 4 spikes of +8 per (row, position): the max sits well above N(0, 9)
        assert np.all(t[0].max() > 8)


def test_filtered_drafts_inside_draft_nucleus():
    x = W.make_inputs(4, 0, B=4, V=20000)
    d = W.bf16_bits_to_f32(x.draft).astype(np.float64)
    for b in range(4):
        for j in range(5):
            q = oracle.softmax(d[b, j], float(x.temperature))[0]
            qf = oracle.nucleus(q, float(x.top_p))[0]
            assert qf[x.draft_tokens[b, j]] > 0


def test_gumbel_sampling_is_softmax():
    rng = np.random.Generator(np.random.PCG64(5))
    l = np.array([[0.0, 1.0, 2.0, -1.0]], np.float32).repeat(20000, 0)
    ids = W._gumbel_argmax(rng, l, 0.7).ravel()
    p = oracle.softmax(l[0].astype(np.float64), float(np.float32(0.7)))[0]
    import scipy.stats
    assert scipy.stats.chisquare(np.bincount(ids, minlength=4), 20000 * p).pvalue > 1e-3


@pytest.mark.slow
def test_full_batched_shape():
    x = W.make_inputs(2, 0)
    assert x.target.shape == (64, 6, 128256) and x.target.dtype == np.uint16
    assert x.logical_bytes() == 180584448 and x.positions() == 320


def test_filtered_drafts_come_from_the_draft_nucleus():
    # the filtered workload drafts from the top-p-filtered draft softmax:
    # every drafted token lies in the oracle's nucleus of its draft row, and
    # over many rows the tokens follow the filtered distribution
    x = W.make_inputs(4, 0, B=6, V=5003)
    for b in range(x.B):
        for j in range(x.K):
            p, _, _ = oracle.softmax(oracle.widen_bf16(x.draft[b, j]), float(x.temperature))
            q, _, _ = oracle.nucleus(p, float(x.top_p))
            assert q[x.draft_tokens[b, j]] > 0.0, (b, j)
    rng = np.random.default_rng(5)
    row = (rng.standard_normal(40) * 2.0).astype(np.float32)
    p, _, _ = oracle.softmax(row.astype(np.float64), 0.7)
    q, _, _ = oracle.nucleus(p, 0.9)
    n = 20000
    toks = W._nucleus_gumbel(np.random.default_rng(6), np.tile(row, (n, 1)), 0.7, 0.9, cand=8)
    counts = np.bincount(toks, minlength=row.size)
    assert np.all(counts[q == 0.0] == 0)
    exp = q * n
    m = exp > 0
    chi2 = float(np.sum((counts[m] - exp[m]) ** 2 / exp[m]))
    from scipy.stats import chi2 as C
    assert C.sf(chi2, int(m.sum()) - 1) > 1e-4, chi2
