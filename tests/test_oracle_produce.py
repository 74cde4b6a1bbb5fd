"""Pins of the synthetic draft producer's oracle (oracle/produce.py) against
what the definition and the mathematics fix: the perturbation's grid, range
and uniformity, independence between ids, positions and rows, round to
nearest even by brute force, and the greedy token by a plain loop."""

import numpy as np
import pytest
from scipy import stats

from oracle import produce as P


def test_delta_grid_range_and_uniformity():
    d = P.deltas(seed=11, b=3, j=1, V=1 << 18).astype(np.float64)
    k = d * 512.0
    assert np.all(k == np.round(k))                      # a 1/512 grid
    assert d.min() == -2.0 and d.max() == 2.0 - 2.0 ** -9  # [-2, 2), both ends reached
    counts = np.bincount((k + 1024).astype(np.int64), minlength=2048)
    assert counts.size == 2048
    assert stats.chisquare(counts).pvalue > 1e-4           # uniform on the 2048 points


def test_delta_streams_are_independent():
    V = 1 << 16
    a = P.deltas(7, 0, 0, V).astype(np.float64)
    # the eight ids of one 16-byte vector draw distinct halves: no two of them
    # move together
    m = a.reshape(-1, 8)
    c = np.corrcoef(m.T)
    assert np.max(np.abs(c - np.eye(8))) < 0.05
    # other positions, rows and seeds draw other numbers
    for other in (P.deltas(7, 0, 1, V), P.deltas(7, 1, 0, V), P.deltas(8, 0, 0, V)):
        o = other.astype(np.float64)
        assert abs(np.corrcoef(a, o)[0, 1]) < 0.03
        assert np.mean(a == o) < 0.01


def _rne_brute(x):
    """Nearest bf16 to a finite float32 by search over the two neighbours,
    ties to the even significand."""
    x = np.float32(x)
    u = int(np.array(x).view(np.uint32))
    lo = u >> 16
    cands = [lo, lo + 1]
    vals = [float(np.array([c << 16], np.uint32).view(np.float32)[0]) for c in cands]
    errs = [abs(v - float(x)) for v in vals]
    if errs[0] < errs[1]:
        return cands[0]
    if errs[1] < errs[0]:
        return cands[1]
    return cands[0] if cands[0] % 2 == 0 else cands[1]


def test_bf16_rounding_is_nearest_even():
    rng = np.random.default_rng(3)
    xs = np.concatenate([rng.standard_normal(2000).astype(np.float32) * 5,
                         # exact halfway cases: bf16 value plus half a unit
                         (np.arange(-50, 50, dtype=np.int64).astype(np.uint32) * 0 +
                          np.array([0x3F808000, 0x3F818000, 0xC0408000, 0x41228000], np.uint32).repeat(25)).view(np.float32)])
    got = P.f32_to_bf16_rne(xs)
    want = np.array([_rne_brute(x) for x in xs], np.uint32) & 0xFFFF
    assert np.array_equal(got.astype(np.uint32), want)
    assert P.f32_to_bf16_rne(np.float32(np.nan)) == 0x7FC0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_draft_is_target_plus_delta_rounded(dtype):
    rng = np.random.default_rng(5)
    B, K, V = 2, 3, 999
    t32 = (rng.standard_normal((B, K + 1, V)) * 3).astype(np.float32)
    t = P.f32_to_bf16_rne(t32) if dtype == "bf16" else t32
    d, tok = P.produce_drafts(t, K, seed=99)
    assert d.shape == (B, K, V) and d.dtype == t.dtype
    for b in range(B):
        for j in range(K):
            tv = (P.bf16_to_f32(t[b, j]) if dtype == "bf16" else t[b, j]).astype(np.float64)
            dv = (P.bf16_to_f32(d[b, j]) if dtype == "bf16" else d[b, j]).astype(np.float64)
            exact = tv + P.deltas(99, b, j, V).astype(np.float64)
            # one rounding of the exact sum: within half a unit of the result's format
            ulp = np.spacing(np.abs(exact).astype(np.float32)).astype(np.float64) * (65536 if dtype == "bf16" else 1)
            assert np.all(np.abs(dv - exact) <= ulp / 2 * (1 + 1e-9) + 2.0 ** -149)
            # the greedy token, by a plain loop: first id of the largest value
            best, bid = -np.inf, 0
            for v in range(V):
                if dv[v] > best:
                    best, bid = dv[v], v
            assert tok[b, j] == bid


def test_tokens_ties_nan_and_masked_rows():
    V = 40
    t = np.full((3, 3, V), -np.inf, np.float32)
    t[0, :, 5] = 100.0
    t[0, :, 30] = 100.0          # equal after the same-size perturbation only by chance
    t[1, 0, 7] = np.nan          # a NaN: the row has no token
    d, tok = P.produce_drafts(t, 2, seed=1)
    assert tok[0, 0] in (5, 30) and tok[1, 0] == -1
    # an all -inf row stays -inf: every id ties, the lowest wins
    assert np.all(np.isneginf(d[2])) and tok[2, 0] == 0 and tok[2, 1] == 0
    # exact ties after rounding go to the lower id
    t2 = np.zeros((1, 2, 16), np.float32)
    t2[0, 0] = 1e30                              # delta vanishes in the rounding
    d2, tok2 = P.produce_drafts(t2, 1, seed=2)
    assert np.all(d2[0, 0] == np.float32(1e30)) and tok2[0, 0] == 0
