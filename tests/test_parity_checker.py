"""The GPU parity checker, exercised on the CPU: the oracle's own outputs pass;
outputs with a mistake planted at a decision outside its band fail; a
near-boundary decision taken the other way passes only when the rest of the
row follows that branch."""

import importlib

import numpy as np
import pytest

import gpu_helpers as gh
from rejection_sampling_verifier_amd import workloads as W

# the module (the package re-exports a function of the same name)
ov = importlib.import_module("oracle.verify")


def _inp():
    return W.synthetic(40, 3, 50, dtype="bf16", temperature=0.8, sigma=1.5, seed=7, gen_seed=3)


def _fake(res):
    return [res.tokens.astype(np.int32).copy(), res.n_accepted.astype(np.int32).copy()]


def test_oracle_outputs_pass():
    inp = _inp()
    res = gh.run_oracle(inp)
    st = gh.check_parity(inp, res, _fake(res))
    assert st.rows == inp.B and st.exact_rows == inp.B and st.decisions > inp.B


def test_wrong_draw_outside_band_fails():
    inp = _inp()
    res = gh.run_oracle(inp)
    g = _fake(res)
    b = 0
    n = g[1][b]
    g[0][b, n] = (g[0][b, n] + 1) % inp.V
    with pytest.raises(AssertionError):
        gh.check_parity(inp, res, g)


def test_switched_acceptance_outside_band_fails():
    inp = _inp()
    res = gh.run_oracle(inp)
    g = _fake(res)
    b = int(np.nonzero(res.n_accepted > 0)[0][0])
    g[1][b] -= 1  # rejects a test the oracle accepted by a wide margin
    n = g[1][b]
    g[0][b, n] = 0
    g[0][b, n + 1:] = -1
    with pytest.raises(AssertionError):
        gh.check_parity(inp, res, g)


def test_switched_acceptance_inside_band(monkeypatch):
    # every acceptance test counts as near its boundary: a switch passes when
    # the row then follows the oracle's forced branch, and fails otherwise
    monkeypatch.setattr(gh, "BAND_ACCEPT", 1.0)
    inp = _inp()
    res = gh.run_oracle(inp)
    b = int(np.nonzero(res.n_accepted > 0)[0][0])
    n_new = int(res.n_accepted[b]) - 1
    alt = gh.run_oracle(inp, rows=[b], forced={b: {n_new: False}})
    g = _fake(res)
    g[0][b] = alt.tokens[b]
    g[1][b] = alt.n_accepted[b]
    st = gh.check_parity(inp, res, g, rows=[b])
    assert st.branch_switches == 1
    g[0][b, n_new] = (g[0][b, n_new] + 1) % inp.V
    if alt.margins[b][-1][2] >= gh.sample_band(alt, b):
        with pytest.raises(AssertionError):
            gh.check_parity(inp, res, g, rows=[b])


def test_neighbour_draw_inside_band(monkeypatch):
    # a draw inside its band may land on a neighbouring positive-weight
    # token; a token whose interval is far from u still fails
    monkeypatch.setattr(ov, "SAMPLE_KEEP_BAND", 2.0)
    monkeypatch.setattr(gh, "BAND_SAMPLE", 0.05)
    inp = _inp()
    res = gh.run_oracle(inp)
    checked = 0
    for b in range(inp.B):
        cdf = res.sample_cdf[b]
        n = int(res.n_accepted[b])
        y = int(res.tokens[b, n])
        u = res.probe_row[b, 2]
        w = np.diff(np.concatenate([[0.0], cdf]))
        near = [v for v in range(inp.V) if v != y and w[v] > 0
                and (cdf[v - 1] if v else 0.0) <= u + 0.05 and cdf[v] >= u - 0.05]
        far = [v for v in range(inp.V) if w[v] > 0 and ((cdf[v - 1] if v else 0.0) > u + 0.06 or cdf[v] < u - 0.06)]
        if not near or not far:
            continue
        g = _fake(res)
        g[0][b, n] = near[0]
        st = gh.check_parity(inp, res, g, rows=[b])
        assert st.neighbour_draws == 1
        g[0][b, n] = far[0]
        with pytest.raises(AssertionError):
            gh.check_parity(inp, res, g, rows=[b])
        checked += 1
    assert checked > 5


def test_structure_after_flagged_nucleus_cut(monkeypatch):
    monkeypatch.setattr(gh, "BAND_NUCLEUS", 1.0)
    inp = W.synthetic(10, 3, 60, dtype="f32", temperature=0.8, top_p=0.7, seed=3, gen_seed=5)
    res = gh.run_oracle(inp)
    g = _fake(res)
    st = gh.check_parity(inp, res, g)
    assert st.structural_rows == inp.B
    bad = _fake(res)
    bad[0][0, int(bad[1][0])] = inp.V  # out of range
    with pytest.raises(AssertionError):
        gh.check_parity(inp, res, bad)


def _fake_probed(res):
    return _fake(res) + [res.probe_pos.copy(), res.probe_row.copy()]


def test_nucleus_cut_read_from_kept_mass(monkeypatch):
    # every cut counts as near top_p; the library's kept mass shows which
    # prefix it kept: a row that took k+1 tokens at one cut must match the
    # oracle forced to that count, and fails when its tokens do not
    monkeypatch.setattr(gh, "BAND_NUCLEUS", 1.0)
    monkeypatch.setattr(ov, "SAMPLE_KEEP_BAND", 2.0)
    inp = W.synthetic(12, 3, 60, dtype="f32", temperature=0.8, top_p=0.7, seed=3, gen_seed=5)
    res = gh.run_oracle(inp)
    st = gh.check_parity(inp, res, _fake_probed(res))
    assert st.cut_switches == 0 and st.structural_rows == 0 and st.exact_rows == inp.B
    switched = 0
    for b in range(inp.B):
        n = int(res.n_accepted[b])
        k, kept3 = res.cuts[b][("t", n)]
        if not np.isfinite(kept3[2]):
            continue
        alt = gh.run_oracle(inp, rows=[b], forced_cuts={b: {("t", n): k + 1}})
        g = _fake_probed(res)
        g[0][b], g[1][b], g[2][b], g[3][b] = alt.tokens[b], alt.n_accepted[b], alt.probe_pos[b], alt.probe_row[b]
        assert g[2][b, n, 6] == kept3[2]
        st = gh.check_parity(inp, res, g, rows=[b])
        assert st.cut_switches == 1 and st.structural_rows == 0
        if alt.tokens[b, int(alt.n_accepted[b])] != res.tokens[b, n]:
            # the kept mass says k+1: the unforced oracle's tokens do not pass
            g2 = _fake_probed(res)
            g2[2][b] = alt.probe_pos[b]
            g2[3][b] = alt.probe_row[b]
            with pytest.raises(AssertionError):
                gh.check_parity(inp, res, g2, rows=[b])
            switched += 1
        nb = int(alt.n_accepted[b])
        g[0][b, nb] = (g[0][b, nb] + 7) % inp.V
        with pytest.raises(AssertionError):
            gh.check_parity(inp, res, g, rows=[b])
    assert switched >= 2
