"""Shared helpers of the GPU tests: move seeded inputs to the device, run the
library through its binding, run the oracle on the same inputs, compare
decision by decision.

The bar (the exactness claim of the page "Speculative Decoding للمحترف: ضاعف
سرعة Llama 70B لـ 2.4x بدون فقد token واحد", section "التعريف الرياضي من
Leviathan et al.", turned into a finite-precision check): accepted counts and
emitted tokens equal the oracle's except at decisions that lie within the
library's own rounding bound of their boundary ("flagged").  Each decision
kind has its band, the rigorous error bound of the kernel arithmetic that
takes it (the derivations are in the design notes):

  accept   |u - r| < BAND_ACCEPT.  r comes from the statistics pass's
           normalisers, float32 exponentials summed in float32 per lane and
           per wave: relative error below 1.2e-6 each, so below 2.4e-6 on r;
           with top-p the kept masses (below 1.6e-6 each) replace them.
  sample   |C - t|/Z < BAND_SAMPLE (plus float64 rounding relative to the
           row's Z) at the token's interval: the draw is float64 throughout.
  nucleus  the running mass at the cut within BAND_NUCLEUS of top_p: float32
           exponentials of the kept tokens against top_p times the float32
           normaliser.

What is checked at a flagged decision instead of equality:
  * an acceptance test decided the other way: everything before it matches,
    and the rest of the row must match the oracle's run forced down the
    library's branch;
  * a draw: the library's token has positive weight and its running-sum
    interval lies within the band of u (a valid neighbour of the oracle's);
  * a nucleus cut: the library's kept mass (a probe value, float32-exact to
    KEPT_TOL) tells which of the prefixes of k-1, k or k+1 tokens it kept; a
    different count than the oracle's is followed by forcing the oracle's cut
    to it, and the row must then match that run.  Only when two prefixes lie
    within KEPT_TOL of the library's mass (the token at the cut carries less
    than that) is the cut undetermined, and from that position on only the
    output's structure is checked (drafted ids, then one token in [0, V),
    then -1).
"""

import math
import sys
from dataclasses import dataclass, field

import numpy as np
import torch

import oracle
from rejection_sampling_verifier_amd import binding

PROBE_RTOL = 1e-5  # probabilities and residual masses (spec tolerance)

BAND_ACCEPT = 2.5e-6
BAND_ACCEPT_TOPP = 3.5e-6
BAND_SAMPLE = 1e-10
# float64 rounding of Z = A - rho*B and of the exponentials, relative to Z
# (in units of the target's kept mass): added to BAND_SAMPLE per row
SAMPLE_REL_EPS = 4e-13
BAND_NUCLEUS = 3e-6
# the library's kept masses: float32 exponentials of the kept tokens over the
# float32 normaliser (relative error below 1.6e-6; kept masses are <= 1)
KEPT_TOL = 2e-6
BANDS = {"accept": BAND_ACCEPT, "sample": BAND_SAMPLE, "nucleus_t": BAND_NUCLEUS, "nucleus_d": BAND_NUCLEUS,
         "degenerate": math.inf}


def dev_array(a, device="cuda"):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_device(inp, device="cuda"):
    t = dev_array(inp.target, device)
    d = dev_array(inp.draft, device)
    x = torch.from_numpy(np.ascontiguousarray(inp.draft_tokens, dtype=np.int32)).to(device)
    dl = None if inp.draft_len is None else torch.from_numpy(np.ascontiguousarray(inp.draft_len, np.int32)).to(device)
    return t, d, x, dl


def run_gpu(inp, probe=True, tensors=None):
    t, d, x, dl = to_device(inp) if tensors is None else tensors
    out = binding.verify(t, d, x, dl, float(inp.temperature), float(inp.top_p), inp.seed, probe=probe)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in out]


def run_oracle(inp, rows=None, forced=None, forced_cuts=None):
    return oracle.verify(inp.target, inp.draft, inp.draft_tokens, inp.draft_len, inp.temperature, inp.top_p,
                         inp.seed, rows=rows, forced=forced, forced_cuts=forced_cuts)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def sample_band(res, b):
    """The draw's band for row b: BAND_SAMPLE plus the float64 rounding of
    the library's mass arithmetic relative to this row's Z (Z is in units of
    the target mass, 1 for a bonus draw)."""
    z = res.probe_row[b, 0]
    return BAND_SAMPLE + (SAMPLE_REL_EPS / z if z > 0 else math.inf)


def accept_band(inp):
    return BAND_ACCEPT_TOPP if float(inp.top_p) < 1.0 else BAND_ACCEPT


def band_of(kind, res, b, inp):
    if kind == "sample":
        return sample_band(res, b)
    if kind == "accept":
        return accept_band(inp)
    if kind.startswith("nucleus"):
        return BAND_NUCLEUS
    return BANDS[kind]


def near_boundary(res, b, top_p):
    """True when a decision of row b of the oracle result `res` lies within
    the library's band for its kind (a row another finite-precision
    implementation may legitimately decide differently)."""
    if b not in res.margins:
        return False
    acc = BAND_ACCEPT_TOPP if float(top_p) < 1.0 else BAND_ACCEPT
    for kind, _, mg in res.margins[b]:
        band = {"accept": acc, "sample": sample_band(res, b)}.get(kind, BAND_NUCLEUS if kind.startswith("nucleus")
                                                                  else math.inf)
        if mg < band:
            return True
    return False


@dataclass
class ParityStats:
    rows: int = 0                 # rows compared
    decisions: int = 0            # oracle decisions on those rows
    flagged: dict = field(default_factory=dict)  # kind -> decisions within their band
    branch_switches: int = 0      # flagged acceptance tests the library took the other way
    cut_switches: int = 0         # flagged nucleus cuts the library took one token to the other side
    neighbour_draws: int = 0      # flagged draws where the library drew a valid neighbour
    structural_rows: int = 0      # rows past a flagged nucleus cut (structure checked only)
    exact_rows: int = 0           # rows equal to the oracle's outputs bit for bit

    @property
    def n_flagged(self):
        return sum(self.flagged.values())

    @property
    def flagged_fraction(self):
        return self.n_flagged / max(1, self.decisions)

    def add(self, o):
        self.rows += o.rows
        self.decisions += o.decisions
        for k, v in o.flagged.items():
            self.flagged[k] = self.flagged.get(k, 0) + v
        self.branch_switches += o.branch_switches
        self.cut_switches += o.cut_switches
        self.neighbour_draws += o.neighbour_draws
        self.structural_rows += o.structural_rows
        self.exact_rows += o.exact_rows
        return self

    def __str__(self):
        kinds = " ".join(f"{k}={v}" for k, v in sorted(self.flagged.items()))
        return (f"rows={self.rows} exact={self.exact_rows} decisions={self.decisions} flagged={self.n_flagged} "
                f"({self.flagged_fraction:.2e}) [{kinds}] switches={self.branch_switches} cut_switches={self.cut_switches} "
                f"neighbours={self.neighbour_draws} structural={self.structural_rows}")


def _structure_ok(inp, b, n, toks):
    L = int(inp.lengths()[b])
    K1 = inp.K + 1
    assert 0 <= n <= L, (b, n, L)
    assert list(toks[:n]) == list(inp.draft_tokens[b, :n]), (b, toks, inp.draft_tokens[b])
    assert 0 <= toks[n] < inp.V, (b, toks)
    assert np.all(toks[n + 1:K1] == -1), (b, toks)


def _check_draw(inp, res, b, g_tok, stats):
    """The draw at the row's n: equal to the oracle's token outside the band;
    inside it, a positive-weight token whose interval lies within the band."""
    m = [mg for k, _, mg in res.margins[b] if k == "sample"][0]
    band = sample_band(res, b)
    o_tok = int(res.tokens[b, res.n_accepted[b]])
    if m >= band:
        assert g_tok == o_tok, (b, g_tok, o_tok, m)
        return
    if g_tok == o_tok:
        return
    cdf = res.sample_cdf.get(b)
    assert cdf is not None, (b, m)
    u = res.probe_row[b, 2]
    lo = cdf[g_tok - 1] if g_tok > 0 else 0.0
    hi = cdf[g_tok]
    assert hi > lo, (b, g_tok, "zero weight")
    assert lo <= u + band and hi >= u - band, (b, g_tok, o_tok, lo, hi, u, band)
    stats.neighbour_draws += 1


def _library_cuts(res, b, pp):
    """The library's count at each nucleus cut of row b within BAND_NUCLEUS
    of top_p, read from its kept mass pp[j, 6|7] against the oracle's
    prefixes of k-1, k and k+1 tokens.  Returns ({(side, j): count} for the
    cuts it took differently, the smallest position of a cut it cannot
    determine, or None)."""
    flips, unknown = {}, None
    for kind, j, mg in res.margins[b]:
        if not kind.startswith("nucleus") or mg >= BAND_NUCLEUS:
            continue
        side = kind[-1]
        k, kept3 = res.cuts[b][(side, j)]
        lib = float(pp[j, 6 if side == "t" else 7])
        d = np.array([abs(lib - v) if np.isfinite(v) else np.inf for v in kept3])
        near = np.sort(d)
        if not near[0] <= KEPT_TOL or near[1] <= KEPT_TOL:
            unknown = j if unknown is None else min(unknown, j)
            continue
        best = int(np.argmin(d))
        if best != 1:
            flips[(side, j)] = k - 1 + best
    return flips, unknown


def _check_row(inp, res, b, gpu_row, stats, forced=None, cuts=None, depth=0):
    """Compares row b of the library's output (n, tokens, probe_pos or None)
    with the oracle's result `res`, decision by decision.  Returns (True when
    equal bit for bit, the oracle result the row was finally compared to)."""
    n_g, toks, pp = gpu_row
    n_o = int(res.n_accepted[b])
    if n_o < 0:
        assert n_g == n_o and np.all(toks == -1), (b, n_g, toks)
        return True, res
    assert depth < 6, (b, "too many near-boundary switches")
    L = int(inp.lengths()[b])
    margins = res.margins[b]
    first_cut = L + 1
    if pp is not None:
        flips, unknown = _library_cuts(res, b, pp)
        if flips:
            stats.cut_switches += len(flips)
            cuts = {**(cuts or {}), **flips}
            alt = run_oracle(inp, rows=[b], forced={b: forced} if forced else None, forced_cuts={b: cuts})
            return _check_row(inp, alt, b, gpu_row, stats, forced, cuts, depth + 1)
        if unknown is not None:
            first_cut = unknown
    else:
        cut_flag = [j for k, j, mg in margins if k.startswith("nucleus") and mg < BAND_NUCLEUS]
        first_cut = min(cut_flag, default=L + 1)
    accepts = res.accepts[b]
    j0 = min(n_g, n_o)
    if first_cut <= j0:
        stats.structural_rows += 1
        _structure_ok(inp, b, n_g, toks)
        return False, res
    if n_g != n_o:
        # the test at j0 went the other way: it must lie within its band
        u, r = accepts[j0]
        assert abs(u - r) < accept_band(inp) and j0 not in (forced or {}), (b, n_g, n_o, u, r)
        stats.branch_switches += 1
        forced = {**(forced or {}), j0: n_g > j0}
        alt = run_oracle(inp, rows=[b], forced={b: forced}, forced_cuts={b: cuts} if cuts else None)
        return _check_row(inp, alt, b, gpu_row, stats, forced, cuts, depth + 1)
    assert list(toks[:n_g]) == list(res.tokens[b, :n_g]), (b, toks, res.tokens[b])
    assert np.all(toks[n_g + 1:] == -1), (b, toks)
    if first_cut <= n_g:
        stats.structural_rows += 1
        _structure_ok(inp, b, n_g, toks)
        return False, res
    if any(k == "degenerate" for k, _, _ in margins):
        _structure_ok(inp, b, n_g, toks)
        return False, res
    _check_draw(inp, res, b, int(toks[n_g]), stats)
    return bool(toks[n_g] == res.tokens[b, n_g]), res


def check_parity(inp, res, gpu, rows=None, check_probes=True):
    """Decision-by-decision comparison on the rows the oracle computed (see
    the module docstring).  Probe values (max logit, softmax normalisers,
    p'(x_j), q'(x_j), kept masses, and Z, t, u where the row's n agrees)
    must agree to PROBE_RTOL relative with the oracle run the row was
    compared to.  Returns ParityStats."""
    tokens, n_acc = gpu[0], gpu[1]
    has_probes = len(gpu) > 2
    rows = res.rows if rows is None else rows
    st = ParityStats()
    for b in rows:
        st.rows += 1
        ms = res.margins.get(b, [])
        st.decisions += len(ms)
        for k, _, mg in ms:
            if mg < band_of(k, res, b, inp):
                st.flagged[k] = st.flagged.get(k, 0) + 1
        row = (int(n_acc[b]), tokens[b], gpu[2][b] if has_probes else None)
        exact, ref = _check_row(inp, res, b, row, st)
        st.exact_rows += int(exact)
        if check_probes and has_probes and ref.n_accepted[b] >= 0:
            pp, pr = gpu[2], gpu[3]
            ok = ~np.isnan(ref.probe_pos[b])
            np.testing.assert_array_equal(np.isnan(pp[b]), ~ok, err_msg=f"probe NaN pattern, row {b}")
            np.testing.assert_allclose(pp[b][ok], ref.probe_pos[b][ok], rtol=PROBE_RTOL, atol=0,
                                       err_msg=f"probe_pos row {b}")
            if int(n_acc[b]) == int(ref.n_accepted[b]) and pr[b][3] == ref.n_accepted[b]:
                np.testing.assert_allclose(pr[b][:3], ref.probe_row[b][:3], rtol=PROBE_RTOL, atol=0,
                                           err_msg=f"probe_row row {b}")
    return st
