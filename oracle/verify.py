"""Float64 oracle of the batched speculative-sampling verify step.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources (the pages this follows, cited by title and section):
  [SD]  "Speculative Decoding للمحترف: ضاعف سرعة Llama 70B لـ 2.4x بدون فقد token
        واحد" -- section "المفهوم بالتقريب" (the K drafted tokens are scored
        in one target pass; every agreed token is accepted, the first
        disagreeing one is rejected and resampled from the target side),
        section "التعريف الرياضي من Leviathan et al." (equation for alpha(x) =
        min(1, p_target(x)/p_draft(x)); equation for the corrected
        distribution p'(x) = max(0, p_target(x) - p_draft(x))/Z; the claim that
        the output distribution is exactly the target's), section "كود شغّال
        على vLLM" (the knobs: K, temperature 0.7, top_p 0.9).
  [SMC] "Faster LLM Inference via Sequential Monte Carlo" -- section 2, the
        scoring step: the target scores K+1 positions in one pass and yields
        one extra ("bonus") token per sequence.
  [HS]  "HiSpec: Hierarchical Speculative Decoding for LLMs" -- section 2,
        batched inference: each sequence in a batch keeps its own accepted
        length, without padding.

Readings taken where the pages are silent (each also listed in the design
notes):
  * temperature divides the logits of both models before the softmax;
  * accept iff u < r with r = p(x)/q(x); because u < 1 this equals
    u < min(1, r); q(x) = 0 gives r = +inf when p(x) > 0 and r = 0 otherwise;
  * the first rejected position n stops the scan; later positions are not
    evaluated;
  * on a rejection the resample is from max(0, p_n - q_n); when every drafted
    token is accepted (including a row with no drafts) the bonus token is drawn
    from the target distribution at position L;
  * inverse CDF: with C the running sum over token ids in increasing order and
    Z = C[-1], the token is the smallest id with C[id] > u * Z;
  * top-p: a stable descending sort (ties broken by the lower id), the shortest
    prefix whose running mass reaches top_p, renormalised; applied after the
    temperature to every target and draft distribution the step uses;
  * a row with a draft length outside [0, K], a drafted id outside [0, V), or
    a needed logit row holding NaN or +inf or only -inf is invalid: it emits
    n = -1 and all tokens -1.

Decision margins: each evaluated acceptance test, each sample and each nucleus
cut records its distance to the decision boundary.  A row holding a decision
whose margin is below FLAG_BAND is "flagged": any correct finite-precision
implementation may legitimately decide it either way.  Besides the margins the
result keeps what a caller needs to judge a decision it takes differently:
the (u, r) pair of every evaluated acceptance test, and, for a draw whose
margin is below SAMPLE_KEEP_BAND, the draw's running sums divided by Z, so
that any token can be placed against u.
"""

from dataclasses import dataclass, field

import numpy as np

from .philox import uniforms

FLAG_BAND = 1e-6
# draws this close to a boundary keep their normalised running sums
SAMPLE_KEEP_BAND = 1e-5

# probe layout per position j (float64):
#   0 target max logit   1 target sum exp((l-max)/T)
#   2 draft max logit    3 draft sum exp((l-max)/T)
#   4 p'(x_j)            5 q'(x_j)
#   6 target kept mass   7 draft kept mass  (1.0 when top-p is off)
PROBE_POS = 8
# probe layout per row: 0 Z, 1 t = u*Z, 2 u_res, 3 n
PROBE_ROW = 4


def widen_bf16(bits):
    """bfloat16 bit patterns (uint16) -> float64, exactly.

    A bfloat16 value is the upper half of a float32 word, so shifting the
    16-bit pattern into the top half reproduces the float32 value exactly.
    """
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _widen(x):
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return widen_bf16(x)
    return x.astype(np.float64)


def softmax(logits, temperature):
    """Temperature softmax in float64: exp((l - max l)/T) / sum.

    Returns (p, max logit, normaliser sum).  [SD] "التعريف الرياضي" uses the
    normalised target and draft probabilities; the temperature reading is in
    the module docstring.
    """
    l = np.asarray(logits, dtype=np.float64)
    m = float(np.max(l))
    e = np.exp((l - m) / temperature)
    s = float(np.sum(e))
    return e / s, m, s


def nucleus(p, top_p, keep=None):
    """Top-p filter by its sorting definition.

    Sort tokens by probability, descending, ties by the lower id (stable
    argsort); keep the shortest prefix whose running mass reaches top_p;
    renormalise by the kept mass.  Returns (filtered p, kept mass, margin):
    the margin is the distance of the two running sums around the cut from
    top_p.  When no running sum reaches top_p (rounding with top_p near 1)
    every token is kept.  `keep` (a count) replaces the cut: the prefix of
    that many tokens is kept instead, the margin still being that of the
    defined cut.
    """
    p, k, c, margin = _nucleus_cut(p, top_p)
    if keep is not None:
        k = int(keep)
    order = np.argsort(-p, kind="stable")
    kept = float(c[k - 1])
    out = np.zeros_like(p)
    out[order[:k]] = p[order[:k]] / kept
    return out, kept, float(margin)


def _nucleus_cut(p, top_p):
    """(p as float64, kept count, running sums in sorted order, margin)."""
    p = np.asarray(p, dtype=np.float64)
    order = np.argsort(-p, kind="stable")
    c = np.cumsum(p[order])
    hit = np.nonzero(c >= top_p)[0]
    k = int(hit[0]) + 1 if hit.size else p.size
    margin = abs(c[k - 1] - top_p)
    if k >= 2:
        margin = min(margin, abs(c[k - 2] - top_p))
    return p, k, c, float(margin)


def nucleus_neighbours(p, top_p):
    """The defined cut's kept count k and the kept masses of the prefixes of
    k-1, k and k+1 tokens (NaN where no such prefix exists): what another
    implementation keeps when it takes a near-boundary cut one token to
    either side."""
    _, k, c, _ = _nucleus_cut(p, top_p)
    prev = float(c[k - 2]) if k >= 2 else np.nan
    nxt = float(c[k]) if k < c.size else np.nan
    return k, (prev, float(c[k - 1]), nxt)


def ratio(p_x, q_x):
    """r = p(x)/q(x) with the q(x) = 0 convention (+inf if p(x) > 0, else 0)."""
    if q_x > 0.0:
        return p_x / q_x
    return np.inf if p_x > 0.0 else 0.0


def accept(u, r):
    """[SD] alpha(x) = min(1, r): accept iff u < min(1, r), i.e. u < r for u < 1."""
    return u < min(1.0, r)


def residual_weights(p, q):
    """[SD] corrected distribution, unnormalised: max(0, p - q)."""
    return np.maximum(0.0, np.asarray(p, dtype=np.float64) - np.asarray(q, dtype=np.float64))


def inverse_cdf(w, u):
    """Inverse-CDF draw from weights w with one uniform u in [0, 1).

    C = running sum of w in id order, Z = C[-1], t = u * Z; the token is the
    smallest id with C[id] > t, else (rounding) the largest id with w > 0.
    Returns (token, Z, t, margin) with margin = distance of t to the nearer
    edge of the token's interval, divided by Z.
    """
    w = np.asarray(w, dtype=np.float64)
    c = np.cumsum(w)
    z = float(c[-1])
    t = u * z
    y = int(np.searchsorted(c, t, side="right"))
    if y >= w.size:
        y = int(np.nonzero(w > 0.0)[0][-1])
        return y, z, t, 0.0
    lo = float(c[y - 1]) if y > 0 else 0.0
    margin = min(t - lo, float(c[y]) - t) / z
    return y, z, t, margin


@dataclass
class RowDecision:
    n: int
    tokens: list
    z: float = np.nan
    t: float = np.nan
    u_res: float = np.nan
    margins: list = field(default_factory=list)  # (kind, position, margin)
    accepts: list = field(default_factory=list)  # (u, r) of each evaluated acceptance test
    cdf: np.ndarray = None                       # running sums / Z of the draw


def decide_row(p, q, x, u_acc, u_res):
    """Accept scan and final draw for one row, given its distributions.

    p: list of L+1 target distributions (positions 0..L), q: list of L draft
    distributions, x: the L drafted ids, u_acc / u_res: per-position uniforms
    (length >= L+1).  [SD] "المفهوم بالتقريب": accept every agreed token and
    reject the first disagreeing one; [SMC] section 2: the bonus token when
    all L are accepted.
    """
    L = len(q)
    margins = []
    accepts = []
    n = L
    for j in range(L):
        r = ratio(p[j][x[j]], q[j][x[j]])
        margins.append(("accept", j, abs(u_acc[j] - r)))
        accepts.append((float(u_acc[j]), float(r)))
        if not accept(u_acc[j], r):
            n = j
            break
    if n < L:
        w = residual_weights(p[n], q[n])
        if not np.sum(w) > 0.0:
            # Cannot happen in exact arithmetic (a rejection needs
            # p(x) < q(x), so some mass of p exceeds q); numerically it falls
            # back to the target distribution and the row is flagged.
            w = np.array(p[n], dtype=np.float64)
            margins.append(("degenerate", n, 0.0))
    else:
        w = np.array(p[L], dtype=np.float64)
    y, z, t, m = inverse_cdf(w, u_res[n])
    margins.append(("sample", n, m))
    cdf = np.cumsum(np.asarray(w, dtype=np.float64)) / z if m < SAMPLE_KEEP_BAND else None
    return RowDecision(n=n, tokens=list(x[:n]) + [y], z=z, t=t, u_res=u_res[n], margins=margins,
                       accepts=accepts, cdf=cdf)


@dataclass
class OracleResult:
    tokens: np.ndarray        # [B, K+1] int64, -1 after the last emitted token
    n_accepted: np.ndarray    # [B] int64, -1 for an invalid row
    probe_pos: np.ndarray     # [B, K+1, PROBE_POS] float64
    probe_row: np.ndarray     # [B, PROBE_ROW] float64
    min_margin: np.ndarray    # [B] smallest decision margin in the row
    n_decisions: np.ndarray   # [B] decisions taken in the row
    n_flagged: np.ndarray     # [B] decisions with margin below FLAG_BAND
    rows: np.ndarray          # the rows computed
    margins: dict = field(default_factory=dict)   # b -> [(kind, position, margin)]
    accepts: dict = field(default_factory=dict)   # b -> [(u, r)] in position order
    sample_cdf: dict = field(default_factory=dict)  # b -> running sums / Z (near-boundary draws)
    u_res: np.ndarray = None  # [B, K+1] resampling uniforms of the evaluated positions
    # b -> {(side "t"/"d", position): (k, (kept of k-1, k, k+1 tokens))} for
    # the nucleus cuts within SAMPLE_KEEP_BAND of top_p
    cuts: dict = field(default_factory=dict)

    @property
    def flagged(self):
        return self.min_margin < FLAG_BAND


def _row_is_bad(l):
    return bool(np.any(np.isnan(l)) or np.any(l == np.inf) or np.all(l == -np.inf))


def verify(target, draft, draft_tokens, draft_len, temperature, top_p, seed, rows=None, stage=0, forced=None,
           forced_cuts=None):
    """The verify step on a batch.

    target: [B, K+1, V] logits (float32/float64 values, or uint16 bfloat16
    bit patterns); draft: [B, K, V] likewise; draft_tokens: [B, K] ints;
    draft_len: [B] ints or None (every row drafts K); temperature and top_p
    are taken as float32, the precision the library's interface carries;
    top_p >= 1 switches the filter off.  seed: 64-bit Philox key.
    rows: optional subset of batch rows to compute (rows are independent);
    the other rows of the result are left at -1 / NaN.  stage: the third
    Philox counter word (0 for the verify step; a second verification of the
    same rows, as in the hierarchical step, draws from stage 1).
    forced: optional {row: {position: accept}} that replaces the uniform
    comparison at those acceptance tests (accept: u taken as 0, which accepts
    any r > 0; reject: u taken as 1, which no r <= 1 passes).  A caller that
    sees another implementation decide a near-boundary test the other way
    uses it to follow that branch; such a test's margin is meaningless.
    forced_cuts: optional {row: {(side, position): count}} with side "t"
    (target) or "d" (draft) that keeps that many tokens at that nucleus cut
    instead of the defined count (see nucleus); the same use for a cut that
    lies within rounding of top_p.  Its margin is reported as infinite.
    """
    tl = _widen(target)
    dl = _widen(draft)
    B, K1, V = tl.shape
    K = K1 - 1
    if dl.shape != (B, K, V):
        raise ValueError("draft logits must be [B, K, V] matching target [B, K+1, V]")
    tok = np.asarray(draft_tokens, dtype=np.int64).reshape(B, K)
    lens = np.full(B, K, dtype=np.int64) if draft_len is None else np.asarray(draft_len, np.int64)
    T = float(np.float32(temperature))
    tp = float(np.float32(top_p))
    use_topp = tp < 1.0
    rows = np.arange(B) if rows is None else np.asarray(rows, dtype=np.int64)

    tokens = np.full((B, K1), -1, dtype=np.int64)
    n_acc = np.full(B, -1, dtype=np.int64)
    probe_pos = np.full((B, K1, PROBE_POS), np.nan)
    probe_row = np.full((B, PROBE_ROW), np.nan)
    min_margin = np.full(B, np.inf)
    n_dec = np.zeros(B, dtype=np.int64)
    n_flag = np.zeros(B, dtype=np.int64)
    margins, accepts, sample_cdf, cuts = {}, {}, {}, {}
    u_res_all = np.full((B, K1), np.nan)

    for b in rows:
        L = int(lens[b])
        if not 0 <= L <= K:
            continue
        x = tok[b, :L]
        if np.any(x < 0) or np.any(x >= V):
            continue
        if any(_row_is_bad(tl[b, j]) for j in range(L + 1)) or any(
            _row_is_bad(dl[b, j]) for j in range(L)
        ):
            continue
        extra = []
        p, q = [], []
        fc = (forced_cuts or {}).get(int(b), {})
        row_cuts = {}

        def filtered(pj, side, j):
            keep = fc.get((side, j))
            out, kept, mg = nucleus(pj, tp, keep=keep)
            if keep is not None:
                mg = np.inf
            if mg < SAMPLE_KEEP_BAND:
                row_cuts[(side, j)] = nucleus_neighbours(pj, tp)
            extra.append(("nucleus_" + side, j, mg))
            return out, kept

        for j in range(L + 1):
            pj, m, s = softmax(tl[b, j], T)
            probe_pos[b, j, 0:2] = (m, s)
            kept = 1.0
            if use_topp:
                pj, kept = filtered(pj, "t", j)
            probe_pos[b, j, 6] = kept
            p.append(pj)
        for j in range(L):
            qj, m, s = softmax(dl[b, j], T)
            probe_pos[b, j, 2:4] = (m, s)
            kept = 1.0
            if use_topp:
                qj, kept = filtered(qj, "d", j)
            probe_pos[b, j, 7] = kept
            q.append(qj)
        for j in range(L):
            probe_pos[b, j, 4] = p[j][x[j]]
            probe_pos[b, j, 5] = q[j][x[j]]
        ua, ur = zip(*(uniforms(seed, b, j, stage) for j in range(L + 1)))
        if forced and int(b) in forced:
            ua = list(ua)
            for j, acc in forced[int(b)].items():
                ua[j] = 0.0 if acc else 1.0
        d = decide_row(p, q, x, ua, ur)
        n_acc[b] = d.n
        tokens[b, : d.n + 1] = d.tokens
        probe_row[b] = (d.z, d.t, d.u_res, d.n)
        all_m = extra + d.margins
        n_dec[b] = len(all_m)
        min_margin[b] = min(m for _, _, m in all_m)
        n_flag[b] = sum(1 for _, _, m in all_m if m < FLAG_BAND)
        margins[b] = all_m
        accepts[b] = d.accepts
        u_res_all[b, : L + 1] = ur
        if d.cdf is not None:
            sample_cdf[b] = d.cdf
        if row_cuts:
            cuts[b] = row_cuts
    return OracleResult(tokens, n_acc, probe_pos, probe_row, min_margin, n_dec, n_flag, rows,
                        margins, accepts, sample_cdf, u_res_all, cuts)
