"""Float64 oracle of one SMC-SD reweight-and-resample step.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: the page "Faster LLM Inference via Sequential Monte Carlo", section 2
("the core mechanism"): N particles are each extended by K draft tokens; the
target scores all N x K tokens in one batched pass and yields one extra
(bonus) token per particle; instead of rejecting, every particle's importance
weight is updated by the ratio of target to draft probabilities; when the
effective sample size falls below a threshold, low-weight particles are
dropped and high-weight ones duplicated (resampling).

Readings taken where the page is silent (each also listed in the design
notes):
  * p_j and q_j are the temperature softmaxes of the target and draft logits
    at position j (the temperature divides both, as in the verify step); no
    top-p filter;
  * the log-weight increment of particle i is sum_j (log p_j(x_ij) -
    log q_j(x_ij)) over its K drafted tokens; the bonus token is drawn from
    p_K and, being drawn from the target, leaves the weight unchanged;
  * log-weights accumulate across rounds: logw_out = logw_in + increment;
  * ESS = (sum w)^2 / sum w^2 over w_i = exp(logw_i - max logw);
  * resample iff ESS < ess_fraction * N (the threshold is an argument; the
    default 0.5 is a proposal, the page gives none);
  * resampling is systematic: with one uniform u0, points s_k = (k + u0)/N,
    k = 0..N-1, and ancestor a_k = the smallest i whose cumulative
    normalised weight C_i exceeds s_k; after resampling every log-weight is
    0 (equal weights); without it a_k = k and the log-weights are kept;
  * uniforms: the bonus draw uses the verify step's resampling uniform at
    counter (i, K, 0, 0), word 1; u0 is word 0 of counter (0, 0, 1, 0);
  * a particle with a drafted id outside [0, V), a needed logit row holding
    NaN or +inf or only -inf, or an input log-weight that is NaN or +inf is
    invalid: its log-weight becomes -inf and its bonus token -1.  With no
    valid particle, ESS = 0 and nothing is resampled.
"""

from dataclasses import dataclass

import numpy as np

from .philox import philox4x32_10, seed_key, uniforms, word_to_uniform
from .verify import FLAG_BAND, _row_is_bad, _widen, inverse_cdf, softmax

DEFAULT_ESS_FRACTION = 0.5


def log_weight_increment(p, q, x):
    """sum_j log p_j(x_j) - log q_j(x_j) for K distributions p, q and ids x."""
    return float(sum(np.log(p[j][x[j]]) - np.log(q[j][x[j]]) for j in range(len(x))))


def ess(logw):
    """(sum w)^2 / sum w^2 with w = exp(logw - max); 0 when every logw is -inf."""
    lw = np.asarray(logw, dtype=np.float64)
    m = np.max(lw) if lw.size else -np.inf
    if not np.isfinite(m):
        return 0.0
    w = np.exp(lw - m)
    return float(np.sum(w) ** 2 / np.sum(w * w))


def systematic(logw, u0):
    """Systematic resampling: ancestors a_k for points (k + u0)/N.

    Returns (ancestors, margin): margin is the smallest distance of a point to
    a cumulative boundary C_i (the decisions a finite-precision cumulative
    sum may take either way)."""
    lw = np.asarray(logw, dtype=np.float64)
    N = lw.size
    w = np.exp(lw - np.max(lw))
    c = np.cumsum(w) / np.sum(w)
    s = (np.arange(N, dtype=np.float64) + u0) / N
    a = np.searchsorted(c, s, side="right")
    last = int(np.nonzero(w > 0.0)[0][-1])
    a = np.minimum(a, last)
    # each point's distance to the two boundaries of its ancestor's interval
    hi = c[a]
    lo = np.where(a > 0, c[np.maximum(a - 1, 0)], 0.0)
    margin = float(np.min(np.minimum(s - lo, np.abs(hi - s)))) if N else np.inf
    return a.astype(np.int64), margin


def systematic_uniform(seed):
    """u0: word 0 of Philox4x32-10 at counter (0, 0, 1, 0)."""
    out = philox4x32_10(np.array([0, 0, 1, 0], dtype=np.uint64), seed_key(seed))
    return float(word_to_uniform(out[0]))


@dataclass
class SmcResult:
    bonus: np.ndarray        # [N] int64, -1 for an invalid particle
    logw: np.ndarray         # [N] float64 after the step
    increment: np.ndarray    # [N] float64 log-weight increment (NaN if invalid)
    ancestors: np.ndarray    # [N] int64
    ess: float               # before resampling
    resampled: bool
    min_margin: float        # smallest decision margin of the step
    n_decisions: int
    n_flagged: int
    bonus_margin: np.ndarray = None  # [N] margin of each bonus draw (inf if invalid)
    ess_margin: float = np.inf       # |ESS - ess_fraction * N| / N
    resample_margin: float = np.inf  # smallest point-to-boundary distance when resampling

    @property
    def flagged(self):
        return self.min_margin < FLAG_BAND


def smc_step(target, draft, draft_tokens, logw_in, temperature, ess_fraction, seed):
    """One SMC-SD step for N particles.

    target [N, K+1, V], draft [N, K, V] logits (float or bfloat16 bit
    patterns), draft_tokens [N, K], logw_in [N] float64, temperature (taken as
    float32), ess_fraction (float64), seed (64-bit Philox key).
    """
    tl = _widen(target)
    dl = _widen(draft)
    N, K1, V = tl.shape
    K = K1 - 1
    tok = np.asarray(draft_tokens, dtype=np.int64).reshape(N, K)
    lw_in = np.asarray(logw_in, dtype=np.float64).reshape(N)
    T = float(np.float32(temperature))
    bonus = np.full(N, -1, dtype=np.int64)
    inc = np.full(N, np.nan)
    lw = np.full(N, -np.inf)
    bm = np.full(N, np.inf)
    em, rm = np.inf, np.inf
    margins = []
    for i in range(N):
        x = tok[i]
        if np.any(x < 0) or np.any(x >= V) or np.isnan(lw_in[i]) or lw_in[i] == np.inf:
            continue
        if any(_row_is_bad(tl[i, j]) for j in range(K1)) or any(_row_is_bad(dl[i, j]) for j in range(K)):
            continue
        p = [softmax(tl[i, j], T)[0] for j in range(K1)]
        q = [softmax(dl[i, j], T)[0] for j in range(K)]
        inc[i] = log_weight_increment(p[:K], q, x)
        lw[i] = lw_in[i] + inc[i]
        _, u_res = uniforms(seed, i, K)
        y, _, _, m = inverse_cdf(p[K], u_res)
        bonus[i] = y
        bm[i] = m
        margins.append(m)
    e = ess(lw)
    resampled = False
    anc = np.arange(N, dtype=np.int64)
    if e > 0.0:
        em = abs(e - ess_fraction * N) / N
        margins.append(em)
        if e < ess_fraction * N:
            resampled = True
            anc, rm = systematic(lw, systematic_uniform(seed))
            margins.append(rm)
            lw = np.zeros(N)
    mm = min(margins) if margins else np.inf
    return SmcResult(bonus, lw, inc, anc, e, resampled, mm, len(margins),
                     sum(1 for m in margins if m < FLAG_BAND), bm, em, rm)
