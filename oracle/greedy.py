"""Float64 oracle of the greedy verify step with the next-next-token top-k.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
  * the page "Speculative Decoding للمحترف: ضاعف سرعة Llama 70B لـ 2.4x بدون فقد
    token واحد", section "المفهوم بالتقريب" (accept the agreed drafted tokens,
    reject the first disagreeing one and take the target's token there),
    with the temperature knob of section "كود شغّال على vLLM" taken to 0;
  * the page on LogitSpec (gist.science 2507.01449), section 2: the k
    largest entries of the last position's logits, leaving out the token
    predicted from them, are the candidates for the token after next (the
    page reports the true next-next token among the top 60 in most steps).

Readings taken where the pages are silent (each also listed in the design
notes):
  * greedy acceptance: x_j is accepted iff it is the target's argmax at
    position j; ties between equal logits go to the lower id (the T -> 0
    limit of the softmax puts equal mass on tied maxima; the lower id is the
    deterministic choice);
  * n = the first rejected position, else L; the emitted token at n is the
    target's argmax there (the corrected token, or the bonus when every draft
    is accepted);
  * the "last logits" are the target logits at position n, the ones the
    emitted token came from; the top-k list orders the other tokens by logit,
    descending, ties by the lower id, and is padded with -1 when V - 1 < k;
  * a row with a draft length outside [0, K], a drafted id outside [0, V), or
    a target row (positions 0..L) holding NaN or +inf or only -inf is
    invalid: n = -1, tokens and top-k all -1.
  Greedy decisions are exact comparisons: nothing is flagged.
"""

from dataclasses import dataclass

import numpy as np

from .verify import _row_is_bad, _widen


def argmax_lowest(l):
    """The id of the largest logit, the lowest id among ties."""
    l = np.asarray(l, dtype=np.float64)
    return int(np.nonzero(l == np.max(l))[0][0])


def top_k_after_first(l, k):
    """Ids of ranks 2..k+1 by (logit descending, id ascending), -1 padded."""
    l = np.asarray(l, dtype=np.float64)
    order = np.lexsort((np.arange(l.size), -l))
    out = np.full(k, -1, dtype=np.int64)
    take = order[1: k + 1]
    out[: take.size] = take
    return out


@dataclass
class GreedyResult:
    tokens: np.ndarray       # [B, K+1] int64: n accepted, the target's token, then -1
    n_accepted: np.ndarray   # [B], -1 for an invalid row
    topk: np.ndarray         # [B, k] int64


def greedy_verify(target, draft_tokens, draft_len, k):
    """target [B, K+1, V] logits (float or bfloat16 bit patterns);
    draft_tokens [B, K]; draft_len [B] or None; k >= 0."""
    tl = _widen(target)
    B, K1, V = tl.shape
    K = K1 - 1
    tok = np.asarray(draft_tokens, dtype=np.int64).reshape(B, K)
    lens = np.full(B, K, dtype=np.int64) if draft_len is None else np.asarray(draft_len, np.int64)
    tokens = np.full((B, K1), -1, dtype=np.int64)
    n_acc = np.full(B, -1, dtype=np.int64)
    topk = np.full((B, k), -1, dtype=np.int64)
    for b in range(B):
        L = int(lens[b])
        if not 0 <= L <= K:
            continue
        x = tok[b, :L]
        if np.any(x < 0) or np.any(x >= V):
            continue
        if any(_row_is_bad(tl[b, j]) for j in range(L + 1)):
            continue
        n = L
        for j in range(L):
            if x[j] != argmax_lowest(tl[b, j]):
                n = j
                break
        n_acc[b] = n
        tokens[b, :n] = x[:n]
        tokens[b, n] = argmax_lowest(tl[b, n])
        topk[b] = top_k_after_first(tl[b, n], k)
    return GreedyResult(tokens, n_acc, topk)
