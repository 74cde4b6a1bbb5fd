"""Float64 oracle of the two-stage (hierarchical) verify step.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: the page "HiSpec: Hierarchical Speculative Decoding for LLMs",
section 2: one early-exit model gives three distributions -- a shallow
draft layer L_d, an intermediate layer L_i and the final layer L_f.  The
intermediate layer verifies the drafts first and rejects early; the final
layer then verifies what the intermediate layer let through, so that
applying the lossless speculative-decoding argument in both stages makes the
output follow the final layer exactly.

Readings taken where the page is silent (each also listed in the design
notes):
  * stage 1 is the verify step with L_i as the target and L_d as the draft:
    n1 accepted drafts plus one token drawn from max(0, p_i - q_d) (or, all
    accepted, the bonus from p_i);
  * the n1 + 1 tokens stage 1 emits follow L_i exactly, so stage 2 is the
    verify step with L_f as the target, those tokens as the drafts and L_i
    (at their positions) as the draft distribution; its n2 accepted tokens
    and its own corrected or bonus token are the output;
  * L_f is evaluated at the positions of the provisional sequence: K+2
    positions for K drafts (the logits given for positions past n1 + 1 are
    never read);
  * stage 2 draws its uniforms from Philox counter (row, position, 1, 0),
    stage 1 from (row, position, 0, 0), the verify step's stream;
  * temperature and top-p apply to every distribution of both stages;
  * a row invalid in stage 1 stays invalid (n = -1).
  The window of N_i provisionally accepted tokens gathered over several
  rounds before the final check is a scheduling policy of the serving loop
  and is not part of one step.
"""

from dataclasses import dataclass

import numpy as np

from .verify import _widen, verify


@dataclass
class HispecResult:
    tokens: np.ndarray       # [B, K+2] int64: n2 accepted + 1, then -1
    n_accepted: np.ndarray   # [B] n2, -1 for an invalid row
    n_stage1: np.ndarray     # [B] n1, -1 for an invalid row
    stage1: object           # OracleResult of stage 1
    stage2: object           # OracleResult of stage 2

    @property
    def flagged(self):
        return self.stage1.flagged | self.stage2.flagged


def hispec_verify(final, inter, draft, draft_tokens, draft_len, temperature, top_p, seed):
    """final [B, K+2, V] (L_f), inter [B, K+1, V] (L_i), draft [B, K, V]
    (L_d) logits; draft_tokens [B, K]; draft_len [B] or None."""
    fl = _widen(final)
    il = _widen(inter)
    B, K1, V = il.shape
    K = K1 - 1
    if fl.shape != (B, K + 2, V):
        raise ValueError("final-layer logits must be [B, K+2, V]")
    s1 = verify(il, draft, draft_tokens, draft_len, temperature, top_p, seed, stage=0)
    # stage 2 drafts: the n1 + 1 tokens stage 1 emitted
    tok2 = np.where(s1.tokens >= 0, s1.tokens, 0)
    len2 = np.where(s1.n_accepted >= 0, s1.n_accepted + 1, -1)
    s2 = verify(fl, il, tok2, len2, temperature, top_p, seed, stage=1)
    return HispecResult(s2.tokens, s2.n_accepted, s1.n_accepted, s1, s2)
