"""Plain CPU oracle for the batched speculative-sampling verify step.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The product path (the
HIP library and its Python binding) never calls it and shares no code with it.

Everything here is float64 NumPy written straight from the method's
definition on the page "Speculative Decoding للمحترف: ضاعف سرعة Llama 70B لـ
2.4x بدون فقد token واحد" (section "التعريف الرياضي من Leviathan et al.",
the acceptance probability alpha(x) and the corrected distribution p'(x)),
with the bonus token of the page "Faster LLM Inference via Sequential Monte
Carlo" (section 2, the scoring step) and the top-p knob of the first page's
vLLM section.  Where the pages leave a step open the reading taken is stated
next to the code that takes it.

Modules:
  philox  -- Philox4x32-10 counter-based generator (Salmon et al., SC'11).
  verify  -- softmax, nucleus filter, accept/first-reject scan, residual and
             bonus inverse-CDF sample, decision margins.
  smc     -- one SMC-SD step: importance log-weights from target and draft
             probabilities, bonus draw, ESS and systematic resampling.
  hispec  -- the two-stage (hierarchical) verify: the verify rule applied
             draft -> intermediate layer -> final layer.
  greedy  -- greedy verify (argmax acceptance) and the top-k of the last
             logits after the emitted token.
  produce -- the synthetic draft producer of the two-batch schedule.
"""

from .greedy import GreedyResult, argmax_lowest, greedy_verify, top_k_after_first  # noqa: F401
from .hispec import HispecResult, hispec_verify  # noqa: F401
from .philox import philox4x32_10, uniforms  # noqa: F401
from .produce import produce_drafts  # noqa: F401
from .smc import SmcResult, ess, log_weight_increment, smc_step, systematic, systematic_uniform  # noqa: F401
from .verify import (  # noqa: F401
    FLAG_BAND,
    OracleResult,
    accept,
    decide_row,
    inverse_cdf,
    nucleus,
    residual_weights,
    softmax,
    verify,
    widen_bf16,
)
