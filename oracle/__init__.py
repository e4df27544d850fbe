"""CPU oracle for the DSpark draft-head-and-verify chain -- TEST INFRASTRUCTURE.

This package is a plain, slow, obviously-correct float64 (numpy) restatement of
what the hot path computes, used to check the HIP library. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. The product path never calls it, and it shares no code with the HIP
path (``draft_verify_sampling_markov_amd``): the two meet only in the seeded
input generators of ``synth``.

Sources (cited by page title and section):
  * "DSpark: Confidence-Scheduled Speculative Decoding with Semi-Autoregressive
    Generation", technical digest at zhao9797.github.io ("DSpark digest"):
    sections "Architecture (drafter)", "Verification scheduling (system side)",
    "Benchmark (offline)", "Infra (online production @ DeepSeek-V4)".
  * "SGLang integrates DSpark" blog (aihot.vn, Vietnamese; aihot.virxact.com,
    Chinese) ("SGLang DSpark blog"): sections "Verify modes", "Ragged verify
    under full CUDA graphs", "Cost-table profiling".
  * "vLLM adaptive verification with DSpark" (agentlenshq.com) ("vLLM adaptive
    verification page"): sections "DSpark confidence-scheduling mechanism",
    "Technical implementation & CUDA graphs", "Configuration & reproduction".

Where the pages stop, the acceptance rule min(1, p_t/p_d), the normalised
residual max(0, p_t - p_d), the bonus token, the Philox stream and inverse-CDF
sampling are the standard speculative-sampling definitions the method relies on
(its digest requires exact per-token softmax probabilities so that rejection
sampling applies).

Parity pins: every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_*.py`` against something other than itself (a library
routine, a closed form, brute force, or a worked example the pages print). The
one result with no independent pin is the exact token sequence of a whole
chain beyond those stage pins ("parity unpinned" for the chain as a whole; each
stage is pinned).
"""
from .philox import philox4x64_10, uniform24, uniforms, PURPOSE_DRAFT, PURPOSE_ACCEPT, \
    PURPOSE_RESIDUAL, PURPOSE_BONUS
from .markov import widen, markov_logits, inverse_cdf, markov_step, markov_draft
from .confidence import confidence
from .schedule import cost_table_prepare, quantize_survival, schedule_topb, \
    SCHED_ARGMAX, SCHED_GREEDY, SCHED_FIXED
from .pack import pack_ragged
from .verify import verify, VERIFY_STATIC, VERIFY_COMPACT, VERIFY_CAP_ACCEPT
from .chain import chain, decode
from .observe import analytic_acceptance, new_stats, observe, ece, utilisation
from .calibrate import sts_fit, ece_of
from . import calibrate

__all__ = [
    "philox4x64_10", "uniform24", "uniforms", "PURPOSE_DRAFT", "PURPOSE_ACCEPT",
    "PURPOSE_RESIDUAL", "PURPOSE_BONUS", "widen", "markov_logits", "inverse_cdf",
    "markov_step", "markov_draft", "confidence", "cost_table_prepare",
    "quantize_survival", "schedule_topb", "SCHED_ARGMAX", "SCHED_GREEDY",
    "SCHED_FIXED", "pack_ragged", "verify", "VERIFY_STATIC", "VERIFY_COMPACT",
    "VERIFY_CAP_ACCEPT", "chain", "decode", "analytic_acceptance", "new_stats", "observe",
    "ece", "utilisation", "sts_fit", "ece_of", "calibrate",
]
