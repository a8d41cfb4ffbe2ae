"""CPU oracle for the speculative-sampling verify step (fp64, numpy).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in
this package.  The product path (the HIP library and its Python binding) never
touches it, and this package imports nothing from the product path.

Modules
-------
philox   Philox4x32-10 counter-based generator, written from its published
         definition (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
         easy as 1, 2, 3", SC'11).
verify   The verify step itself: logit processing, top-p, TV distance, the
         mentored-decoding mixture, acceptance, first-rejection scan,
         correction/bonus draw, and greedy verify.
confidence  The draft-side confidence step before it: each draft row's top-1
         probability and the draft length an early-stop threshold implies.
lmhead   The step fed from hidden states through the LM heads: logits as the
         fp64 product of hidden states and head weights, then verify.

Parity status of each function is stated in its docstring.  Two readings are
"parity unpinned" by the pages (the repetition-penalty formula and the top-p
boundary rule); they are pinned by hand-computed cases of the stated rule and
by brute force against a full sort, see tests/test_oracle_*.py.
"""

from .philox import philox4x32_10, uniforms_for
from .verify import (
    ST_BAD_K, ST_BAD_TEMP, ST_BAD_DRAFT_ID, ST_NONFINITE, ST_BAD_PRIOR,
    ST_Q_ZERO, ST_RESID_ZERO, ST_BAD_PARAM, ST_INVALID_MASK, FLAG_NO_BONUS,
    FLAG_PENALTY_PRIOR_ONLY, penalty_keys, softmax64, top_p_filter,
    process_dist, draft_row_over_target, tv_distance, mentored_theta, inverse_cdf, verify_sample_ref,
    verify_greedy_ref, SampleResult, GreedyResult,
)
from .confidence import top1_prob, draft_lengths, draft_confidence_ref
from .lmhead import lmhead_logits, lmhead_verify_sample_ref, lmhead_verify_greedy_ref

__all__ = [n for n in dir() if not n.startswith("_")]
