"""Oracle of the verify step fed from hidden states through the LM heads.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The pages run the verify step on logits that an LM head computes for just the
rows being verified: "What I Gave Up to Make Speculative Decoding Faster",
section "Finding the break-even point" (the engine scores the verify rows
with a row-wise GEMV at small batch and a quantized matmul at 6-8 rows), and
the Adaptive-SpecDecode-Lab README, implementation section (one target forward
keeps the logits of the M + 1 positions being verified).  The step is then the
one of oracle/verify.py on those logits:

    target logits z_t[r, j, i] = sum_k h_t[r, j, k] * W_t[i, k]
    draft logits  z_d[r, j, i] = sum_k h_d[r, j, k] * W_d[i, k]

with W_t [V][H_t] (one output row per token id) and W_d [V_d][H_d] (a draft
vocabulary of V_d <= V ids; the rest have q = 0).  Inputs are bf16 (given here
as fp32 arrays holding bf16 values); the products and sums are taken in fp64,
which for the test inputs below is the exact value.  The fused path takes no
top-p and no repetition penalty (top_p = 1, penalty 1).
"""

import numpy as np

from .verify import verify_greedy_ref, verify_sample_ref


def lmhead_logits(hidden, weight):
    """z = hidden . weight^T in fp64: hidden [..., H], weight [V, H] -> [..., V].

    The definition written out with a library matmul as its only step.
    """
    h = np.asarray(hidden, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    return h @ w.T


def lmhead_verify_sample_ref(target_hidden, draft_hidden, target_weight, draft_weight,
                             draft_ids, k_per_row=None, temperature=None, tv_budget=0.0,
                             seed=0, offset=0, flags=0, rows=None):
    """Sampling verify on logits from the LM heads (no top-p, no penalty)."""
    zt = lmhead_logits(target_hidden, target_weight)
    zd = lmhead_logits(draft_hidden, draft_weight)
    return verify_sample_ref(zt, zd, draft_ids, k_per_row, temperature, 1.0, 1.0, None, None,
                             tv_budget, seed, offset, flags, rows=rows)


def lmhead_verify_greedy_ref(target_hidden, target_weight, draft_ids, k_per_row=None,
                             flags=0, rows=None):
    """Greedy verify on target logits from the LM head (no penalty)."""
    zt = lmhead_logits(target_hidden, target_weight)
    return verify_greedy_ref(zt, draft_ids, k_per_row, 1.0, None, None, flags, rows=rows)
