"""Draft-side confidence: the top-1 probability of each draft row and the
draft length it implies.  Plain fp64 numpy.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py): the product path never
imports this module.

Page: "What I Gave Up to Make Speculative Decoding Faster", section
"Confidence-guided early stop".  After each draft token the draft takes,
from the logits it already has, the probability of its most likely token;
when that falls below a threshold it proposes nothing more, and the
low-confidence token itself is still sent to the target for verification.
No extra forward pass is spent on it.  (The page's run used 0.6.)

Readings where the section is silent (each is listed in the design doc):
  * the distribution is softmax(z / T) of the draft row at the request's
    temperature T, with no repetition penalty and no top-p: the section
    names only the logits;
  * "below" is strict: row j stops the proposal when top1_j < threshold;
  * a request proposes K_r = j + 1 tokens when j is its first row below the
    threshold, and K_max when no row is;
  * a logit of -inf is a masked token (probability 0); a row holding a NaN
    or +inf logit, a row with no finite logit, or a request with T not in
    (0, inf) has no defined top-1 probability: NaN, which never stops a
    proposal.

Parity: pinned by closed forms (uniform rows, two-level rows), the
temperature scaling identity, and brute force over scipy-free explicit sums
(tests/test_oracle_confidence.py).
"""
import math

import numpy as np


def top1_prob(z, T):
    """max_i softmax(z / T)_i = 1 / sum_i exp((z_i - max z) / T), in fp64.

    z: one row of logits (any float dtype); T: temperature > 0."""
    z = np.asarray(z, dtype=np.float64)
    T = float(T)
    if z.size == 0 or not (T > 0.0 and math.isfinite(T)) or np.any(np.isnan(z)) or np.any(z == np.inf):
        return float("nan")
    m = z.max()
    if m == -np.inf:
        return float("nan")
    return float(1.0 / np.exp((z - m) / T).sum())


def draft_lengths(top1, threshold):
    """K_r per request from its rows' top-1 probabilities [B][K_max]: the
    first row strictly below the threshold is the last one proposed."""
    top1 = np.asarray(top1, dtype=np.float64)
    B, K = top1.shape
    out = np.full(B, K, dtype=np.int32)
    for r in range(B):
        for j in range(K):
            if top1[r, j] < threshold:   # NaN compares false: no stop
                out[r] = j + 1
                break
    return out


def draft_confidence_ref(rows, temperature, threshold):
    """rows [B][K_max][V] (fp32 values, bf16 already widened), temperature
    [B] or None (T = 1): returns (top1 [B][K_max] fp64, K [B] int32)."""
    rows = np.asarray(rows)
    B, K, _ = rows.shape
    top1 = np.empty((B, K), dtype=np.float64)
    for r in range(B):
        T = 1.0 if temperature is None else float(temperature[r])
        for j in range(K):
            top1[r, j] = top1_prob(rows[r, j], T)
    return top1, draft_lengths(top1, threshold)
