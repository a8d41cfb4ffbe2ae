"""Chi-square check of the oracle's sampled output against the analytic law
(CPU only): 10^6 trials on a tiny vocabulary.  Draft ids are drawn from q by
the harness; each trial is one row of a batched call, so its Philox stream is
its own (row word of the counter).

Expected laws come from the pages' statements: accept + correction together
produce pi ("What I Gave Up...", section "A knob for accepting more draft
tokens"), so the first emitted token follows pi_0; the accepted length
follows the product of the per-position acceptance probabilities
alpha_j = 1 - (1 - theta_j) d_j (derived from the same definitions).
"""
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np
from scipy import stats

from oracle import verify as ov
from workloads import random_case

N_TRIALS = 1_000_000
CHUNK = 25_000


def _case():
    w = random_case(11, B=1, K_max=2, V=4, sigma=1.2, corr=0.4, T_range=(0.9, 0.9))
    return w.target_f32()[0], w.draft_f32()[0], float(w.temperature[0])


def _laws(D):
    tgt, drf, T = _case()
    P = [ov.process_dist(tgt[j], [], 1.0, T, 1.0).p for j in range(3)]
    Q = [ov.process_dist(drf[j], [], 1.0, T, 1.0).p for j in range(2)]
    pis, alphas = [], []
    for j in range(2):
        d = float(np.maximum(P[j] - Q[j], 0).sum())
        th = 1.0 if d <= D else D / d
        pis.append((1 - th) * P[j] + th * Q[j])
        alphas.append(1.0 - (1.0 - th) * d)
    return P, Q, pis, alphas


def _chunk(args):
    D, c = args
    tgt, drf, T = _case()
    _, Q, _, _ = _laws(D)
    rng = np.random.default_rng([77, c])
    B = CHUNK
    ids = np.stack([rng.choice(4, size=B, p=Q[0]), rng.choice(4, size=B, p=Q[1])],
                   axis=1).astype(np.int32)
    res = ov.verify_sample_ref(np.broadcast_to(tgt, (B,) + tgt.shape),
                               np.broadcast_to(drf, (B,) + drf.shape), ids,
                               None, np.full(B, T, np.float32), 1.0, 1.0, None,
                               None, D, c, 0)
    return res.tokens[:, 0].copy(), res.accepted.copy()


def _run(D):
    n_chunks = N_TRIALS // CHUNK
    workers = max(1, min(8, os.cpu_count() or 1))
    with ProcessPoolExecutor(max_workers=workers) as ex:
        parts = list(ex.map(_chunk, [(D, c) for c in range(n_chunks)]))
    first = np.concatenate([p[0] for p in parts])
    acc = np.concatenate([p[1] for p in parts])
    return first, acc


def test_chi_square_first_token_and_accepted_length():
    for D in (0.0, 0.15):
        _, _, pis, alphas = _laws(D)
        first, acc = _run(D)
        n = first.size
        obs = np.bincount(first, minlength=4)
        exp = n * pis[0]
        assert stats.chisquare(obs, exp).pvalue > 1e-4, (D, obs, exp)
        a0, a1 = alphas
        obs_n = np.bincount(acc, minlength=3)
        exp_n = n * np.array([1 - a0, a0 * (1 - a1), a0 * a1])
        assert stats.chisquare(obs_n, exp_n).pvalue > 1e-4, (D, obs_n, exp_n)
