"""Pins for the oracle (CPU only): the pages' worked example, the closed forms
the pages state, values derived by hand from the pages' definitions,
textbook special cases, hand-computed cases of the readings, and brute force
against independent formulations.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import verify as ov
from lawtools import RowModel, marginal
from workloads import worked_example, random_case, bf16_bits_to_f32, f32_to_bf16_bits

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _example_model(D):
    w = worked_example(D=D)
    return RowModel(w.target_f32()[0], w.draft_f32()[0], T=1.0, D=D)


# --- the pages' worked example ("Speculative Decoding" note, "Eigenes Beispiel")

def test_worked_example_processing_recovers_p_and_q():
    g = _load("worked_example.json")
    m = _example_model(0.0)
    p = ov.process_dist(m.tgt[0], [], 1.0, 1.0, 1.0).p
    q = ov.process_dist(m.drf[0], [], 1.0, 1.0, 1.0).p
    np.testing.assert_allclose(p, g["p"], atol=1e-7)
    np.testing.assert_allclose(q, g["q"], atol=1e-7)


def test_worked_example_accepted_mass_and_residual_split():
    g = _load("worked_example.json")
    law = _example_model(0.0).law()
    # K = 1: a one-token sequence comes from a rejection (correction), a
    # two-token sequence from an accepted draft followed by the bonus.
    acc = np.zeros(3)
    rej = np.zeros(3)
    for seq, pr in law.items():
        if len(seq) == 2:
            acc[seq[0]] += pr
        else:
            rej[seq[0]] += pr
    np.testing.assert_allclose(acc, g["accepted_mass"], atol=1e-6)
    assert abs(rej.sum() - g["rejected_mass"]) < 1e-6
    np.testing.assert_allclose(rej, g["residual_mass_split"], atol=1e-6)
    total = acc + rej
    np.testing.assert_allclose(total, g["p"], atol=1e-6)
    # ... and not the wrong redraw from plain p
    assert np.abs(total - np.array(g["wrong_redraw_from_p"])).max() > 0.05


def test_worked_example_wrong_redraw_value_is_what_the_page_says():
    # The page's counterexample: correcting from p instead of the residual.
    # accepted [.2,.3,.1] + 0.4 * p = [.28,.50,.22]; shown here with the
    # oracle's own accepted mass so the fixture stays tied to the oracle.
    g = _load("worked_example.json")
    law = _example_model(0.0).law()
    acc = np.zeros(3)
    for seq, pr in law.items():
        if len(seq) == 2:
            acc[seq[0]] += pr
    wrong = acc + (1.0 - acc.sum()) * np.array(g["p"])
    np.testing.assert_allclose(wrong, g["wrong_redraw_from_p"], atol=1e-6)


# --- values derived by hand from "What I Gave Up...", "A knob ..."

@pytest.mark.parametrize("row", _load("mentored_example_table.json")["rows"],
                         ids=lambda r: f"D={r['D']}")
def test_mentored_table(row):
    g = _load("mentored_example_table.json")
    D = row["D"]
    m = _example_model(D)
    p = ov.process_dist(m.tgt[0], [], 1.0, 1.0, 1.0).p
    q = ov.process_dist(m.drf[0], [], 1.0, 1.0, 1.0).p
    d = ov.tv_distance(p, q)
    assert abs(d - g["d"]) < 1e-6
    th = ov.mentored_theta(d, D)
    assert abs(th - row["theta"]) < 1e-6
    # per-token acceptance probability and stats through the row function
    for x in range(3):
        r = m.run([x], [0.0, 0.0], [0.0, 0.0])
        assert abs(r.stats[0, 4] - row["pi"][x]) < 1e-6       # pi(x)
        assert abs(r.stats[0, 1] - row["theta"]) < 1e-6
    law = m.law()
    first, _ = marginal(law, 0)
    np.testing.assert_allclose([first.get(i, 0.0) for i in range(3)], row["pi"],
                               atol=1e-6)
    p_rej = sum(pr for seq, pr in law.items() if len(seq) == 1)
    assert abs(p_rej - row["p_reject"]) < 1e-6
    # accept probability of each proposal = accepted mass / q(x)
    for x in range(3):
        acc = sum(pr for seq, pr in law.items() if len(seq) == 2 and seq[0] == x)
        assert abs(acc / g["q"][x] - row["accept_prob"][x]) < 1e-6


# --- closed forms ("What I Gave Up...", "A knob ..."; "Speculative Decoding", "Warum ...")

def test_budget_zero_preserves_target_and_one_gives_draft():
    w = random_case(1, B=1, K_max=1, V=4, sigma=1.0)
    tgt, drf = w.target_f32()[0], w.draft_f32()[0]
    p = ov.process_dist(tgt[0], [], 1.0, w.temperature[0], 1.0).p
    q = ov.process_dist(drf[0], [], 1.0, w.temperature[0], 1.0).p
    for D, want in ((0.0, p), (1.0, q), (2.5, q)):
        law = RowModel(tgt, drf, T=w.temperature[0], D=D).law()
        first, _ = marginal(law, 0)
        np.testing.assert_allclose([first.get(i, 0) for i in range(4)], want,
                                   atol=2e-6)
        if D >= 1.0:   # every draft accepted
            assert sum(pr for s, pr in law.items() if len(s) == 1) < 1e-12


def test_d_zero_gives_theta_one_and_p_equal_q_never_rejects():
    assert ov.mentored_theta(0.0, 0.0) == 1.0
    assert ov.mentored_theta(0.0, 0.3) == 1.0
    z = np.array([0.3, -1.0, 2.0, 0.0], np.float32)
    m = RowModel(np.stack([z, z]), z[None], T=0.8, D=0.0)
    law = m.law()
    assert sum(pr for s, pr in law.items() if len(s) == 1) == 0.0


def test_accepted_plus_correction_gives_pi_at_intermediate_budgets():
    w = random_case(2, B=1, K_max=1, V=4, sigma=1.5, corr=0.3)
    tgt, drf, T = w.target_f32()[0], w.draft_f32()[0], w.temperature[0]
    p = ov.process_dist(tgt[0], [], 1.0, T, 1.0).p
    q = ov.process_dist(drf[0], [], 1.0, T, 1.0).p
    d = float(np.maximum(p - q, 0).sum())     # TV written as the positive part
    for D in (0.05, 0.1, 0.2):
        th = 1.0 if d <= D else D / d
        pi = (1 - th) * p + th * q
        law = RowModel(tgt, drf, T=T, D=D).law()
        first, _ = marginal(law, 0)
        np.testing.assert_allclose([first.get(i, 0) for i in range(4)], pi, atol=2e-6)
        # P(reject) = (1 - theta) d and TV(pi, p) = min(D, d)
        p_rej = sum(pr for s, pr in law.items() if len(s) == 1)
        assert abs(p_rej - (1 - th) * d) < 2e-6
        assert abs(0.5 * np.abs(pi - p).sum() - min(D, d)) < 1e-9


def test_two_positions_law_with_penalty_prefix():
    # K = 2 with the draft prefix in the penalty set: each emitted position
    # follows pi_j computed with the prefix that precedes it.
    w = random_case(3, B=1, K_max=2, V=3, sigma=1.0, corr=0.5)
    tgt, drf, T = w.target_f32()[0], w.draft_f32()[0], w.temperature[0]
    r_pen, D = 1.7, 0.1
    m = RowModel(tgt, drf, prior=[1], T=T, r_pen=r_pen, D=D)
    law = m.law()
    assert abs(sum(law.values()) - 1.0) < 1e-9

    def pi_of(j, prefix):
        pen = [1] + list(prefix)
        p = ov.process_dist(tgt[j], pen, r_pen, T, 1.0).p
        q = ov.process_dist(drf[j], pen, r_pen, T, 1.0).p
        d = float(np.maximum(p - q, 0).sum())
        th = 1.0 if d <= D else D / d
        return (1 - th) * p + th * q

    first, _ = marginal(law, 0)
    np.testing.assert_allclose([first.get(i, 0) for i in range(3)], pi_of(0, []),
                               atol=3e-6)
    for a in range(3):
        cond, tot = marginal(law, 1, cond_prefix=[a])
        if tot < 1e-9:
            continue
        got = np.array([cond.get(i, 0) for i in range(3)]) / tot
        np.testing.assert_allclose(got, pi_of(1, [a]), atol=3e-5)


def test_no_bonus_flag_emits_exactly_the_accepted_drafts():
    w = worked_example(D=1.0)
    m = RowModel(w.target_f32()[0], w.draft_f32()[0], T=1.0, D=1.0,
                 flags=ov.FLAG_NO_BONUS)
    law = m.law()
    assert all(len(s) == 1 for s in law)
    first, _ = marginal(law, 0)
    np.testing.assert_allclose([first.get(i, 0) for i in range(3)], [0.6, 0.3, 0.1],
                               atol=1e-6)


# --- temperature / softmax (textbook)

def test_two_token_softmax_is_logistic():
    for l0, l1, T in ((0.0, 1.0, 1.0), (-2.0, 3.0, 0.7), (5.0, 5.5, 2.0)):
        p = ov.softmax64(np.array([l0, l1], np.float32), T)
        want = 1.0 / (1.0 + np.exp(-(np.float32(l1) - np.float32(l0)) / np.float64(np.float32(T))))
        assert abs(p[1] - want) < 1e-15


def test_softmax_rejects_nan_inf_and_all_neg_inf():
    assert ov.softmax64(np.array([0.0, np.nan], np.float32), 1.0) is None
    assert ov.softmax64(np.array([0.0, np.inf], np.float32), 1.0) is None
    assert ov.softmax64(np.array([-np.inf, -np.inf], np.float32), 1.0) is None
    p = ov.softmax64(np.array([0.0, -np.inf], np.float32), 1.0)
    assert p[0] == 1.0 and p[1] == 0.0


# --- repetition penalty (a reading; hand-computed cases)

def test_penalty_hand_cases():
    z = np.array([2.0, -1.0, 0.5, 3.0, 0.0], np.float32)
    k = ov.penalty_keys(z, [0, 1, 0, 4], 2.0)     # duplicates: set semantics
    assert k.tolist() == [1.0, -2.0, 0.5, 3.0, 0.0]
    k = ov.penalty_keys(z, [3], 1.1)
    assert k[3] == np.float32(np.float32(3.0) / np.float32(1.1))
    assert k[3] < 3.0
    assert np.array_equal(ov.penalty_keys(z, [0, 1], 1.0), z)


def test_penalty_moves_greedy_argmax_and_uses_draft_prefix():
    V = 4
    t = np.zeros((1, 3, V), np.float32)
    t[0, 0] = [3.0, 2.9, 0.0, 0.0]     # prior {0}: 3/1.1 = 2.727 < 2.9 -> 1
    t[0, 1] = [0.0, 2.0, 0.0, 1.95]    # set {0, x_0=1}: 2/1.1 = 1.818 < 1.95 -> 3
    t[0, 2] = [0.0, 0.0, 1.0, 1.05]    # set {0, 1, x_1=3}: 1.05/1.1 < 1.0 -> 2
    ids = np.array([[1, 3]], np.int32)
    kw = dict(rep_penalty=1.1, prior_ids=np.array([0], np.int32),
              prior_offsets=np.array([0, 1], np.int32))
    g = ov.verify_greedy_ref(t, ids, **kw)
    assert g.argmax[0].tolist() == [1, 3, 2]
    assert g.accepted[0] == 2 and g.tokens[0].tolist() == [1, 3, 2]
    g2 = ov.verify_greedy_ref(t, ids, flags=ov.FLAG_PENALTY_PRIOR_ONLY, **kw)
    assert g2.argmax[0].tolist() == [1, 1, 3]
    assert g2.accepted[0] == 1 and g2.tokens[0].tolist() == [1, 1, -1]


# --- top-p (a reading; brute force against an O(V^2) formulation)

def _topp_bruteforce(keys, p, top_p):
    V = len(p)
    keep = np.zeros(V, bool)
    for k in range(V):
        above = sum(p[i] for i in range(V) if keys[i] > keys[k])
        keep[k] = above < top_p
    pk = np.where(keep, p, 0.0)
    return pk / pk.sum()


@pytest.mark.parametrize("seed", range(12))
def test_top_p_matches_bruteforce_with_ties(seed):
    rng = np.random.default_rng(seed)
    V = int(rng.integers(2, 64))
    keys = np.round(rng.normal(0, 1.5, V) * 2) / 2     # many exact ties
    keys = keys.astype(np.float32)
    T = float(rng.uniform(0.5, 2.0))
    p = ov.softmax64(keys, T)
    for tp in (1e-7, 0.3, 0.5, 0.9, 0.999):
        got, margin = ov.top_p_filter(keys, p, tp)
        want = _topp_bruteforce(keys, p, np.float64(np.float32(tp)))
        np.testing.assert_allclose(got, want, atol=1e-15)
        assert margin >= 0


def test_top_p_special_cases():
    keys = np.array([1.0, 3.0, 3.0, 2.0], np.float32)
    p = ov.softmax64(keys, 1.0)
    one, _ = ov.top_p_filter(keys, p, 1e-9)
    assert one.tolist() == [0.0, 0.5, 0.5, 0.0]      # the tied maxima are both kept
    two, _ = ov.top_p_filter(keys, p, 0.5)
    assert two.tolist() == [0.0, 0.5, 0.5, 0.0]      # mass above the pair is 0 < 0.5
    p2 = ov.softmax64(np.array([1.0, 3.0, 2.5, 2.0], np.float32), 1.0)
    three, _ = ov.top_p_filter(np.array([1.0, 3.0, 2.5, 2.0], np.float32), p2, p2[1] + 1e-12)
    assert (three > 0).tolist() == [False, True, True, False]
    full, m = ov.top_p_filter(keys, p, 1.0)
    assert np.array_equal(full, p) and m == np.inf


def test_tiny_top_p_reduces_sampling_to_greedy():
    # one-hot p and q (continuous logits: no tied maxima): sampling verify
    # with D = 0 and draft ids = argmax q is greedy verify.
    for seed in range(6):
        w = random_case(seed, B=4, K_max=3, V=50, sigma=2.0, corr=0.9,
                        n_prior=3, rep_penalty=1.3, top_p=1e-7)
        tf, df = w.target_f32(), w.draft_f32()
        # draft ids = argmax of the penalized draft rows
        ids = np.zeros_like(w.draft_ids)
        for r in range(w.B):
            prior = w.prior_ids[w.prior_offsets[r]:w.prior_offsets[r + 1]].tolist()
            for j in range(w.K_max):
                ids[r, j] = np.argmax(ov.penalty_keys(df[r, j], prior + ids[r, :j].tolist(), 1.3))
        s = ov.verify_sample_ref(tf, df, ids, w.k_per_row, w.temperature, 1e-7,
                                 1.3, w.prior_ids, w.prior_offsets, 0.0, seed, 0)
        g = ov.verify_greedy_ref(tf, ids, w.k_per_row, 1.3, w.prior_ids,
                                 w.prior_offsets)
        assert np.array_equal(s.accepted, g.accepted)
        assert np.array_equal(s.tokens, g.tokens)


# --- inverse CDF (exact over the 2^24 uniform grid)

def test_inverse_cdf_grid_frequencies():
    from lawtools import _first_true, GRID
    rng = np.random.default_rng(5)
    for _ in range(5):
        w = rng.random(6) * (rng.random(6) < 0.7)
        if w.sum() == 0:
            continue
        counts = np.zeros(6)
        k = 0
        while k < GRID:
            y = ov.inverse_cdf(w, k / GRID)[0]
            nxt = _first_true(lambda m: ov.inverse_cdf(w, m / GRID)[0] != y, k, GRID)
            counts[y] += nxt - k
            k = nxt
        np.testing.assert_allclose(counts / GRID, w / w.sum(), atol=2.0 ** -23)
        assert np.all(counts[w == 0] == 0)


# --- greedy (exact; lowest index on ties)

def test_greedy_ties_and_mismatch():
    t = np.array([[[1, 3, 3, 2], [5, 5, 0, 0], [0, 0, 0, 9]]], np.float32)
    g = ov.verify_greedy_ref(t, np.array([[1, 0]], np.int32))
    assert g.argmax[0].tolist() == [1, 0, 3]
    assert g.accepted[0] == 2 and g.tokens[0].tolist() == [1, 0, 3]
    g = ov.verify_greedy_ref(t, np.array([[2, 0]], np.int32))
    assert g.accepted[0] == 0 and g.tokens[0].tolist() == [1, -1, -1]
    g = ov.verify_greedy_ref(t, np.array([[1, 0]], np.int32), flags=ov.FLAG_NO_BONUS)
    assert g.tokens[0].tolist() == [1, 0, -1]


def test_greedy_matches_numpy_argmax_on_bf16_rows():
    rng = np.random.default_rng(0)
    t = bf16_bits_to_f32(f32_to_bf16_bits(rng.normal(0, 3, (20, 3, 5000))))
    ids = rng.integers(0, 5000, (20, 2)).astype(np.int32)
    g = ov.verify_greedy_ref(t, ids)
    assert np.array_equal(g.argmax, np.argmax(t, axis=-1))


# --- edge cases and status bits

def test_invalid_rows_and_status_bits():
    w = random_case(7, B=6, K_max=2, V=20)
    tf, df = w.target_f32().copy(), w.draft_f32().copy()
    ids = w.draft_ids.copy()
    ks = w.k_per_row.copy()
    T = w.temperature.copy()
    ks[0] = 3                      # BAD_K
    T[1] = 0.0                     # BAD_TEMP
    ids[2, 1] = 20                 # BAD_DRAFT_ID
    tf[3, 1, 5] = np.nan           # NONFINITE
    ks[4] = 0                      # bonus only: valid
    prior = np.array([0, 1, 2, 3, 4, 5, 99, 6, 7, 8, 9, 10], np.int32)
    offs = np.array([0, 2, 4, 6, 8, 10, 12], np.int32)  # row 3 has id 99
    s = ov.verify_sample_ref(tf, df, ids, ks, T, 1.0, 1.2, prior, offs, 0.3, 1, 0)
    assert s.status[0] == ov.ST_BAD_K and s.accepted[0] == -1
    assert s.status[1] == ov.ST_BAD_TEMP and (s.tokens[1] == -1).all()
    assert s.status[2] == ov.ST_BAD_DRAFT_ID
    assert s.status[3] & ov.ST_NONFINITE and s.status[3] & ov.ST_BAD_PRIOR
    assert s.status[4] == 0 and s.accepted[4] == 0 and s.tokens[4, 0] >= 0
    assert s.status[5] == 0 and s.accepted[5] >= 0


def test_q_zero_proposal_is_rejected_and_flagged():
    # top-p on the draft leaves token 2 out of q's nucleus; proposing it is a
    # caller error: status bit, rejection when pi(x) = 0.
    t = np.log(np.array([[0.2, 0.5, 0.3], [0.3, 0.3, 0.4]], np.float32))[None]
    d = np.log(np.array([[0.7, 0.25, 0.05]], np.float32))[None]
    s = ov.verify_sample_ref(t, d, np.array([[2]], np.int32), None, None, 0.9,
                             1.0, None, None, 0.0, 0, 0)
    # p restricted to its nucleus keeps token 2 (0.3), so pi(2) = p(2) > 0:
    # accepted (u * 0 < pi).
    assert s.status[0] & ov.ST_Q_ZERO
    assert s.accepted[0] == 1
    s = ov.verify_sample_ref(t, d, np.array([[2]], np.int32), None, None, 0.9,
                             1.0, None, None, 1.0, 0, 0)
    # D = 1: pi = q, pi(2) = 0 -> rejected
    assert s.accepted[0] == 0 and s.status[0] & ov.ST_Q_ZERO


def test_vocab_of_one():
    t = np.zeros((2, 3, 1), np.float32)
    d = np.zeros((2, 2, 1), np.float32)
    ids = np.zeros((2, 2), np.int32)
    s = ov.verify_sample_ref(t, d, ids, None, None, 0.5, 1.1, None, None, 0.4, 3, 9)
    assert s.accepted.tolist() == [2, 2] and s.tokens.tolist() == [[0, 0, 0]] * 2


def test_per_request_top_p_and_budget():
    """Per-request top-p and TV budget arrays act request by request exactly
    as the scalars would, and an out-of-range value invalidates only its
    request (status bit 7)."""
    import workloads as wl
    from oracle.verify import verify_sample_ref, ST_BAD_PARAM, ST_INVALID_MASK
    w = wl.random_case(41, B=6, K_max=3, V=300, dtype="f32", top_p=0.9, sigma=2.0)
    tps = np.array([0.5, 0.9, 1.0, 0.0, 1.5, 0.8], dtype=np.float32)
    Ds = np.array([0.0, 0.3, 1.0, 0.2, 0.2, np.nan], dtype=np.float32)
    args = (w.target_f32(), w.draft_f32(), w.draft_ids, w.k_per_row, w.temperature)
    got = verify_sample_ref(*args, top_p=tps, rep_penalty=1.0, tv_budget=Ds, seed=7, offset=3)
    for r in range(3):
        one = verify_sample_ref(*args, top_p=float(tps[r]), rep_penalty=1.0, tv_budget=float(Ds[r]),
                                seed=7, offset=3, rows=[r])
        assert got.accepted[r] == one.accepted[r] and got.status[r] == one.status[r]
        assert np.array_equal(got.tokens[r], one.tokens[r])
        assert np.array_equal(got.stats[r], one.stats[r])
    for r in (3, 4, 5):
        assert got.status[r] & ST_BAD_PARAM and got.status[r] & ST_INVALID_MASK
        assert got.accepted[r] == -1 and (got.tokens[r] == -1).all()


def test_q_zero_acceptance_rule_and_margin():
    """A proposal outside the draft's nucleus (q(x) = 0): the test u q(x) <
    pi(x) accepts iff pi(x) = (1 - theta) p(x) > 0 ("What I Gave Up...",
    section "A knob for accepting more draft tokens").  Hand-worked: target
    p = [.5, .3, .2] and draft q = [.1, .2, .7] as log-probabilities, T = 1,
    top-p 0.7 keep {0, 1} (p~ = [.625, .375, 0]) and {2} (q~ = [0, 0, 1]), so
    d = 1.  x = 0: D = 0.5 gives theta = 0.5, pi(0) = 0.3125 and acceptance
    whatever u, with the margin |d - D| = 0.5 (the decision flips only where
    theta reaches 1); D = 1 gives theta = 1, pi(0) = 0 and a rejection that no
    rounding can change (margin inf).  x = 1 with p~(1) = .375 > 0 likewise;
    for an x outside both nuclei pi(x) = 0 whatever theta (margin inf)."""
    from oracle.verify import verify_sample_row, ST_Q_ZERO
    lp = np.log(np.array([0.5, 0.3, 0.2])).astype(np.float32)
    lq = np.log(np.array([0.1, 0.2, 0.7])).astype(np.float32)
    tgt = np.stack([lp, lp])
    for x, D, acc, margin in ((0, 0.5, 1, 0.5), (0, 1.0, 0, np.inf), (1, 0.25, 1, 0.75)):
        for u in (0.0, 0.5, 0.999):
            rr = verify_sample_row(tgt, lq[None], np.array([x]), 1, [], 1.0, 0.7, 1.0, D,
                                   np.array([u, 0.3]), np.array([0.1, 0.6]), 3)
            assert rr.status & ST_Q_ZERO
            # (the logits are fp32 roundings of log-probabilities: 1e-7)
            assert rr.stats[0, 0] == pytest.approx(1.0, abs=1e-7)
            assert rr.stats[0, 2] == pytest.approx([0.625, 0.375][x], abs=1e-7)
            assert rr.stats[0, 3] == 0.0
            assert rr.accepted == acc
            assert rr.accept_margin[0] == pytest.approx(margin, abs=1e-7)
    # outside both nuclei: x = 2 has p~ = 0 and, with a draft nucleus of {1},
    # q~ = 0 as well
    lq2 = np.log(np.array([0.1, 0.8, 0.1])).astype(np.float32)
    rr = verify_sample_row(tgt, lq2[None], np.array([2]), 1, [], 1.0, 0.7, 1.0, 0.5,
                           np.array([0.0, 0.3]), np.array([0.1, 0.6]), 3)
    assert rr.accepted == 0 and rr.stats[0, 2] == 0.0 and rr.stats[0, 3] == 0.0
    assert rr.accept_margin[0] == np.inf


# --- a draft vocabulary shorter than the target's (Adaptive-SpecDecode-Lab
#     README, implementation section: fully mapped tokenizers; the draft's
#     logit row covers ids 0..V_d-1 only)

def _softmax_T(z, T):
    e = np.exp((np.asarray(z, np.float64) - np.max(z)) / T)
    return e / e.sum()


@pytest.mark.parametrize("D", [0.0, 0.2, 1.0])
def test_short_draft_vocabulary_law(D):
    """V = 5 target tokens, V_d = 3 draft tokens.  The enumerated law of the
    first emitted token is pi = (1 - theta) p + theta q with q extended by
    zeros over ids 3 and 4 (p and q by textbook softmax here, d = TV(p, q)):
    the tail tokens are only ever emitted as corrections, with mass
    (1 - theta) p(i), and P(reject) = (1 - theta) d."""
    tgt = np.array([[0.5, 1.0, -0.5, 1.5, 0.25], [0.0, 0.3, 1.2, -1.0, 0.6]], np.float32)
    drf = np.array([[1.0, 0.75, 0.1]], np.float32)
    T = 0.9
    p = _softmax_T(tgt[0], T)
    q = np.concatenate([_softmax_T(drf[0], T), [0.0, 0.0]])
    d = 0.5 * np.abs(p - q).sum()
    th = 1.0 if d <= D else D / d
    pi = (1 - th) * p + th * q
    law = RowModel(tgt, drf, T=T, D=D).law()
    first, _ = marginal(law, 0)
    np.testing.assert_allclose([first.get(i, 0) for i in range(5)], pi, atol=2e-6)
    p_rej = sum(pr for s, pr in law.items() if len(s) == 1)
    assert abs(p_rej - (1 - th) * d) < 2e-6
    if D < 1.0:
        assert first.get(3, 0) > 0.05 and first.get(4, 0) > 0.02


def test_short_draft_vocabulary_rows_and_proposals():
    """The oracle's processed draft row over the target's ids has q = 0 past
    V_d, with and without top-p and a penalty on a tail id; a proposal in the
    tail is a q(x) = 0 proposal (status bit, accepted iff pi(x) > 0), while an
    id beyond V is a bad draft id."""
    z = np.array([2.0, 0.5, 1.0, -1.0], np.float32)
    full = ov.draft_row_over_target(z, 7)
    assert full.shape == (7,) and np.isneginf(full[4:]).all() and np.array_equal(full[:4], z)
    for top_p in (1.0, 0.8):
        dq = ov.process_dist(full, [5, 1], 1.3, 0.7, top_p)
        assert (dq.p[4:] == 0).all() and abs(dq.p.sum() - 1.0) < 1e-12
        ref = _softmax_T(ov.penalty_keys(z, [1], 1.3), float(np.float32(0.7)))   # T as fp32
        if top_p == 1.0:
            np.testing.assert_allclose(dq.p[:4], ref, rtol=1e-12)
    tgt = np.array([[0.1, 0.2, 0.3, 0.4, 0.5, 2.5, 0.0]] * 2, np.float32)
    for D, acc in ((0.0, 1), (1.0, 0)):
        rr = ov.verify_sample_row(tgt, z[None], np.array([5]), 1, [], 1.0, 1.0, 1.0, D,
                                  np.array([0.99, 0.5]), np.array([0.5, 0.5]), 7)
        assert rr.status & ov.ST_Q_ZERO and rr.stats[0, 3] == 0.0 and rr.stats[0, 2] > 0
        assert rr.accepted == acc
    w = random_case(5, B=2, K_max=2, V=9)
    res = ov.verify_sample_ref(w.target_f32(), w.draft_f32()[:, :, :6],
                               np.array([[8, 1], [9, 0]], np.int32), tv_budget=0.3)
    assert res.status[0] & ov.ST_Q_ZERO and not res.status[0] & ov.ST_BAD_DRAFT_ID
    assert res.status[1] == ov.ST_BAD_DRAFT_ID
