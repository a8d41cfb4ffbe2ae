"""Pins of the draft-confidence oracle ("What I Gave Up to Make Speculative
Decoding Faster", section "Confidence-guided early stop") against closed
forms, identities and brute force, each independent of the oracle's own
arithmetic."""
import math

import numpy as np
import pytest

from oracle.confidence import top1_prob, draft_lengths, draft_confidence_ref


@pytest.mark.parametrize("V", [1, 2, 7, 1000])
@pytest.mark.parametrize("T", [0.25, 1.0, 3.0])
def test_uniform_row_is_one_over_v(V, T):
    assert top1_prob(np.full(V, 1.7), T) == pytest.approx(1.0 / V, rel=1e-14)


@pytest.mark.parametrize("a,b,V,T", [(3.0, 1.0, 10, 1.0), (3.0, 1.0, 10, 0.5), (0.5, -2.0, 152064, 0.8),
                                     (10.0, 9.9, 5, 2.0)])
def test_two_level_row_closed_form(a, b, V, T):
    # one logit a, V-1 logits b: p_max = e^{a/T} / (e^{a/T} + (V-1) e^{b/T})
    z = np.full(V, b)
    z[V // 2] = a
    want = 1.0 / (1.0 + (V - 1) * math.exp((b - a) / T))
    assert top1_prob(z, T) == pytest.approx(want, rel=1e-12)


def test_temperature_and_shift_identities():
    rng = np.random.default_rng(5)
    z = rng.normal(0, 3, 4096)
    for T in (0.3, 1.0, 1.7):
        assert top1_prob(z, T) == pytest.approx(top1_prob(z / T, 1.0), rel=1e-12)
        assert top1_prob(z + 123.0, T) == pytest.approx(top1_prob(z, T), rel=1e-12)
    # hotter is flatter: the top-1 probability falls as T rises, toward 1/V
    ps = [top1_prob(z, T) for T in (0.1, 0.5, 1.0, 4.0, 100.0)]
    assert all(x > y for x, y in zip(ps, ps[1:]))
    assert ps[-1] == pytest.approx(1.0 / z.size, rel=0.2)


def test_cold_limit_counts_the_maxima():
    z = np.array([1.0, 5.0, -2.0, 5.0, 3.9])
    assert top1_prob(z, 1e-3) == pytest.approx(0.5, rel=1e-12)
    assert top1_prob(np.array([2.0, 1.0]), 1e-3) == pytest.approx(1.0, rel=1e-12)


def test_brute_force_small_rows():
    rng = np.random.default_rng(11)
    for _ in range(50):
        V = int(rng.integers(1, 9))
        z = rng.normal(0, 2, V)
        T = float(rng.uniform(0.3, 2.0))
        # unshifted softmax with plain floats
        e = [math.exp(x / T) for x in z]
        assert top1_prob(z, T) == pytest.approx(max(e) / sum(e), rel=1e-12)


def test_undefined_rows_give_nan():
    assert math.isnan(top1_prob([1.0, float("nan")], 1.0))
    assert math.isnan(top1_prob([1.0, float("inf")], 1.0))
    assert math.isnan(top1_prob([1.0, 2.0], 0.0))
    assert math.isnan(top1_prob([1.0, 2.0], float("inf")))
    assert math.isnan(top1_prob([-np.inf, -np.inf], 1.0))


def test_masked_tokens_have_zero_mass():
    # -inf logits drop out: the row behaves as the row of its finite logits
    assert top1_prob([2.0, -np.inf, 0.0, -np.inf], 1.0) == pytest.approx(1.0 / (1.0 + math.exp(-2.0)),
                                                                          rel=1e-12)


def test_draft_lengths_rule():
    top1 = np.array([[0.9, 0.7, 0.5, 0.3],    # first below 0.6 is row 2: three proposed
                     [0.9, 0.8, 0.7, 0.61],   # none below: K_max
                     [0.1, 0.9, 0.9, 0.9],    # the first row already: one
                     [0.6, 0.6, 0.59, 0.9],   # equal is not below
                     [np.nan, 0.7, 0.2, 0.1]])  # undefined never stops
    assert list(draft_lengths(top1, 0.6)) == [3, 4, 1, 3, 3]


def test_reference_on_hand_rows():
    # request 0: a confident row (two-level, p ~ 0.88) then a uniform row of 4
    # (0.25): stops after two.  request 1 at T = 2 halves the gap.
    rows = np.array([[[4.0, 0.0, 0.0, 0.0], [1.0, 1.0, 1.0, 1.0]],
                     [[4.0, 0.0, 0.0, 0.0], [9.0, 0.0, 0.0, 0.0]]])
    top1, K = draft_confidence_ref(rows, np.array([1.0, 2.0]), 0.6)
    p0 = 1.0 / (1.0 + 3.0 * math.exp(-4.0))
    p1 = 1.0 / (1.0 + 3.0 * math.exp(-2.0))
    assert top1[0, 0] == pytest.approx(p0, rel=1e-12)
    assert top1[0, 1] == pytest.approx(0.25, rel=1e-12)
    assert top1[1, 0] == pytest.approx(p1, rel=1e-12)
    assert list(K) == [2, 2]
