"""Pins of the LM-head oracle (oracle/lmhead.py), CPU only."""
import numpy as np
import pytest

import workloads as wl
from oracle import lmhead as olm
from oracle import verify as ov


def test_logits_hand_case():
    """z_i = sum_k h_k W[i, k]: h = [1, 2], W rows [1, 0], [0, 1], [1, 1], [-2, 0.5]."""
    h = np.array([[1.0, 2.0]])
    W = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0], [-2.0, 0.5]])
    np.testing.assert_array_equal(olm.lmhead_logits(h, W), [[1.0, 2.0, 3.0, -1.0]])


def test_permutation_head_reduces_to_the_plain_step():
    """With W the permutation matrix of i -> (i + 1) mod V (not its own
    inverse), the logits are z_i = h_{(i+1) mod V}: the fused oracle must equal
    the plain verify step on those logits (a transposed head would give
    h_{(i-1) mod V} instead)."""
    rng = np.random.default_rng(3)
    B, K, V = 3, 2, 7
    W = np.zeros((V, V))
    W[np.arange(V), (np.arange(V) + 1) % V] = 1.0
    th = rng.normal(0, 2, size=(B, K + 1, V)).astype(np.float32)
    dh = rng.normal(0, 2, size=(B, K, V)).astype(np.float32)
    ids = rng.integers(0, V, size=(B, K)).astype(np.int32)
    T = np.array([0.7, 1.0, 1.3], np.float32)
    for D in (0.0, 0.4, 1.0):
        a = olm.lmhead_verify_sample_ref(th, dh, W, W, ids, None, T, D, seed=5)
        b = ov.verify_sample_ref(np.roll(th, -1, axis=-1), np.roll(dh, -1, axis=-1), ids, None, T,
                                 tv_budget=D, seed=5)
        assert np.array_equal(a.tokens, b.tokens) and np.array_equal(a.accepted, b.accepted)
        np.testing.assert_array_equal(a.stats, b.stats)
    g = olm.lmhead_verify_greedy_ref(th, W, ids)
    assert np.array_equal(g.argmax, np.argmax(np.roll(th, -1, axis=-1), axis=-1))


def test_short_draft_head_pads_with_zero_mass():
    """A draft head of V_d < V rows: ids past it have q = 0 (the reading of a
    draft vocabulary shorter than the target's)."""
    rng = np.random.default_rng(4)
    th = rng.normal(0, 1, size=(1, 2, 8)).astype(np.float32)
    Wt = rng.normal(0, 1, size=(6, 8))
    Wd = Wt[:4] * 1.1
    res = olm.lmhead_verify_sample_ref(th, th[:, :1], Wt, Wd, np.array([[5]], np.int32), None,
                                       np.array([1.0], np.float32), 0.0)
    assert res.status[0] & ov.ST_Q_ZERO and res.stats[0, 0, 3] == 0.0


@pytest.mark.parametrize("H", [64, 896, 3584, 4096])
def test_dyadic_inputs_make_fp32_logits_exact(H):
    """The exact workloads' premise: integer hidden components in [-2, 2]
    times weights m 2^-8 (|m| <= 255) have partial sums that fp32 represents
    exactly in any order, so fp32 sums in two different orders both equal the
    fp64 value."""
    w = wl.lmhead_case(9, B=2, K_max=1, V=64, H_t=H, H_d=min(H, 64), proposals=False)
    h, W = w.f32("target_hidden"), w.f32("target_weight")
    assert np.abs(h).max() <= 2 and np.all(h == np.rint(h))
    assert np.all(W * 256 == np.rint(W * 256)) and np.abs(W).max() < 1.0
    z64 = olm.lmhead_logits(h, W)
    prods = (h[:, :, None, :] * W[None, None, :, :]).astype(np.float32)
    fwd = np.cumsum(prods, axis=-1, dtype=np.float32)[..., -1]
    rev = np.cumsum(prods[..., ::-1], axis=-1, dtype=np.float32)[..., -1]
    np.testing.assert_array_equal(fwd, z64)
    np.testing.assert_array_equal(rev, z64)
