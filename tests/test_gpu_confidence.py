"""Draft-side confidence on the GPU (sd_draft_confidence) against the fp64
oracle ("What I Gave Up to Make Speculative Decoding Faster", section
"Confidence-guided early stop"): each row's top-1 probability to a relative
2e-5 (fp32 exponentials, fp64 sums), and the draft lengths exactly wherever
no row lies within that tolerance of the threshold."""
import math

import numpy as np
import pytest

import oracle
import workloads as wl
from parity import to_device

pytestmark = pytest.mark.gpu

RTOL = 2e-5


def _sdv():
    import speculative_sampling_verify_temp_amd as sdv
    return sdv


def _check(w, top1, K, threshold, rows=None):
    df = w.draft_f32()
    Bc = range(w.B) if rows is None else rows
    checked = 0
    for r in Bc:
        T = float(w.temperature[r])
        ref = [oracle.top1_prob(df[r, j], T) for j in range(w.K_max)]
        for j in range(w.K_max):
            if math.isnan(ref[j]):
                assert math.isnan(top1[r, j]), (r, j, top1[r, j])
            else:
                assert top1[r, j] == pytest.approx(ref[j], rel=RTOL, abs=1e-9), (r, j)
        near = any(abs(x - threshold) <= 4 * RTOL * max(abs(threshold), 1e-30) for x in ref if not math.isnan(x))
        if not near:
            assert K[r] == oracle.draft_lengths(np.array([ref]), threshold)[0], (r, ref, K[r])
            checked += 1
    return checked


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V", [1, 7, 300, 3001, 20011])
def test_confidence_matches_oracle(dtype, V):
    sdv = _sdv()
    w = wl.random_case(900 + V % 97, B=24, K_max=5, V=V, dtype=dtype, sigma=3.0,
                       T_range=(0.3, 1.5))
    d = to_device(w)
    thr = 0.3
    top1, K = sdv.draft_confidence(d["draft"], d["temperature"], thr)
    n = _check(w, top1.cpu().numpy(), K.cpu().numpy(), thr)
    assert n >= 20


def test_confidence_edge_rows():
    """NaN and +inf logits, masked (-inf) tokens, an all-masked row, bad
    temperatures, no temperature array, and thresholds that never or always
    stop."""
    import torch
    sdv = _sdv()
    w = wl.random_case(931, B=6, K_max=3, V=1000, dtype="f32", sigma=2.0)
    x = w.draft.copy()
    x[0, 0, 17] = np.nan
    x[0, 1, 5] = np.inf
    x[1, 0, :500] = -np.inf
    x[1, 1, :] = -np.inf
    x[1, 2, :] = -np.inf           # a NaN among masked tokens only
    x[1, 2, 999] = np.nan
    w.draft[...] = x
    w.temperature[2] = 0.0
    w.temperature[3] = np.inf
    d = to_device(w)
    top1, K = sdv.draft_confidence(d["draft"], d["temperature"], 0.5)
    t = top1.cpu().numpy()
    assert math.isnan(t[0, 0]) and math.isnan(t[0, 1]) and not math.isnan(t[0, 2])
    assert not math.isnan(t[1, 0]) and math.isnan(t[1, 1]) and math.isnan(t[1, 2])
    assert np.isnan(t[2]).all() and np.isnan(t[3]).all()
    _check(w, t, K.cpu().numpy(), 0.5)
    # no temperature: T = 1
    top1n, _ = sdv.draft_confidence(d["draft"], None, 0.5)
    df = w.draft_f32()
    assert top1n[4, 2].item() == pytest.approx(oracle.top1_prob(df[4, 2], 1.0), rel=RTOL)
    # threshold 0 never stops, threshold 2 stops at the first defined row
    _, K0 = sdv.draft_confidence(d["draft"], d["temperature"], 0.0)
    assert (K0.cpu().numpy() == w.K_max).all()
    _, K2 = sdv.draft_confidence(d["draft"], d["temperature"], 2.0)
    assert list(K2.cpu().numpy()[4:]) == [1, 1]


def test_confidence_padded_rows():
    """Rows with a leading dimension past V (padding never read as logits)."""
    import torch
    sdv = _sdv()
    w = wl.random_case(932, B=4, K_max=2, V=1003, dtype="bf16", sigma=3.0)
    d = to_device(w)
    full = d["draft"]
    buf = torch.full((4, 2, 1024 + 8), 0x7F80, dtype=torch.int16, device=full.device).view(torch.bfloat16)
    buf[..., :1003] = full
    top1, K = sdv.draft_confidence(buf[..., :1003], d["temperature"], 0.3)
    _check(w, top1.cpu().numpy(), K.cpu().numpy(), 0.3)


def test_confidence_full_size_sampled():
    """256 requests x 8 draft rows of V = 152064 bf16 (the verify step's
    draft rows): eight requests checked row by row."""
    sdv = _sdv()
    w = wl.config4()
    d = to_device(w)
    top1, K = sdv.draft_confidence(d["draft"], d["temperature"], 0.6)
    t, k = top1.cpu().numpy(), K.cpu().numpy()
    rows = [0, 1, 37, 100, 128, 200, 254, 255]
    assert _check(w, t, k, 0.6, rows=rows) >= 6
    assert np.isfinite(t).all() and ((k >= 1) & (k <= 8)).all()
