"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the GPU.

Sizes: small cases span several 4096-logit block steps with ragged tails;
the full-size workloads (V = 152064 / 151936) run in the launch
configuration the bench times, with the oracle evaluated on sampled rows.
"""
import numpy as np
import pytest

import workloads as wl
from parity import (compare_greedy, compare_sample, gpu_greedy, gpu_sample,
                    oracle_greedy, oracle_sample, to_device, EPS)

pytestmark = pytest.mark.gpu


def _sdv():
    import speculative_sampling_verify_temp_amd as sdv
    return sdv


# ---------------------------------------------------------------- Philox

def test_uniforms_bit_exact():
    from oracle.philox import uniforms_for
    sdv = _sdv()
    for seed, off in ((0, 0), (12345678901234, 7), (2**64 - 1, 2**40 + 3)):
        u, v = sdv.debug_uniforms(seed, off, 1000, 33)
        rr, jj = np.meshgrid(np.arange(1000), np.arange(33), indexing="ij")
        uo, vo = uniforms_for(seed, off, rr, jj)
        assert np.array_equal(u.cpu().numpy().astype(np.float64), uo)
        assert np.array_equal(v.cpu().numpy().astype(np.float64), vo)


# ---------------------------------------------------------------- greedy

GREEDY_CASES = [
    dict(seed=1, B=6, K_max=3, V=5003, dtype="bf16"),
    dict(seed=2, B=5, K_max=4, V=9000, dtype="f32", ragged=True),
    dict(seed=3, B=4, K_max=2, V=20011, dtype="bf16", n_prior=40, rep_penalty=1.3),
    dict(seed=4, B=4, K_max=5, V=4096, dtype="f32", n_prior=9, rep_penalty=0.8),
    dict(seed=5, B=3, K_max=1, V=1, dtype="bf16"),
    dict(seed=6, B=4, K_max=0, V=777, dtype="f32"),
]


@pytest.mark.parametrize("case", GREEDY_CASES, ids=lambda c: f"seed{c['seed']}")
@pytest.mark.parametrize("flags", [0, 1, 2])
def test_greedy_small(case, flags):
    w = wl.random_case(**case, flags=flags)
    # plant exact ties and make some drafts match the target argmax
    tf = w.target_f32()
    rng = np.random.default_rng(case["seed"])
    for r in range(w.B):
        for j in range(w.K_max + 1):
            if w.V > 2 and rng.random() < 0.3:
                a, b = rng.choice(w.V, 2, replace=False)
                w.target[r, j, max(a, b)] = w.target[r, j, int(np.argmax(tf[r, j]))]
        for j in range(w.K_max):
            if rng.random() < 0.7:
                w.draft_ids[r, j] = int(np.argmax(w.target_f32()[r, j]))
    g = gpu_greedy(w)
    o = oracle_greedy(w)
    compare_greedy(g, o, range(w.B))


@pytest.mark.parametrize("K", [1, 2, 4, 8])
def test_greedy_config3_batched(K):
    w = wl.config3(K=K, call=0, B=48)
    g = gpu_greedy(w)
    o = oracle_greedy(w)
    compare_greedy(g, o, range(w.B))


@pytest.mark.parametrize("K", [1, 8])
def test_greedy_config3_batch_one_calls(K):
    for call in range(1, 13):
        w = wl.config3(K=K, call=call, B=1)
        compare_greedy(gpu_greedy(w), oracle_greedy(w), [0])


def test_greedy_invalid_rows():
    w = wl.random_case(8, B=5, K_max=3, V=3000, dtype="bf16", n_prior=4, rep_penalty=1.2)
    w.k_per_row[0] = 4                      # bad K
    w.draft_ids[1, 1] = 3000                # bad draft id
    w.target[2, 2, 17] = 0x7FC0             # NaN
    w.prior_ids[3 * 4] = -5                 # bad prior id (ignored)
    compare_greedy(gpu_greedy(w), oracle_greedy(w), range(w.B))


# ---------------------------------------------------------------- sampling

def test_worked_example_all_budgets_and_proposals():
    for D in (0.0, 0.1, 0.2, 0.4, 0.5, 1.0):
        for x in range(3):
            for seed in range(4):
                w = wl.worked_example(draft_id=x, D=D, seed=seed)
                g, o = gpu_sample(w), oracle_sample(w)
                c, f = compare_sample(g, o, w)
                assert c + f == 1


PROC_CASES = [
    dict(seed=11, B=2, K_max=2, V=1000, dtype="f32", top_p=0.9),
    dict(seed=12, B=2, K_max=3, V=5003, dtype="bf16", top_p=0.8, n_prior=30, rep_penalty=1.25),
    dict(seed=13, B=2, K_max=2, V=20000, dtype="bf16", sigma=3.0, top_p=0.95, T_range=(0.5, 1.0)),
    dict(seed=14, B=2, K_max=2, V=9001, dtype="f32", sigma=0.3, top_p=0.5),
    dict(seed=15, B=2, K_max=1, V=4099, dtype="bf16", sigma=6.0, top_p=0.3, n_prior=100, rep_penalty=1.1),
    dict(seed=16, B=1, K_max=2, V=3000, dtype="f32", top_p=1.0, n_prior=50, rep_penalty=2.0),
]


@pytest.mark.parametrize("case", PROC_CASES, ids=lambda c: f"seed{c['seed']}")
def test_processed_rows_match_oracle(case):
    from oracle import verify as ov
    sdv = _sdv()
    w = wl.random_case(**case)
    d = to_device(w)
    p, q = sdv.debug_process_rows(d["target"], d["draft"], d["draft_ids"], d["k_per_row"],
                                  d["temperature"], w.top_p, w.rep_penalty, d["prior_ids"],
                                  d["prior_offsets"], w.flags)
    p, q = p.cpu().numpy(), q.cpu().numpy()
    tf, df = w.target_f32(), w.draft_f32()
    checked = 0
    for r in range(w.B):
        prior = [] if w.prior_ids is None else [
            int(t) for t in w.prior_ids[w.prior_offsets[r]:w.prior_offsets[r + 1]]]
        for j in range(int(w.k_per_row[r]) + 1):
            pen = prior + [int(t) for t in w.draft_ids[r, :j]]
            for side, rowv, got in (("p", tf[r, j], p[r, j]), ("q", df[r, j] if j < w.K_max else None,
                                                               q[r, j] if j < w.K_max else None)):
                if rowv is None or (side == "q" and j >= w.k_per_row[r]):
                    continue
                dd = ov.process_dist(rowv, pen, w.rep_penalty, w.temperature[r], w.top_p)
                if dd.topp_margin < EPS:
                    continue
                np.testing.assert_allclose(got, dd.p, atol=5e-7, rtol=1e-6,
                                           err_msg=f"row {r} {side}{j}")
                # kept set (fp32 may underflow far-tail probabilities to 0)
                sel = (dd.p == 0) | (dd.p > 1e-30)
                assert np.array_equal((got > 0)[sel], (dd.p > 0)[sel]), f"kept set row {r} {side}{j}"
                checked += 1
    assert checked > 0


@pytest.mark.parametrize("D", [0.0, 0.5, 1.0])
def test_config1(D):
    for seed in range(8):
        w = wl.config1(seed=seed, D=D, philox_seed=seed)
        compare_sample(gpu_sample(w), oracle_sample(w), w)


SWEEP = [
    dict(B=6, K_max=3, V=5003, dtype="bf16", D=0.3, top_p=0.9, n_prior=20, rep_penalty=1.2, ragged=True),
    dict(B=6, K_max=4, V=4096, dtype="f32", D=0.0, T_range=(0.3, 2.0)),
    dict(B=5, K_max=2, V=12289, dtype="bf16", D=0.75, top_p=0.9, sigma=3.0, corr=0.9),
    dict(B=5, K_max=5, V=999, dtype="f32", D=1.0, top_p=0.7, n_prior=5, rep_penalty=1.5),
    dict(B=4, K_max=3, V=8191, dtype="bf16", D=0.1, sigma=0.5, corr=0.2, flags=1),
    dict(B=4, K_max=3, V=3001, dtype="f32", D=0.6, n_prior=30, rep_penalty=1.1, flags=2, ragged=True),
    dict(B=4, K_max=2, V=40000, dtype="bf16", D=0.25, top_p=0.99, sigma=2.0),
]


@pytest.mark.parametrize("i", range(len(SWEEP)))
def test_sample_sweep(i):
    tot_c = tot_f = 0
    for seed in range(3):
        w = wl.random_case(100 * i + seed, **SWEEP[i])
        c, f = compare_sample(gpu_sample(w), oracle_sample(w), w)
        tot_c += c
        tot_f += f
    print(f"sweep {i}: checked {tot_c} rows, near-tie rows {tot_f}")
    # near-ties that can change a row's output are rare (the oracle flags at
    # most 1 of 12..18 rows per case here): nearly every row is compared
    assert tot_c >= 0.9 * (tot_c + tot_f)


def test_sample_edge_cases():
    w = wl.random_case(21, B=8, K_max=3, V=2000, dtype="bf16", D=0.4, top_p=0.9,
                       n_prior=3, rep_penalty=1.2)
    w.k_per_row[:] = 3
    w.k_per_row[0] = -1                 # bad K
    w.temperature[1] = 0.0              # bad temperature
    w.draft_ids[2, 0] = -3              # bad draft id
    w.target[3, 3, 5] = 0x7F80          # +inf logit
    w.draft[4, 1, :] = 0xFF80           # draft row of only -inf
    w.k_per_row[5] = 0                  # bonus only
    w.prior_ids[6 * 3] = 99999          # bad prior id: ignored
    g, o = gpu_sample(w), oracle_sample(w)
    compare_sample(g, o, w)
    assert g["status"][0] == 1 and g["status"][1] == 2 and g["status"][2] == 4
    assert g["status"][3] & 8 and g["status"][4] & 8 and g["status"][6] & 16


def test_sample_q_zero_and_vocab_one():
    t = np.log(np.array([[0.2, 0.5, 0.3], [0.3, 0.3, 0.4]], np.float32))[None]
    d = np.log(np.array([[0.7, 0.25, 0.05]], np.float32))[None]
    for D in (0.0, 1.0):
        w = wl.Workload("qzero", "f32", t.copy(), d.copy(), np.array([[2]], np.int32),
                        np.array([1], np.int32), np.array([1.0], np.float32), top_p=0.9,
                        tv_budget=D)
        compare_sample(gpu_sample(w), oracle_sample(w), w)
    w = wl.Workload("v1", "f32", np.zeros((2, 3, 1), np.float32), np.zeros((2, 2, 1), np.float32),
                    np.zeros((2, 2), np.int32), np.full(2, 2, np.int32), np.ones(2, np.float32),
                    top_p=0.5, rep_penalty=1.1, tv_budget=0.4, seed=3, offset=9)
    compare_sample(gpu_sample(w), oracle_sample(w), w)


def test_config2_calls():
    tot = [0, 0]
    for call in range(12):
        for D in (0.0, 0.5, 0.75, 1.0):
            w = wl.config2(call=call, D=D)
            c, f = compare_sample(gpu_sample(w), oracle_sample(w), w)
            tot[0] += c
            tot[1] += f
    print(f"config2: checked {tot[0]}, near-tie {tot[1]}")
    assert tot[0] >= 0.9 * (tot[0] + tot[1])


@pytest.fixture(scope="module")
def cfg4():
    return wl.config4()


@pytest.fixture(scope="module")
def cfg4_odd():
    return wl.config4(odd_share=0.15)


def _full_size_properties(g, w):
    """Properties every valid row of a full-size call must have."""
    assert ((g["accepted"] >= 0) & (g["accepted"] <= w.k_per_row)).all()
    for r in range(w.B):
        n = g["accepted"][r]
        assert np.array_equal(g["tokens"][r, :n], w.draft_ids[r, :n])
        assert 0 <= g["tokens"][r, n] < w.V


def test_config4_full_size_sampled_rows(cfg4):
    """The measured workload at full size: every row the GPU rejects among the
    first 96 plus every 8th row, compared with the oracle."""
    w = cfg4
    g = gpu_sample(w)
    rej = [r for r in range(96) if g["accepted"][r] < w.k_per_row[r]]
    rows = sorted(set(rej) | set(range(0, w.B, 8)))
    o = oracle_sample(w, rows=rows)
    c, f = compare_sample(g, o, w, rows=rows)
    print(f"config4: compared {len(rows)} rows ({len(rej)} rejecting), checked {c}, "
          f"near-tie {f}; mean accepted {g['accepted'].mean():.3f}")
    assert len(rows) >= 64 and c >= 0.9 * len(rows)
    assert (g["status"] & 0x8F).sum() == 0
    _full_size_properties(g, w)


@pytest.mark.parametrize("D", [0.75, 0.0])
def test_config4_full_size_odd_proposals(cfg4_odd, D):
    """Full-size single-pass calls whose proposals include ids drawn uniformly
    from [0, V) and from the prior ids (15% of positions): q(x) = 0, p(x) = 0
    and penalized proposals, and at D = 0 (lossless) a rejection in nearly
    every row, so the full-vocabulary correction draw is compared row by row."""
    w = cfg4_odd.with_(tv_budget=D)
    g = gpu_sample(w)
    rows = list(range(80))
    o = oracle_sample(w, rows=rows)
    c, f = compare_sample(g, o, w, rows=rows)
    rej = sum(int(o.accepted[r] < w.k_per_row[r]) for r in rows)
    # decided positions (j <= n) whose proposal falls in each branch
    qz = pz = pen = 0
    for r in rows:
        n = int(o.accepted[r])
        prior = set(w.prior_ids[w.prior_offsets[r]:w.prior_offsets[r + 1]].tolist())
        for j in range(min(n + 1, w.K_max)):
            x = int(w.draft_ids[r, j])
            qz += o.stats[r, j, 3] == 0.0
            pz += o.stats[r, j, 2] == 0.0
            pen += x in prior or x in set(w.draft_ids[r, :j].tolist())
    print(f"config4 odd D={D}: checked {c}, near-tie {f}, rejecting rows {rej}; decided "
          f"positions with q(x)=0 {qz}, p(x)=0 {pz}, penalized x {pen}")
    assert c >= 0.9 * len(rows)
    assert rej >= (64 if D == 0.0 else 40)
    assert qz >= 10 and pz >= 10 and pen >= 3
    assert (g["status"] & 0x8F).sum() == 0
    _full_size_properties(g, w)


@pytest.mark.parametrize("forced", [False, True])
def test_config5_full_size_sampled_rows(forced):
    """Config 5 at full size.  Under its statistics (N(0, 3^2) logits, T = 0.7)
    the draft's top-1 probability is already below 0.6 at the first position
    in most rows, so the early-stop rule gives K_r = 1 to 474 of the 512 rows
    (the oracle's own rule reproduces the workload's K exactly); the forced
    variant (K_r ~ U{1..8}) carries the ragged coverage."""
    from oracle import draft_confidence_ref
    w = wl.config5(forced_ragged=forced)
    hist = np.bincount(w.k_per_row, minlength=9)
    if not forced:
        _, k_rule = draft_confidence_ref(w.draft_f32(), w.temperature, 0.6)
        assert np.array_equal(w.k_per_row, k_rule)
        assert hist[1] == 474 and hist[1:].sum() == w.B
    else:
        assert (hist[1:] > 0).all()
    g = gpu_sample(w)
    rows = list(range(0, w.B, 4))
    o = oracle_sample(w, rows=rows)
    c, f = compare_sample(g, o, w, rows=rows)
    rej = sum(int(o.accepted[r] < w.k_per_row[r]) for r in rows)
    print(f"config5 forced={forced}: K hist {hist.tolist()}, compared {len(rows)}, checked {c}, "
          f"near-tie {f}, rejecting {rej}")
    assert c >= 0.9 * len(rows)
    _full_size_properties(g, w)


def test_repeat_runs_identical():
    w = wl.random_case(31, B=8, K_max=4, V=30011, dtype="bf16", D=0.5, top_p=0.9,
                       n_prior=10, rep_penalty=1.1, sigma=3.0)
    d = to_device(w)
    a = gpu_sample(w, dev=d)
    for _ in range(3):
        b = gpu_sample(w, dev=d)
        for k in ("accepted", "tokens", "status"):
            assert np.array_equal(a[k], b[k])
        assert np.array_equal(a["stats"], b["stats"])


def test_gpu_chi_square_law():
    """10^6 trials on V = 4, K = 2: first emitted token vs pi_0 and the
    accepted length vs the product of acceptance probabilities."""
    import torch
    from scipy import stats as ss
    from oracle import verify as ov
    w0 = wl.random_case(11, B=1, K_max=2, V=4, sigma=1.2, corr=0.4, T_range=(0.9, 0.9))
    tgt, drf, T = w0.target_f32()[0], w0.draft_f32()[0], float(w0.temperature[0])
    N = 1_000_000
    for D in (0.0, 0.15):
        P = [ov.process_dist(tgt[j], [], 1.0, T, 1.0).p for j in range(3)]
        Q = [ov.process_dist(drf[j], [], 1.0, T, 1.0).p for j in range(2)]
        pis, al = [], []
        for j in range(2):
            d = float(np.maximum(P[j] - Q[j], 0).sum())
            th = 1.0 if d <= D else D / d
            pis.append((1 - th) * P[j] + th * Q[j])
            al.append(1 - (1 - th) * d)
        rng = np.random.default_rng(5)
        ids = np.stack([rng.choice(4, N, p=Q[0]), rng.choice(4, N, p=Q[1])], 1).astype(np.int32)
        dev = "cuda"
        tt = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(np.pad(tgt, ((0, 0), (0, 4))), (N, 3, 8)))).to(dev)[..., :4]
        dd = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(np.pad(drf, ((0, 0), (0, 4))), (N, 2, 8)))).to(dev)[..., :4]
        sdv = _sdv()
        acc, tok, st, _ = sdv.verify_sample(tt, dd, torch.from_numpy(ids).to(dev), None,
                                            torch.full((N,), T, device=dev), 1.0, 1.0, None,
                                            None, D, 17, 0)
        first = tok[:, 0].cpu().numpy()
        a = acc.cpu().numpy()
        assert ss.chisquare(np.bincount(first, minlength=4), N * pis[0]).pvalue > 1e-4
        exp_n = N * np.array([1 - al[0], al[0] * (1 - al[1]), al[0] * al[1]])
        assert ss.chisquare(np.bincount(a, minlength=3), exp_n).pvalue > 1e-4


def _fast_fallbacks(w):
    """Units of workload w that the single-pass kernel hands to its fallback."""
    import torch
    import speculative_sampling_verify_temp_amd as sdv
    d = to_device(w)
    args = sdv.make_args(d["target"], d["draft"], d["draft_ids"], d["k_per_row"],
                         d["temperature"], w.top_p, w.rep_penalty, d["prior_ids"],
                         d["prior_offsets"], w.tv_budget, w.seed, w.offset, w.flags)
    assert sdv.phase_kernel(args, 0) == "k_pair_fast"
    ws = sdv.alloc_workspace(args, d["target"].device)
    B = w.target.shape[0]
    acc = torch.empty(B, dtype=torch.int32, device=d["target"].device)
    tok = torch.empty((B, w.target.shape[1]), dtype=torch.int32, device=d["target"].device)
    sdv.run_phase(args, ws, 0, acc, tok)
    return sdv.fallback_units(args, ws)


@pytest.mark.parametrize("case", ["rep_below_one", "many_entries"])
def test_single_pass_penalty_sets(case):
    """Penalty sets settled after each stream, on the single-pass path: a
    penalty below 1 (penalized keys rise and may enter the nucleus), and more
    penalty entries than threads per block drawn from few distinct ids."""
    if case == "rep_below_one":
        kw = dict(B=4, K_max=3, V=20011, dtype="bf16", D=0.5, top_p=0.9, sigma=3.0,
                  T_range=(0.5, 0.9), n_prior=60, rep_penalty=0.8)
    else:
        kw = dict(B=3, K_max=3, V=30000, dtype="bf16", D=0.5, top_p=0.9, sigma=3.0,
                  T_range=(0.5, 0.9), n_prior=1500, prior_pool=150, rep_penalty=1.3)
    tot = [0, 0]
    for seed in range(3):
        w = wl.random_case(500 + seed, **kw)
        assert _fast_fallbacks(w) == 0
        c, f = compare_sample(gpu_sample(w), oracle_sample(w), w)
        tot[0] += c
        tot[1] += f
    print(f"{case}: checked {tot[0]} rows, near-tie rows {tot[1]}")
    assert tot[0] >= 3


@pytest.mark.parametrize("case", ["negative", "mixed_signs"])
def test_single_pass_window_signs(case):
    """A window of negative keys (codes from the full orderable key), and a
    positive window over rows that are mostly negative (negative logits must
    code below the window)."""
    tot = [0, 0]
    for seed in range(3):
        w = wl.random_case(610 + seed, B=3, K_max=3, V=20011, dtype="bf16", D=0.5, top_p=0.9,
                           sigma=3.0, T_range=(0.5, 0.9))
        if case == "negative":   # every logit negative
            w.target[:] = wl.f32_to_bf16_bits(w.target_f32() - 20.0)
            w.draft[:] = wl.f32_to_bf16_bits(w.draft_f32() - 20.0)
        else:   # negative logits moved further down; the window stays positive
            t, d = w.target_f32(), w.draft_f32()
            w.target[:] = wl.f32_to_bf16_bits(np.where(t < 0, t - 10.0, t))
            w.draft[:] = wl.f32_to_bf16_bits(np.where(d < 0, d - 10.0, d))
        assert _fast_fallbacks(w) == 0
        c, f = compare_sample(gpu_sample(w), oracle_sample(w), w)
        tot[0] += c
        tot[1] += f
    print(f"{case}: checked {tot[0]} rows, near-tie rows {tot[1]}")
    assert tot[0] >= 3


def test_single_pass_draw_order():
    """Corrections drawn on the single-pass path over large nuclei: a lane
    then holds several weighted candidates in one 8-logit vector, and the
    inverse CDF must walk them in ascending token id."""
    tot = [0, 0]
    rejected = 0
    for seed in range(4):
        w = wl.random_case(700 + seed, B=64, K_max=2, V=20011, dtype="bf16", D=0.0, top_p=0.9,
                           sigma=3.0, corr=0.3, T_range=(0.9, 1.0))
        assert _fast_fallbacks(w) == 0
        g = gpu_sample(w)
        rejected += int((g["accepted"] < w.k_per_row).sum())
        c, f = compare_sample(g, oracle_sample(w), w)
        tot[0] += c
        tot[1] += f
    print(f"draw order: checked {tot[0]} rows, near-tie rows {tot[1]}, rejected rows {rejected}")
    assert tot[0] >= 128 and rejected >= 64


@pytest.mark.parametrize("case", ["penalty_ragged", "raise_tail", "whole_vectors"])
def test_single_pass_unit_loop(case):
    """More units than the device has compute units: the single-pass
    workgroups run in several waves per CU, with units past K_r (skipped),
    accepted and rejected positions, bonus rows and penalties mixed among
    them, at a modest V that the oracle covers row by row."""
    kw = {"penalty_ragged": dict(seed=810, V=12007, rep_penalty=1.2, n_prior=24, D=0.0),
          "raise_tail": dict(seed=811, V=12007, rep_penalty=0.9, n_prior=8, D=0.5),
          "whole_vectors": dict(seed=812, V=12008, rep_penalty=1.0, n_prior=0, D=0.0)}[case]
    seed = kw.pop("seed")
    w = wl.random_case(seed, B=160, K_max=4, dtype="bf16", top_p=0.9, sigma=3.0, corr=0.8,
                       T_range=(0.7, 1.2), ragged=True, **kw)
    assert w.B * (w.K_max + 1) > 512   # at least two units per CU on 256 CUs
    g = gpu_sample(w)
    c, f = compare_sample(g, oracle_sample(w), w)
    print(f"unit loop {case}: checked {c} rows, near-tie rows {f}")
    assert c >= 120


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_per_request_top_p_and_budget(dtype):
    """Per-request top-p and TV budget arrays (device [B]): every request
    runs with its own values, on the single-pass path (bf16) and the general
    path (fp32); top-p = 1 rows go to the exact routines; out-of-range
    values invalidate just their request."""
    w = wl.random_case(960, B=48, K_max=4, V=20011 if dtype == "bf16" else 3001, dtype=dtype,
                       D=0.0, top_p=0.9, sigma=3.0, corr=0.8, T_range=(0.7, 1.2), ragged=True,
                       rep_penalty=1.1, n_prior=16)
    rng = np.random.default_rng(5)
    w.top_p = rng.choice([0.5, 0.8, 0.9, 0.95, 1.0], size=w.B).astype(np.float32)
    w.tv_budget = rng.choice([0.0, 0.2, 0.5, 1.0, 2.0], size=w.B).astype(np.float32)
    w.top_p[3], w.top_p[7] = 0.0, 1.5
    w.tv_budget[11], w.tv_budget[13] = -0.1, np.nan
    g = gpu_sample(w)
    c, f = compare_sample(g, oracle_sample(w), w)
    print(f"per-request parameters ({dtype}): checked {c} rows, near-tie rows {f}")
    assert c >= 30
    for r in (3, 7, 11, 13):
        assert g["status"][r] & (1 << 7) and g["accepted"][r] == -1


def test_single_pass_fallback_routes():
    """bf16 + top-p cases that the single-pass kernel hands to its exact
    fallback: a flat distribution (nucleus larger than the per-lane slots), a
    draft far above the target (draft window overflow), and heavy penalty
    sets (penalized tokens near the cut)."""
    tot = [0, 0]
    flat = wl.random_case(41, B=3, K_max=2, V=60000, dtype="bf16", sigma=0.05, top_p=0.9, D=0.4)
    shifted = wl.random_case(42, B=3, K_max=2, V=30000, dtype="bf16", sigma=2.0, top_p=0.9, D=0.4)
    d = shifted.draft_f32() + 40.0
    shifted.draft[:] = wl.f32_to_bf16_bits(d)
    heavy = wl.random_case(43, B=4, K_max=3, V=20000, dtype="bf16", sigma=3.0, top_p=0.95,
                           n_prior=3000, rep_penalty=1.5, D=0.3)
    for w in (flat, shifted, heavy):
        c, f = compare_sample(gpu_sample(w), oracle_sample(w), w)
        tot[0] += c
        tot[1] += f
    print(f"fallback routes: checked {tot[0]}, near-tie {tot[1]}")
    assert tot[0] >= 4


@pytest.mark.parametrize("rep", [1.1, 0.8])
def test_single_pass_wide_target_cut(rep):
    """Temperatures in [1, 1.5] over V = 152064 (the batched workload's rows
    otherwise): the target's top-p crossing often lies below the single
    pass's 254-key window.  Such a unit takes the exact route, whose cuts
    then come from the rows' key histograms (exact for 4096 keys below each
    window's top) instead of the rows' own passes; the outputs and
    per-position statistics must match the oracle's.  A penalty below 1
    raises the penalized keys (some above the window)."""
    sdv = _sdv()
    w = wl.config4(seed=9 if rep > 1 else 10, B=24, K=8, T_range=(1.0, 1.5), odd_share=0.3,
                   rep_penalty=rep)
    d = to_device(w)
    args = sdv.make_args(d["target"], d["draft"], d["draft_ids"], d["k_per_row"],
                         d["temperature"], w.top_p, w.rep_penalty, d["prior_ids"],
                         d["prior_offsets"], w.tv_budget, w.seed, w.offset, w.flags)
    assert sdv.phase_kernel(args, 0) == "k_pair_fast"
    import torch
    ws = sdv.alloc_workspace(args, "cuda")
    acc = torch.empty(w.B, dtype=torch.int32, device="cuda")
    tok = torch.empty((w.B, w.K_max + 1), dtype=torch.int32, device="cuda")
    sdv.run_phase(args, ws, 0, acc, tok)
    n, why = sdv.fallback_units(args, ws, why=True)
    wide = int(((why & 32) != 0).sum())
    pcut = int(((why & 2) != 0).sum())
    assert (((why & 32) == 0) | ((why & 2) != 0)).all()
    assert (((why & 64) == 0) | ((why & 8) != 0)).all()
    g = gpu_sample(w, dev=d)
    c, f = compare_sample(g, oracle_sample(w), w)
    print(f"wide target cut: {n} of {len(why)} units flagged, {pcut} target cuts below the "
          f"window, {wide} of them settled from the histogram; checked {c} rows, near-tie {f}")
    assert wide >= 10 and c >= 0.9 * w.B


def test_single_pass_crossing_above_window():
    """A few logits far above the sampled rounds' maximum (ids past the
    rounds that set the window's anchor) carry most of each row's mass: the
    top-p crossing then lies among the exact entries above the window (bin
    0), which the single pass settles itself, for target and draft rows."""
    w = wl.random_case(1300, B=8, K_max=3, V=wl.V_QWEN25, dtype="bf16", sigma=3.0, corr=0.9,
                       T_range=(0.5, 1.0), top_p=0.9, rep_penalty=1.1, n_prior=24, D=0.5,
                       odd_share=0.3)
    rng = np.random.default_rng(77)
    t, d = w.target_f32(), w.draft_f32()
    for r in range(w.B):
        for j in range(w.K_max + 1):
            ids = rng.choice(np.arange(40000, w.V), size=6, replace=False)
            top = float(t[r, j].max()) + 8.0
            t[r, j, ids] = top + 0.5 * np.arange(6)
            if j < w.K_max:
                d[r, j, ids] = top + 0.5 * rng.permutation(6)
    w.target[:] = wl.f32_to_bf16_bits(t)
    w.draft[:] = wl.f32_to_bf16_bits(d)
    assert _fast_fallbacks(w) == 0
    c, f = compare_sample(gpu_sample(w), oracle_sample(w), w)
    print(f"crossing above the window: checked {c} rows, near-tie {f}")
    assert c >= 6


def test_general_path_split_draw_matches_one_workgroup():
    """Small batches split the general path's draw over workgroups by chunk
    ranges (and its TV pass by vector ranges); the draw takes the same chunk
    totals, scan and walk as the one-workgroup draw of a large batch, so
    each request's emitted tokens must be identical whether it runs in a
    batch of 512 (one workgroup per request) or of 8 (split)."""
    import torch
    sdv = _sdv()
    B, K, V, dev = 512, 2, 40000, "cuda"
    g = torch.Generator(device=dev).manual_seed(123)
    tgt = torch.randn((B, K + 1, V), generator=g, device=dev) * 3.0
    drf = 0.8 * tgt[:, :K] + 1.8 * torch.randn((B, K, V), generator=g, device=dev)
    u = torch.rand((B, K, V), generator=g, device=dev).clamp_(1e-20, 1.0)
    ids = torch.argmax(drf / 0.8 - torch.log(-torch.log(u)), dim=-1).to(torch.int32)
    ids[::5, 0] = torch.randint(0, V, (ids[::5, 0].numel(),), generator=g, device=dev, dtype=torch.int32)
    prior = torch.randint(0, V, (B * 16,), generator=g, device=dev, dtype=torch.int32)
    offs = torch.arange(0, B * 16 + 1, 16, dtype=torch.int32, device=dev)
    temp = torch.full((B,), 0.8, device=dev)
    for top_p in (0.9, 1.0):
        full = sdv.verify_sample(tgt, drf, ids, None, temp, top_p, 1.1, prior, offs, 0.0, 77, 0)
        args = sdv.make_args(tgt[:8], drf[:8], ids[:8], None, temp[:8], top_p, 1.1, prior[:8 * 16 + 0],
                             offs[:9], 0.0, 77, 0)
        assert "k_draw_pick" in sdv.phase_kernel(args, 2)
        part = sdv.verify_sample(tgt[:8], drf[:8], ids[:8], None, temp[:8], top_p, 1.1, prior[:8 * 16],
                                 offs[:9], 0.0, 77, 0)
        torch.cuda.synchronize()
        for x, y, name in zip(full[:3], part[:3], ("accepted", "tokens", "status")):
            np.testing.assert_array_equal(x[:8].cpu().numpy(), y.cpu().numpy(), err_msg=f"top_p={top_p} {name}")
        rejected = int((part[0].cpu().numpy() < K).sum())
        print(f"split draw, top_p={top_p}: 8 requests identical ({rejected} corrections, "
              f"{8 - rejected} bonus draws)")


def test_general_path_zero_residual():
    """A draft row equal to its target row and a proposal outside both
    nuclei: the proposal is rejected and the residual max(p - q, 0) has no
    mass, so the correction is drawn from p (status bit RESID_ZERO), on the
    general path split over workgroups."""
    w = wl.random_case(1400, B=3, K_max=2, V=20011, dtype="f32", sigma=3.0, corr=0.9,
                       T_range=(0.7, 0.9), top_p=0.9, D=0.0, odd_share=0.0)
    w.draft[:] = w.target[:, :w.K_max]
    from oracle import verify as ov
    tf = w.target_f32()
    for r in range(w.B):
        p = ov.process_dist(tf[r, 0], [], w.rep_penalty, float(w.temperature[r]), w.top_p).p
        w.draft_ids[r, 0] = int(np.flatnonzero(p == 0)[r])
    g, o = gpu_sample(w), oracle_sample(w)
    c, f = compare_sample(g, o, w)
    assert c == w.B and (o.status & (1 << 6)).all() and (g["status"] & (1 << 6)).all()
    print(f"zero residual: {c} requests checked, RESID_ZERO on all")


def test_single_pass_cut_beyond_histogram():
    """Temperatures in [2, 3]: the nucleus reaches deep into the negative
    logits, below the 4096 exact keys under each window's top, so the cuts
    from the key histograms do not settle and the exact route runs the
    rows' own radix-select passes; outputs must still match the oracle.
    (Such flat rows put many tokens within 1e-6 of the top-p threshold, so
    near-tie rows are common; the checked rows are compared bit for bit.)"""
    import torch
    sdv = _sdv()
    w = wl.config4(seed=12, B=24, K=4, T_range=(2.0, 3.0), odd_share=0.3)
    d = to_device(w)
    args = sdv.make_args(d["target"], d["draft"], d["draft_ids"], d["k_per_row"],
                         d["temperature"], w.top_p, w.rep_penalty, d["prior_ids"],
                         d["prior_offsets"], w.tv_budget, w.seed, w.offset, w.flags)
    assert sdv.phase_kernel(args, 0) == "k_pair_fast"
    ws = sdv.alloc_workspace(args, "cuda")
    acc = torch.empty(w.B, dtype=torch.int32, device="cuda")
    tok = torch.empty((w.B, w.K_max + 1), dtype=torch.int32, device="cuda")
    sdv.run_phase(args, ws, 0, acc, tok)
    n, why = sdv.fallback_units(args, ws, why=True)
    deep = int((((why & 2) != 0) & ((why & 32) == 0)).sum())
    g = gpu_sample(w, dev=d)
    c, f = compare_sample(g, oracle_sample(w), w)
    print(f"cuts beyond the histogram: {n} of {len(why)} units flagged, {deep} target cuts left to "
          f"the radix passes; checked {c} rows, near-tie {f}")
    assert deep >= 5 and c >= 8
