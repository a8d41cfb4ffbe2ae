"""Single-pass kernel branches at full size, its sampling law, and status rules.

The single-pass kernel (bf16 logits, top-p < 1) decides a proposal x through
different code for q(x) = 0 (a proposal outside the draft's nucleus), p(x) = 0
(outside the target's) and a penalized x; these tests choose the proposals so
that every branch is decided at V = 152064 and compared with the oracle, and
check the step's law (emitted token ~ pi_0, accepted length ~ prod a_j) by a
chi-square through the same kernel.  The status tests cover requests with
several defects and a workspace reused across calls.
"""
import numpy as np
import pytest

import workloads as wl
from parity import (compare_greedy, compare_sample, gpu_greedy, gpu_sample,
                    oracle_greedy, oracle_sample, to_device)

pytestmark = pytest.mark.gpu

BRANCHES = ("draft", "p_only", "q_only", "neither", "penalized")


def _sdv():
    import speculative_sampling_verify_temp_amd as sdv
    return sdv


def _plant_branches(w, rng):
    """Rewrite the proposals of w so that position j of request r falls in
    branch (r + j) mod 5: the draft's own sample; inside the target's nucleus
    only (q(x) = 0 < p(x)); inside the draft's only (p(x) = 0 < q(x)); inside
    neither; a prior id (penalized).  Nuclei come from the oracle's processed
    rows under each position's own penalty set (prior ids + draft prefix)."""
    from oracle import verify as ov
    tf, df = w.target_f32(), w.draft_f32()
    kinds = np.zeros(w.draft_ids.shape, dtype=np.int32)
    for r in range(w.B):
        prior = [int(t) for t in w.prior_ids[w.prior_offsets[r]:w.prior_offsets[r + 1]]]
        T = float(w.temperature[r])
        for j in range(w.K_max):
            b = (r + j) % len(BRANCHES)
            kinds[r, j] = b
            if BRANCHES[b] == "draft":
                continue
            if BRANCHES[b] == "penalized":
                w.draft_ids[r, j] = prior[int(rng.integers(0, len(prior)))]
                continue
            pen = prior + [int(t) for t in w.draft_ids[r, :j]]
            p = ov.process_dist(tf[r, j], pen, w.rep_penalty, T, w.top_p).p
            q = ov.process_dist(df[r, j], pen, w.rep_penalty, T, w.top_p).p
            sel = {"p_only": (p > 0) & (q == 0), "q_only": (p == 0) & (q > 0),
                   "neither": (p == 0) & (q == 0)}[BRANCHES[b]]
            cand = np.flatnonzero(sel)
            if cand.size:
                w.draft_ids[r, j] = int(cand[rng.integers(0, cand.size)])
            else:
                kinds[r, j] = 0
    return kinds


@pytest.mark.parametrize("D", [0.0, 0.5])
def test_single_pass_branches_full_size(D):
    sdv = _sdv()
    w = wl.random_case(1200 + int(D * 10), B=40, K_max=4, V=wl.V_QWEN25, dtype="bf16", sigma=3.0,
                       corr=0.9, T_range=(0.5, 1.0), top_p=0.9, rep_penalty=1.1, n_prior=24,
                       D=D, odd_share=0.0)
    kinds = _plant_branches(w, np.random.default_rng(12))
    d = to_device(w)
    args = sdv.make_args(d["target"], d["draft"], d["draft_ids"], d["k_per_row"],
                         d["temperature"], w.top_p, w.rep_penalty, d["prior_ids"],
                         d["prior_offsets"], w.tv_budget, w.seed, w.offset, w.flags)
    assert sdv.phase_kernel(args, 0) == "k_pair_fast"
    g = gpu_sample(w, dev=d)
    o = oracle_sample(w)
    c, f = compare_sample(g, o, w)
    decided = np.zeros(len(BRANCHES), dtype=int)
    deciding = np.zeros(len(BRANCHES), dtype=int)   # the position that ended the row
    for r in range(w.B):
        n = int(o.accepted[r])
        for j in range(min(n + 1, w.K_max)):
            decided[kinds[r, j]] += 1
        if n < w.K_max:
            deciding[kinds[r, n]] += 1
    print(f"branches D={D}: checked {c}, near-tie {f}; decided per branch "
          f"{dict(zip(BRANCHES, decided.tolist()))}; rejections per branch "
          f"{dict(zip(BRANCHES, deciding.tolist()))}")
    assert c >= 0.9 * w.B
    # every branch is decided, and each off-nucleus kind ends some rows
    assert (decided >= 4).all()
    assert deciding[BRANCHES.index("neither")] >= 2 and deciding[BRANCHES.index("q_only")] >= 2


def test_single_pass_law_bf16_top_p():
    """10^5 trials through the single-pass kernel (bf16, top-p 0.8, V = 8,
    K = 2): the first emitted token against pi_0 and the accepted length
    against prod a_j, where a_j = 1 - (1 - theta_j) d_j, from the oracle's
    processed rows ("What I Gave Up...", section "A knob for accepting more
    draft tokens": the accepted mass plus the residual make up pi)."""
    import torch
    from scipy import stats as ss
    from oracle import verify as ov
    sdv = _sdv()
    zt = np.array([[2.0, 1.5, 1.0, 0.5, 0.0, -0.5, -1.0, -3.0],
                   [0.25, 2.0, 1.75, -1.0, 0.5, 1.0, -2.0, 0.0],
                   [1.0, 1.0, 0.5, 2.5, -1.0, 0.0, 0.75, 1.5]], np.float32)
    zd = np.array([[1.5, 2.0, 0.5, 1.0, -0.5, 0.0, -1.0, 1.25],
                   [0.5, 1.5, 2.25, 0.0, 0.75, -0.25, -1.5, 1.0]], np.float32)
    T, top_p, N = 0.8, 0.8, 100_000
    tb, db = wl.f32_to_bf16_bits(zt), wl.f32_to_bf16_bits(zd)
    tf, df = wl.bf16_bits_to_f32(tb), wl.bf16_bits_to_f32(db)
    assert np.array_equal(tf, zt) and np.array_equal(df, zd)   # exact in bf16
    P = [ov.process_dist(tf[j], [], 1.0, T, top_p).p for j in range(3)]
    Q = [ov.process_dist(df[j], [], 1.0, T, top_p).p for j in range(2)]
    assert all((p == 0).any() for p in P[:2]) and all((q == 0).any() for q in Q)
    dev = "cuda"

    def rows(x, n):
        t = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(x.view(np.int16), (N,) + x.shape)))
        return t.to(dev).view(torch.bfloat16)

    tt, dd = rows(tb, 3), rows(db, 2)
    for D in (0.0, 0.3):
        pis, al = [], []
        for j in range(2):
            d = ov.tv_distance(P[j], Q[j])
            th = ov.mentored_theta(d, D)
            pis.append((1 - th) * P[j] + th * Q[j])
            al.append(1 - (1 - th) * d)
        rng = np.random.default_rng(7 + int(D * 10))
        ids = np.stack([rng.choice(8, N, p=Q[0]), rng.choice(8, N, p=Q[1])], 1).astype(np.int32)
        args = sdv.make_args(tt, dd, torch.from_numpy(ids).to(dev), None,
                             torch.full((N,), T, device=dev), top_p, 1.0, None, None, D, 23, 0)
        assert sdv.phase_kernel(args, 0) == "k_pair_fast"
        acc, tok, st, _ = sdv.verify_sample(tt, dd, torch.from_numpy(ids).to(dev), None,
                                            torch.full((N,), T, device=dev), top_p, 1.0, None,
                                            None, D, 23, 0)
        torch.cuda.synchronize()
        assert int((st.cpu().numpy() & 0x8F).sum()) == 0
        first = tok[:, 0].cpu().numpy()
        a = acc.cpu().numpy()
        keep = pis[0] > 0
        h = np.bincount(first, minlength=8)
        assert h[~keep].sum() == 0
        p1 = ss.chisquare(h[keep], N * pis[0][keep] / pis[0][keep].sum()).pvalue
        exp_n = N * np.array([1 - al[0], al[0] * (1 - al[1]), al[0] * al[1]])
        p2 = ss.chisquare(np.bincount(a, minlength=3), exp_n).pvalue
        print(f"law D={D}: first-token p-value {p1:.3g}, accepted-length p-value {p2:.3g}")
        assert p1 > 1e-4 and p2 > 1e-4


def test_exact_route_for_every_unit():
    """Every unit of a batch of 4400 units leaves the single pass for its
    exact route (each workgroup settles its own flagged units at once, with
    the general-path routines).  Rows whose maximum is small and whose mass
    sits largely on keys within 2^-20 of zero (here exact zeros) leave it by
    construction; the results must equal the general path's on the same
    values (fp32 input), which runs the same exact routines."""
    import torch
    sdv = _sdv()
    rng = np.random.default_rng(31)
    B, K, V = 2200, 1, 64
    base = np.zeros((K + 1, V), np.float32)
    base[:, : V // 2] = rng.integers(-8, 9, size=(K + 1, V // 2)) / 16.0   # exact in bf16
    dbase = np.zeros((K, V), np.float32)
    dbase[:, : V // 2] = rng.integers(-8, 9, size=(K, V // 2)) / 16.0
    tb, db = wl.f32_to_bf16_bits(base), wl.f32_to_bf16_bits(dbase)
    assert np.array_equal(wl.bf16_bits_to_f32(tb), base)
    dev = "cuda"
    tt = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(tb.view(np.int16), (B, K + 1, V)))).to(dev)
    tt = tt.view(torch.bfloat16)
    dd = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(db.view(np.int16), (B, K, V)))).to(dev)
    dd = dd.view(torch.bfloat16)
    tf = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(base, (B, K + 1, V)))).to(dev)
    df = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(dbase, (B, K, V)))).to(dev)
    ids = torch.from_numpy(rng.integers(0, V, size=(B, K)).astype(np.int32)).to(dev)
    temp = torch.from_numpy(rng.uniform(0.7, 1.2, size=B).astype(np.float32)).to(dev)
    for D in (0.0, 0.4):
        args = sdv.make_args(tt, dd, ids, None, temp, 0.9, 1.0, None, None, D, 41, 0)
        assert sdv.phase_kernel(args, 0) == "k_pair_fast"
        ws = sdv.alloc_workspace(args, dev)
        acc = torch.empty(B, dtype=torch.int32, device=dev)
        tok = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
        sdv.run_phase(args, ws, 0, acc, tok)
        assert sdv.fallback_units(args, ws) == B * (K + 1)
        g = sdv.verify_sample(tt, dd, ids, None, temp, 0.9, 1.0, None, None, D, 41, 0, stats=True)
        r = sdv.verify_sample(tf, df, ids, None, temp, 0.9, 1.0, None, None, D, 41, 0, stats=True)
        torch.cuda.synchronize()
        for x, y, name in zip(g, r, ("accepted", "tokens", "status", "stats")):
            np.testing.assert_array_equal(x.cpu().numpy(), y.cpu().numpy(), err_msg=f"D={D} {name}")
        assert (g[1][:, 0].cpu().numpy() >= 0).all()


@pytest.mark.parametrize("path", ["single_pass", "general"])
def test_status_precedence_and_workspace_reuse(path):
    """One invalidating defect per request, the first in the order K, draft
    ids, temperature (oracle/verify.py's row checks); logits of an invalid
    request are never examined; a workspace reused across calls carries no
    state into a request that the kernels skip."""
    import torch
    sdv = _sdv()
    dtype = "bf16" if path == "single_pass" else "f32"
    w = wl.random_case(1300, B=8, K_max=3, V=6007, dtype=dtype, sigma=3.0, top_p=0.9, D=0.4,
                       n_prior=4, rep_penalty=1.2, T_range=(0.6, 1.0))
    nan = 0x7FC0 if dtype == "bf16" else np.float32("nan")
    w.draft_ids[0, 1] = 6007; w.target[0, 2, 11] = nan           # bad id + NaN -> bad id
    w.k_per_row[1] = 9; w.temperature[1] = -1.0                  # bad K + bad T -> bad K
    w.draft_ids[2, 0] = -1; w.temperature[2] = 0.0               # bad id + bad T -> bad id
    w.temperature[3] = np.inf; w.draft[3, 0, 5] = nan            # bad T + NaN -> bad T
    w.target[4, 1, 100] = nan                                    # NaN alone
    w.prior_ids[5 * 4] = 99999; w.draft_ids[5, 2] = 7000         # bad prior + bad id
    d = to_device(w)
    args = sdv.make_args(d["target"], d["draft"], d["draft_ids"], d["k_per_row"],
                         d["temperature"], w.top_p, w.rep_penalty, d["prior_ids"],
                         d["prior_offsets"], w.tv_budget, w.seed, w.offset, w.flags)
    assert sdv.phase_kernel(args, 0) == ("k_pair_fast" if path == "single_pass" else "k_row_prepare")
    ws = torch.full((sdv.workspace_bytes(args),), 0x5A, dtype=torch.uint8, device="cuda")
    g = gpu_sample(w, dev=d)
    o = oracle_sample(w)
    compare_sample(g, o, w)
    assert list(g["status"][:6]) == [4, 1, 4, 2, 8, 4 | 16]
    # Call 1 leaves a NaN request's records in the workspace; call 2 gives the
    # same request a bad per-request top-p, so the kernels skip it.
    w1 = wl.random_case(1301, B=6, K_max=3, V=6007, dtype=dtype, sigma=3.0, top_p=0.9, D=0.4,
                        T_range=(0.6, 1.0))
    w1.target[2, 1, 40] = nan
    d1 = to_device(w1)
    import ctypes  # noqa: F401  (the workspace is passed by pointer through the binding)
    acc, tok, st, _ = sdv.verify_sample(d1["target"], d1["draft"], d1["draft_ids"], d1["k_per_row"],
                                        d1["temperature"], 0.9, 1.0, None, None, 0.4, w1.seed, 0,
                                        workspace=ws)
    torch.cuda.synchronize()
    assert st.cpu().numpy()[2] == 8
    w2 = w1.with_(target=w1.target.copy())
    w2.target[2, 1, 40] = w2.target[2, 1, 41]
    w2.top_p = np.full(w2.B, 0.9, np.float32)
    w2.top_p[2] = 1.5
    d2 = to_device(w2)
    acc, tok, st, _ = sdv.verify_sample(d2["target"], d2["draft"], d2["draft_ids"], d2["k_per_row"],
                                        d2["temperature"], torch.from_numpy(w2.top_p).cuda(), 1.0,
                                        None, None, 0.4, w2.seed, 0, workspace=ws)
    torch.cuda.synchronize()
    o2 = oracle_sample(w2)
    st2 = st.cpu().numpy().astype(np.uint32)
    assert st2[2] == o2.status[2] == 0x80
    assert np.array_equal(st2, o2.status)
    assert np.array_equal(acc.cpu().numpy(), o2.accepted)


def test_greedy_status_precedence():
    """Greedy: a bad draft id hides a NaN in the same request; a NaN alone
    invalidates; a bad prior id is reported beside a bad id."""
    w = wl.random_case(1310, B=5, K_max=3, V=3000, dtype="bf16", n_prior=4, rep_penalty=1.2)
    w.draft_ids[0, 2] = 3000; w.target[0, 1, 7] = 0x7FC0
    w.target[1, 3, 9] = 0x7FC0
    w.k_per_row[2] = -2; w.target[2, 0, 0] = 0x7FC0
    w.prior_ids[3 * 4] = -1; w.draft_ids[3, 0] = -4
    g, o = gpu_greedy(w), oracle_greedy(w)
    compare_greedy(g, o, range(w.B))
    assert list(g["status"][:4]) == [4, 8, 1, 4 | 16]
