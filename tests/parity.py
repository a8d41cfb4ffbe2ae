"""GPU-vs-oracle comparison helpers (test infrastructure).

Decisions (accepted length, emitted tokens, status bits) must be bit-exact
except in rows where the oracle reports a near-tie that can change the
output: at a position up to the accepted length, a uniform within EPS of its
acceptance threshold or a cumulative top-p mass within EPS of top_p, or a
draw uniform within EPS (in mass) of a CDF boundary.  Such rows are counted,
not compared.  Probabilities (d, theta, p(x), q(x), pi(x), S) agree within
TOL absolute wherever that position's top-p margins are clear of EPS;
uniforms are exact.
"""
import numpy as np

from workloads import bf16_bits_to_f32

EPS = 1e-6
TOL = 1e-5


def to_device(w, device="cuda"):
    """Workload arrays -> device tensors (each row padded to a multiple of 16
    bytes when its length is not one, so every row is 16-byte aligned; draft
    rows of a shorter draft vocabulary get their own, shorter stride)."""
    import torch
    es_mult = 8 if w.dtype == "bf16" else 4

    def rows(x):
        if x is None or x.size == 0:
            return None
        B, R, V = x.shape
        ld = -(-V // es_mult) * es_mult
        if w.dtype == "bf16":
            buf = np.zeros((B, R, ld), dtype=np.uint16)
            buf[..., :V] = x
            t = torch.from_numpy(buf.view(np.int16)).to(device).view(torch.bfloat16)
        else:
            buf = np.zeros((B, R, ld), dtype=np.float32)
            buf[..., :V] = x
            t = torch.from_numpy(buf).to(device)
        return t[..., :V]

    def i32(x):
        return None if x is None else torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(device)

    return dict(
        target=rows(w.target), draft=rows(w.draft),
        draft_ids=i32(w.draft_ids), k_per_row=i32(w.k_per_row),
        temperature=torch.from_numpy(np.ascontiguousarray(w.temperature, np.float32)).to(device),
        prior_ids=i32(w.prior_ids), prior_offsets=i32(w.prior_offsets))


def gpu_sample(w, stats=True, dev=None):
    import torch
    import speculative_sampling_verify_temp_amd as sdv
    d = dev or to_device(w)

    def per_request(x):   # a [B] array of per-request values goes to the device
        if np.ndim(x) == 0:
            return x
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(d["target"].device)

    acc, tok, st, sts = sdv.verify_sample(
        d["target"], d["draft"], d["draft_ids"], d["k_per_row"], d["temperature"],
        per_request(w.top_p), w.rep_penalty, d["prior_ids"], d["prior_offsets"],
        per_request(w.tv_budget), w.seed, w.offset, w.flags, stats=stats)
    torch.cuda.synchronize()
    return dict(accepted=acc.cpu().numpy(), tokens=tok.cpu().numpy(),
                status=st.cpu().numpy().astype(np.uint32),
                stats=None if sts is None else sts.cpu().numpy().astype(np.float64))


def gpu_greedy(w, dev=None):
    import torch
    import speculative_sampling_verify_temp_amd as sdv
    d = dev or to_device(w)
    acc, tok, st, am = sdv.verify_greedy(d["target"], d["draft_ids"], d["k_per_row"],
                                         w.rep_penalty, d["prior_ids"], d["prior_offsets"],
                                         w.flags, argmax=True)
    torch.cuda.synchronize()
    return dict(accepted=acc.cpu().numpy(), tokens=tok.cpu().numpy(),
                status=st.cpu().numpy().astype(np.uint32), argmax=am.cpu().numpy())


def oracle_sample(w, rows=None):
    from oracle import verify_sample_ref
    return verify_sample_ref(w.target_f32(), w.draft_f32(), w.draft_ids, w.k_per_row,
                             w.temperature, w.top_p, w.rep_penalty, w.prior_ids,
                             w.prior_offsets, w.tv_budget, w.seed, w.offset, w.flags,
                             rows=rows)


def oracle_greedy(w, rows=None):
    from oracle import verify_greedy_ref
    return verify_greedy_ref(w.target_f32(), w.draft_ids, w.k_per_row, w.rep_penalty,
                             w.prior_ids, w.prior_offsets, w.flags, rows=rows)


def tie_position(rr, K, eps=EPS):
    """First position j (0..K) whose own margins put a decision within eps
    of its threshold: the top-p cumulative mass of p_j or q_j against top_p,
    or u_j against pi_j(x_j) / q_j(x_j); K + 1 when there is none."""
    for j in range(K + 1):
        m = [rr.topp_margin_p[j]]
        if j < K:
            m += [rr.topp_margin_q[j], rr.accept_margin[j]]
        if min(m) < eps:
            return j
    return K + 1


def near_tie(rr, K, eps=EPS):
    """Can a near-tie change this row's output?  Only positions 0..n (n the
    oracle's accepted length) and the draw decide it: a tie at a later
    position cannot."""
    if rr is None or rr.stats is None:
        return False
    return tie_position(rr, K, eps) <= rr.accepted or rr.draw_margin < eps


def compare_sample(g, o, w, rows=None, eps=EPS, tol=TOL):
    """Assert parity; return (checked, flagged) row counts.

    A row whose output a near-tie can change (near_tie) is flagged and its
    decisions are not compared; every other row is compared bit for bit.
    Per-position statistics are compared at every position j < K_r whose
    own top-p margins are clear of eps (a tie at another position does not
    touch them), in flagged rows too; the draw mass S only where the
    decisions were compared."""
    rows = range(w.B) if rows is None else rows
    checked = flagged = 0
    for r in rows:
        K = int(w.k_per_row[r])
        rr = o.rows[r]
        ctx = f"row {r} (K={K})"
        tied = near_tie(rr, K, eps)
        if tied:
            flagged += 1
        else:
            checked += 1
            assert g["status"][r] == o.status[r], (ctx, g["status"][r], o.status[r])
            assert g["accepted"][r] == o.accepted[r], (ctx, g["accepted"][r], o.accepted[r])
            assert np.array_equal(g["tokens"][r], o.tokens[r]), (ctx, g["tokens"][r], o.tokens[r])
        if g["stats"] is None or rr is None or rr.stats is None or (o.status[r] & 0x8F):
            continue
        gs, os_ = g["stats"][r], o.stats[r]
        for j in range(K):
            if min(rr.topp_margin_p[j], rr.topp_margin_q[j]) < eps:
                continue
            np.testing.assert_allclose(gs[j, :5], os_[j, :5], atol=tol, rtol=0,
                                       err_msg=f"{ctx} stats j={j}")
        np.testing.assert_array_equal(gs[:K + 1, 5:7], os_[:K + 1, 5:7], err_msg=f"{ctx} uniforms")
        if not tied:
            n = o.accepted[r]
            np.testing.assert_allclose(gs[n, 7], os_[n, 7], atol=tol, rtol=0, err_msg=f"{ctx} S")
    return checked, flagged


def compare_greedy(g, o, rows):
    for r in rows:
        assert g["status"][r] == o.status[r], (r, g["status"][r], o.status[r])
        assert g["accepted"][r] == o.accepted[r], (r, g["accepted"][r], o.accepted[r])
        assert np.array_equal(g["tokens"][r], o.tokens[r]), (r, g["tokens"][r], o.tokens[r])
        if not (o.status[r] & 0xF):
            assert np.array_equal(g["argmax"][r], o.argmax[r]), (r, g["argmax"][r], o.argmax[r])
