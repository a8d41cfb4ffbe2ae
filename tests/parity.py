"""GPU-vs-oracle comparison helpers (test infrastructure).

Decisions (accepted length, emitted tokens, status bits) must be bit-exact
except in rows where the oracle reports a near-tie: a uniform within EPS of
its acceptance threshold, a cumulative top-p mass within EPS of top_p, or a
draw uniform within EPS (in mass) of a CDF boundary.  Such rows are counted,
not compared.  Probabilities (d, theta, p(x), q(x), pi(x), S) agree within
TOL absolute; uniforms are exact.
"""
import numpy as np

from workloads import bf16_bits_to_f32

EPS = 1e-6
TOL = 1e-5


def to_device(w, device="cuda"):
    """Workload arrays -> device tensors (bf16 rows padded to a multiple of 8
    elements when V is not one, so every row is 16-byte aligned)."""
    import torch
    es_mult = 8 if w.dtype == "bf16" else 4
    ld = -(-w.V // es_mult) * es_mult

    def rows(x):
        if x is None or x.size == 0:
            return None
        B, R, V = x.shape
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


def near_tie(rr, K, eps=EPS):
    """Does any margin that can change this row's output fall below eps?"""
    if rr is None or rr.stats is None:
        return False
    n = rr.accepted
    m = [rr.draw_margin]
    m += list(rr.accept_margin[:min(n + 1, K)])
    m += list(rr.topp_margin_p[:K + 1]) + list(rr.topp_margin_q[:K])
    return bool(np.min(m) < eps) if m else False


def compare_sample(g, o, w, rows=None, eps=EPS, tol=TOL):
    """Assert parity; return (checked, flagged) row counts."""
    rows = range(w.B) if rows is None else rows
    checked = flagged = 0
    for r in rows:
        K = int(w.k_per_row[r])
        rr = o.rows[r]
        if near_tie(rr, K, eps):
            flagged += 1
            continue
        checked += 1
        ctx = f"row {r} (K={K})"
        assert g["status"][r] == o.status[r], (ctx, g["status"][r], o.status[r])
        assert g["accepted"][r] == o.accepted[r], (ctx, g["accepted"][r], o.accepted[r])
        assert np.array_equal(g["tokens"][r], o.tokens[r]), (ctx, g["tokens"][r], o.tokens[r])
        if g["stats"] is None or (o.status[r] & 0xF):
            continue
        gs, os_ = g["stats"][r], o.stats[r]
        for j in range(K):
            np.testing.assert_allclose(gs[j, :5], os_[j, :5], atol=tol, rtol=0,
                                       err_msg=f"{ctx} stats j={j}")
        np.testing.assert_array_equal(gs[:K + 1, 5:7], os_[:K + 1, 5:7], err_msg=f"{ctx} uniforms")
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
