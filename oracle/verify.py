"""Plain fp64 CPU oracle of the speculative-sampling verify step.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py): the product path never
imports this module.

Everything here is numpy on the CPU, one request row at a time, with no
blocking or fusion: a reader can set each function beside the passage it
follows.  The pages cited are

  [WGU]  "What I Gave Up to Make Speculative Decoding Faster", section
         "A knob for accepting more draft tokens" (the TV distance d, the
         weight theta = min(1, D/d), the mixture pi = (1-theta)p + theta q,
         the acceptance a(x) = min(1, pi(x)/q(x)), the correction from the
         normalized positive residual max(p-q, 0), p and q taken after
         temperature and repetition penalty), and section "Even full
         acceptance did not buy a speedup" (an engine that emits no bonus
         token after a fully accepted proposal).
  [ASL]  "Adaptive-SpecDecode-Lab" README, section on the implementation
         (longest-prefix acceptance; a target correction at the first
         mismatch; a bonus token after a full match; greedy mode).
  [SDN]  "Speculative Decoding" note, section "Warum eine Korrektur noetig
         ist" (p and q after temperature and top-p; accept x~q with
         min(1, p(x)/q(x)); after a rejection draw from a distribution
         proportional to max(0, p-q); a drawn proposal has q(x) > 0) and
         section "Eigenes Beispiel" (the worked example pinned in tests).

Readings where the pages are silent (each is listed in the design doc):
  * repetition penalty: a logit z of a penalized id becomes z/r if z > 0 and
    z*r otherwise, once per id (set semantics), computed in fp32 so that the
    order of processed logits is decided in one precision on both sides;
  * penalty set of target and draft position j: the row's prior ids plus the
    draft prefix x_0..x_{j-1} (flag PENALTY_PRIOR_ONLY drops the prefix);
  * order of steps: penalty, then division by the row temperature, softmax,
    then top-p and renormalization, for both p and q;
  * top-p: keep a token iff the mass of the strictly more probable tokens
    is < top_p (tokens tied at the boundary are all kept); probabilities
    are compared through the processed logits; top_p = 1 disables
    truncation;
  * theta = 1 when d <= D (covers d = 0), else D/d; d is clamped to <= 1;
  * acceptance is tested as u * q(x) < pi(x), equal to u < min(1, pi/q) for
    q(x) > 0, with no division;
  * inverse CDF over ascending token id, unnormalized cumulative sums, the
    first index whose cumulative sum exceeds v * S;
  * the bonus token is drawn from the processed target p_K unless the flag
    NO_BONUS is set ([WGU] "Even full acceptance..." describes that variant);
  * greedy ties go to the lowest index; greedy ignores temperature and top-p
    (neither can move an argmax) and honours the penalty.
"""

from dataclasses import dataclass, field

import numpy as np

from .philox import uniforms_for

# Per-row status bits (same meaning as the C header's SD_ST_* constants).
ST_BAD_K = 1 << 0          # K_r outside [0, K_max]                 (invalid)
ST_BAD_TEMP = 1 << 1       # temperature not finite or <= 0         (invalid)
ST_BAD_DRAFT_ID = 1 << 2   # a draft id x_j, j < K_r, outside [0,V) (invalid)
ST_NONFINITE = 1 << 3      # NaN/+Inf logit, or a row of only -Inf  (invalid)
ST_BAD_PRIOR = 1 << 4      # a prior id outside [0, V) was ignored  (info)
ST_Q_ZERO = 1 << 5         # q(x_j) = 0 at a position j < K_r       (info)
ST_RESID_ZERO = 1 << 6     # residual mass was 0; drew from p       (info)
ST_BAD_PARAM = 1 << 7      # per-request top-p outside (0, 1] or TV
                           # budget < 0 or NaN                      (invalid)
ST_INVALID_MASK = ST_BAD_K | ST_BAD_TEMP | ST_BAD_DRAFT_ID | ST_NONFINITE | ST_BAD_PARAM

FLAG_NO_BONUS = 1 << 0
FLAG_PENALTY_PRIOR_ONLY = 1 << 1

NSTAT = 8   # d, theta, p(x), q(x), pi(x), u, v, S


def penalty_keys(z, pen_ids, r):
    """Processed logits before temperature ("keys"), fp32.

    [WGU] "A knob...": p and q are taken after repetition penalty; the
    formula is not on the pages.  Reading: for every id in the set, z -> z/r
    when z > 0, else z -> z*r, each a single IEEE fp32 operation.  Parity
    unpinned by the pages; pinned by hand-computed cases of this rule.
    """
    z = np.asarray(z, dtype=np.float32)
    key = z.copy()
    r32 = np.float32(r)
    ids = np.unique(np.asarray(list(pen_ids), dtype=np.int64))
    if r32 != np.float32(1.0) and ids.size:
        zi = z[ids]
        with np.errstate(invalid="ignore", over="ignore"):
            key[ids] = np.where(zi > 0, zi / r32, zi * r32).astype(np.float32)
    return key


def softmax64(keys, temperature):
    """p = softmax(keys / T) in fp64 ([WGU] "A knob...": p, q after temperature).

    Returns None when the distribution is undefined (NaN or +Inf logit, or
    every logit -Inf).
    """
    k64 = np.asarray(keys, dtype=np.float64)
    if np.isnan(k64).any() or np.isposinf(k64).any():
        return None
    t = np.float64(np.float32(temperature))
    lg = k64 / t
    m = lg.max()
    if not np.isfinite(m):
        return None
    e = np.exp(lg - m)
    return e / e.sum()


def top_p_filter(keys, p, top_p):
    """Nucleus truncation and renormalization ([SDN] "Warum...": p, q after top-p).

    Reading (the pages give no boundary rule): a token is kept iff the total
    probability of the tokens that are strictly more probable than it is
    < top_p.  Probabilities are compared through the processed logits (p is
    strictly increasing in them), so tokens tied with the boundary token are
    all kept: the nucleus is the smallest set of the form {x : p(x) >= tau}
    whose mass reaches top_p, a function of the distribution alone.
    Returns (p_tilde, margin) where margin = min over distinct logit values of
    |mass strictly above - top_p| (inf when top_p >= 1: truncation off).
    Parity unpinned by the pages (the boundary rule is a reading); pinned by
    brute force against a direct O(V^2) enumeration in tests.
    """
    if top_p >= 1.0:
        return p, np.inf
    k64 = np.asarray(keys, dtype=np.float64)
    order = np.argsort(-k64, kind="stable")
    ks, ps = k64[order], p[order]
    csum = np.concatenate(([0.0], np.cumsum(ps)))
    # first sorted position of each element's group of equal keys
    new_group = np.concatenate(([True], ks[1:] != ks[:-1]))
    group_start = np.maximum.accumulate(np.where(new_group, np.arange(ks.size), 0))
    above = csum[group_start]
    tp = np.float64(np.float32(top_p))
    keep = np.zeros(p.size, dtype=bool)
    keep[order[above < tp]] = True
    pk = np.where(keep, p, 0.0)
    margin = float(np.min(np.abs(above[new_group] - tp)))
    return pk / pk.sum(), margin


@dataclass
class Dist:
    keys: np.ndarray        # fp32 processed logits (penalty applied)
    p: np.ndarray           # fp64 processed, truncated, renormalized probs
    topp_margin: float


def process_dist(z, pen_ids, r, temperature, top_p):
    """Penalty -> /T -> softmax -> top-p -> renormalize, for one row."""
    keys = penalty_keys(z, pen_ids, r)
    p = softmax64(keys, temperature)
    if p is None:
        return None
    pt, margin = top_p_filter(keys, p, top_p)
    return Dist(keys, pt, margin)


def draft_row_over_target(z, V):
    """A draft logit row over the target's vocabulary.

    [ASL] implementation section: the draft and target tokenizers are fully
    mapped, while the two models' logit rows need not have the same length
    (the pages' Qwen2.5 7B / 0.5B pair pads its vocabularies to 152064 and
    151936).  Reading: the draft's row covers token ids 0..V_d-1 and every id
    from V_d to V-1 is a token the draft cannot propose, logit -inf, q = 0.
    Returns the row padded to V entries (a copy only when V_d < V).
    """
    z = np.asarray(z, dtype=np.float32)
    if z.shape[-1] == V:
        return z
    if z.shape[-1] > V:
        raise ValueError("a draft row longer than the target's vocabulary")
    pad = np.full(z.shape[:-1] + (V - z.shape[-1],), -np.inf, dtype=np.float32)
    return np.concatenate([z, pad], axis=-1)


def tv_distance(p, q):
    """d = TV(p, q) = 1/2 sum_x |p(x) - q(x)|  ([WGU] "A knob...", eq. for d).

    Clamped to <= 1 (exact arithmetic never exceeds 1).
    """
    return min(0.5 * float(np.abs(p - q).sum()), 1.0)


def mentored_theta(d, D):
    """theta = min(1, D/d), theta = 1 when d = 0 ([WGU] "A knob...", eq. for theta).

    Written as: theta = 1 if d <= D else D/d, so d = 0 and D >= 1 give 1
    without a division.
    """
    return 1.0 if d <= D else D / d


def inverse_cdf(w, v):
    """Draw from w / sum(w) with the uniform v by the inverse CDF.

    C_i = sum_{k<=i} w_k over ascending token id; S = C_{V-1}; t = v*S;
    y = min{ i : C_i > t }.  Returns (y, S, margin) where margin is the
    distance from t to the nearest cumulative boundary around y, in
    probability-mass units; returns None when S = 0.
    """
    c = np.cumsum(np.asarray(w, dtype=np.float64))
    s = float(c[-1])
    if not s > 0.0:
        return None
    t = v * s
    y = int(np.searchsorted(c, t, side="right"))
    lo = c[y - 1] if y > 0 else 0.0
    margin = min(t - lo, c[y] - t)
    return y, s, float(margin)


@dataclass
class RowResult:
    status: int = 0
    accepted: int = -1
    tokens: list = field(default_factory=list)
    stats: np.ndarray = None            # [K_r+1][NSTAT]
    accept_margin: np.ndarray = None    # [K_r]  |u_j - pi_j/q_j|
    topp_margin_p: np.ndarray = None    # [K_r+1]
    topp_margin_q: np.ndarray = None    # [K_r]
    draw_margin: float = np.inf


def _penalty_set(prior, x, j, flags):
    if flags & FLAG_PENALTY_PRIOR_ONLY:
        return list(prior)
    return list(prior) + [int(t) for t in x[:j]]


def verify_sample_row(tgt, drf, x, K, prior, T, top_p, r_pen, D, u, v, V,
                      flags=0):
    """One request row of the sampling verify step.

    tgt: fp32 [K+1][V] target logits; drf: fp32 [K][V] draft logits;
    x: draft ids [K]; prior: valid prior ids; u, v: uniforms [K+1].

    Steps ([WGU] "A knob..."; [SDN] "Warum..."; [ASL] implementation):
      for each position j < K: p_j, q_j processed; d_j = TV(p_j, q_j);
      theta_j; pi_j(x_j) = (1-theta_j) p_j(x_j) + theta_j q_j(x_j);
      accept_j <=> u_j * q_j(x_j) < pi_j(x_j);
      n = first rejected position (else K);
      n < K: correction from max(p_n - q_n, 0) with v_n;
      n = K: bonus from p_K with v_K (unless NO_BONUS).
    """
    res = RowResult()
    drf = draft_row_over_target(drf, V)   # a shorter draft vocabulary: q = 0 beyond it
    res.stats = np.zeros((K + 1, NSTAT))
    res.accept_margin = np.full(K, np.inf)
    res.topp_margin_p = np.full(K + 1, np.inf)
    res.topp_margin_q = np.full(K, np.inf)

    P, Q = [], []
    for j in range(K + 1):
        pen = _penalty_set(prior, x, j, flags)
        dp = process_dist(tgt[j], pen, r_pen, T, top_p)
        if dp is None:
            res.status |= ST_NONFINITE
            return res
        P.append(dp)
        res.topp_margin_p[j] = dp.topp_margin
        if j < K:
            dq = process_dist(drf[j], pen, r_pen, T, top_p)
            if dq is None:
                res.status |= ST_NONFINITE
                return res
            Q.append(dq)
            res.topp_margin_q[j] = dq.topp_margin

    n = K
    for j in range(K):
        p, q = P[j].p, Q[j].p
        d = tv_distance(p, q)
        th = mentored_theta(d, D)
        px, qx = float(p[x[j]]), float(q[x[j]])
        pix = (1.0 - th) * px + th * qx
        res.stats[j, :7] = (d, th, px, qx, pix, u[j], v[j])
        if qx == 0.0:
            res.status |= ST_Q_ZERO
            # u * 0 < pi(x) holds iff pi(x) = (1 - theta) p(x) > 0: decided
            # by p(x) > 0 (nucleus membership, which has its own margin) and
            # by theta < 1, i.e. d > D.  D >= 1 always gives theta = 1 (d is
            # at most 1), and p(x) = 0 gives pi(x) = 0 whatever theta is.
            res.accept_margin[j] = abs(d - D) if (px > 0.0 and D < 1.0) else np.inf
        else:
            res.accept_margin[j] = abs(u[j] - pix / qx)
        if n == K and not (u[j] * qx < pix):
            n = j
    res.stats[K, 5:7] = (u[K], v[K])

    res.accepted = n
    res.tokens = [int(t) for t in x[:n]]
    if n < K:
        w = np.maximum(P[n].p - Q[n].p, 0.0)
    elif flags & FLAG_NO_BONUS:
        return res
    else:
        w = P[K].p
    drawn = inverse_cdf(w, v[n])
    if drawn is None:
        res.status |= ST_RESID_ZERO
        drawn = inverse_cdf(P[n].p, v[n])
    y, s, margin = drawn
    res.stats[n, 7] = s
    res.draw_margin = margin
    res.tokens.append(y)
    return res


@dataclass
class SampleResult:
    accepted: np.ndarray      # int32 [B]
    tokens: np.ndarray        # int32 [B][K_max+1], -1 padded
    status: np.ndarray        # uint32 [B]
    stats: np.ndarray         # float64 [B][K_max+1][NSTAT]
    rows: list                # RowResult per row (margins)


def _row_prior(prior_ids, prior_offsets, r, V):
    if prior_ids is None or prior_offsets is None:
        return [], 0
    seg = np.asarray(prior_ids[prior_offsets[r]:prior_offsets[r + 1]],
                     dtype=np.int64)
    ok = (seg >= 0) & (seg < V)
    return [int(t) for t in seg[ok]], (0 if ok.all() else ST_BAD_PRIOR)


def _row_checks(x, K, K_max, V):
    if not (0 <= K <= K_max):
        return ST_BAD_K
    xs = np.asarray(x[:K], dtype=np.int64)
    if ((xs < 0) | (xs >= V)).any():
        return ST_BAD_DRAFT_ID
    return 0


def verify_sample_ref(target, draft, draft_ids, k_per_row=None,
                      temperature=None, top_p=1.0, rep_penalty=1.0,
                      prior_ids=None, prior_offsets=None, tv_budget=0.0,
                      seed=0, offset=0, flags=0, rows=None):
    """Batched sampling verify, row by row.

    target: fp32 [B][K_max+1][V]; draft: fp32 [B][K_max][V_d] with V_d <= V
    (tokens V_d..V-1 have q = 0, see draft_row_over_target);
    draft_ids: int [B][K_max]; k_per_row: int [B] or None (= K_max);
    temperature: fp32 [B] or None (= 1); prior CSR or None.
    top_p, tv_budget: a scalar for every request, or an array [B] of
    per-request values (fp32); a per-request value out of range (top-p
    outside (0, 1], budget negative or NaN) makes that request invalid
    (ST_BAD_PARAM), as the library does.
    rows: optional subset of rows to evaluate (others stay at -1 / 0).
    """
    B, K1, V = target.shape
    K_max = K1 - 1
    accepted = np.full(B, -1, dtype=np.int32)
    tokens = np.full((B, K_max + 1), -1, dtype=np.int32)
    status = np.zeros(B, dtype=np.uint32)
    stats = np.zeros((B, K_max + 1, NSTAT))
    out_rows = [None] * B
    for r in (range(B) if rows is None else rows):
        K = K_max if k_per_row is None else int(k_per_row[r])
        x = np.asarray(draft_ids[r], dtype=np.int64)
        st = _row_checks(x, K, K_max, V)
        T = 1.0 if temperature is None else float(np.float32(temperature[r]))
        if st == 0 and not (np.isfinite(T) and T > 0.0):
            st = ST_BAD_TEMP
        tp_r = float(np.float32(top_p[r])) if np.ndim(top_p) else float(top_p)
        D_r = float(np.float32(tv_budget[r])) if np.ndim(tv_budget) else float(tv_budget)
        if np.ndim(top_p) or np.ndim(tv_budget):
            if not (tp_r > 0.0 and tp_r <= 1.0) or not (D_r >= 0.0):
                st |= ST_BAD_PARAM
        prior, st_prior = _row_prior(prior_ids, prior_offsets, r, V)
        if st:
            status[r] = st | st_prior
            out_rows[r] = RowResult(status=int(status[r]))
            continue
        u, v = uniforms_for(seed, offset, np.full(K + 1, r), np.arange(K + 1))
        rr = verify_sample_row(
            np.asarray(target[r, :K + 1], dtype=np.float32),
            np.asarray(draft[r, :K], dtype=np.float32), x[:K], K, prior, T,
            tp_r, rep_penalty, D_r, u, v, V, flags)
        rr.status |= st_prior
        status[r] = rr.status
        out_rows[r] = rr
        if rr.status & ST_INVALID_MASK:
            continue
        accepted[r] = rr.accepted
        tokens[r, :len(rr.tokens)] = rr.tokens
        stats[r, :K + 1] = rr.stats
    return SampleResult(accepted, tokens, status, stats, out_rows)


@dataclass
class GreedyResult:
    accepted: np.ndarray
    tokens: np.ndarray
    status: np.ndarray
    argmax: np.ndarray        # int32 [B][K_max+1], -1 beyond K_r


def verify_greedy_ref(target, draft_ids, k_per_row=None, rep_penalty=1.0,
                      prior_ids=None, prior_offsets=None, flags=0, rows=None):
    """Greedy verify ([ASL] implementation: longest prefix of drafts equal to
    the target argmax; the target's token at the first mismatch; a bonus
    after a full match).  g_j = argmax of the penalized target row j, lowest
    index on ties; n = first j < K_r with x_j != g_j, else K_r; y = g_n.
    """
    B, K1, V = target.shape
    K_max = K1 - 1
    accepted = np.full(B, -1, dtype=np.int32)
    tokens = np.full((B, K_max + 1), -1, dtype=np.int32)
    status = np.zeros(B, dtype=np.uint32)
    amax = np.full((B, K_max + 1), -1, dtype=np.int32)
    for r in (range(B) if rows is None else rows):
        K = K_max if k_per_row is None else int(k_per_row[r])
        x = np.asarray(draft_ids[r], dtype=np.int64)
        st = _row_checks(x, K, K_max, V)
        prior, st_prior = _row_prior(prior_ids, prior_offsets, r, V)
        if st:
            status[r] = st | st_prior
            continue
        g = []
        for j in range(K + 1):
            keys = penalty_keys(target[r, j], _penalty_set(prior, x, j, flags),
                                rep_penalty)
            if np.isnan(keys).any():
                st |= ST_NONFINITE
                break
            g.append(int(np.argmax(keys)))
        status[r] = st | st_prior
        if st:
            continue
        amax[r, :K + 1] = g
        n = K
        for j in range(K):
            if x[j] != g[j]:
                n = j
                break
        accepted[r] = n
        toks = [int(t) for t in x[:n]]
        if not (n == K and flags & FLAG_NO_BONUS):
            toks.append(g[n])
        tokens[r, :len(toks)] = toks
    return GreedyResult(accepted, tokens, status, amax)
