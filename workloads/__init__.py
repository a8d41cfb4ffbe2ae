"""Seeded synthetic inputs for the verify step.

This module is shared by the tests, the bench and the oracle's callers.  It
holds input synthesis only: normal logits, bf16 rounding of them, draft-token
proposals, prior-context ids, and the draft-side early-stop rule that sets a
ragged K.  None of the verify step's own arithmetic lives here (no penalty, no
top-p, no TV distance, no acceptance and no residual).

Workloads (stand-ins for the pages' creative-writing and code prompts run
through Qwen models, which are not available; logits are synthetic):

  worked_example  V=3, p=[.2,.5,.3], q=[.6,.3,.1] as log-probabilities
                  ("Speculative Decoding" note, section "Eigenes Beispiel").
  config1         1 row, K=4, V=1000, fp32, target ~N(0, 2^2), draft = target
                  + N(0,1), T=0.7, no penalty, no top-p.
  config2         1 row, K=8, V=152064, fp32, target ~N(0, 3^2), draft =
                  0.8*target + N(0, 1.5^2), T=0.7, penalty 1.1 over 64 prior
                  ids drawn uniformly (duplicates allowed).
  config3         greedy, V=151936, bf16, target ~N(0, 3^2), draft rows
                  correlated 0.9 with the target, draft ids = argmax of the
                  draft rows.
  config4         256 rows x K=8, V=152064, bf16, target ~N(0, 3^2), draft
                  correlated 0.9, T_r ~ U[0.5, 1.0], top-p 0.9, penalty 1.1
                  over 128 prior ids per row, TV budget 0.75.
  config5         512 rows, V=151936, bf16, per-row correlation U[0.3, 0.95],
                  T=0.7, budget 0, K_r from the draft-side early stop rule
                  (first position whose top-1 draft probability is < 0.6,
                  "Adaptive-SpecDecode-Lab" README, section "Confidence-guided
                  early stop"); variant "5b" draws K_r ~ U{1..8} instead.

"Correlation c" means draft = c*t + sqrt(1-c^2)*sigma*eps, same marginal
sigma as the target.  N(0, s) means standard deviation s.

Draft ids are proposals from the draft model's sampler: Gumbel-max over the
whole raw draft row divided by T (an exact sample of softmax(z/T)).  Nothing
restricts them to the nucleus: with top-p on, some land outside the draft's
(q(x) = 0) or the target's (p(x) = 0) nucleus.  Workloads built for parity
also replace a seeded share of the proposals (`odd_share`) by an id drawn
uniformly from [0, V) or from the request's prior ids (a penalized token), so
that those branches of the step are exercised on purpose.
"""

from dataclasses import dataclass, replace

import numpy as np

V_QWEN25 = 152064     # vocabulary of the pages' Qwen2.5 models
V_QWEN3 = 151936      # vocabulary of the pages' Qwen3 models


def f32_to_bf16_bits(a):
    """Round fp32 to bf16 (round to nearest even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rnd = ((u >> np.uint64(16)) & np.uint64(1)) + np.uint64(0x7FFF)
    return ((u + rnd) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(b):
    """Exact upcast of bf16 bit patterns to fp32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Workload:
    name: str
    dtype: str                  # "f32" or "bf16"
    target: np.ndarray          # [B][K_max+1][V] fp32, or uint16 bf16 bits
    draft: np.ndarray           # [B][K_max][V] same storage as target
    draft_ids: np.ndarray       # int32 [B][K_max]
    k_per_row: np.ndarray       # int32 [B]
    temperature: np.ndarray     # float32 [B]
    top_p: float = 1.0
    rep_penalty: float = 1.0
    prior_ids: np.ndarray = None      # int32 [nnz]
    prior_offsets: np.ndarray = None  # int32 [B+1]
    tv_budget: float = 0.0
    seed: int = 0
    offset: int = 0
    flags: int = 0

    @property
    def B(self):
        return self.target.shape[0]

    @property
    def K_max(self):
        return self.target.shape[1] - 1

    @property
    def V(self):
        return self.target.shape[2]

    def target_f32(self):
        return self.target if self.dtype == "f32" else bf16_bits_to_f32(self.target)

    def draft_f32(self):
        return self.draft if self.dtype == "f32" else bf16_bits_to_f32(self.draft)

    def positions(self):
        """Verified draft positions in one call: sum of K_r."""
        return int(np.sum(self.k_per_row))

    @property
    def V_draft(self):
        return self.draft.shape[2]

    def logit_bytes(self):
        """Bytes of logits the sampling verify must read once: K_r + 1
        target rows of V and K_r draft rows of V_draft per request row."""
        es = 4 if self.dtype == "f32" else 2
        k = self.k_per_row.astype(np.int64)
        return int(np.sum(k + 1) * self.V + np.sum(k) * self.V_draft) * es

    def with_(self, **kw):
        return replace(self, **kw)


def _store(x, dtype):
    return x.astype(np.float32) if dtype == "f32" else f32_to_bf16_bits(x)


def _load(x, dtype):
    return x if dtype == "f32" else bf16_bits_to_f32(x)


def gumbel_proposal(rng, z, T):
    """Draft proposal: Gumbel-max over the whole row z/T (an exact sample of
    softmax(z/T))."""
    z = np.asarray(z, dtype=np.float64)
    g = rng.gumbel(size=z.size)
    return int(np.argmax(z / T + g))


def propose(rng, z, T, odd_share=0.0, prior=None, V=None):
    """One draft id: with probability odd_share an odd proposal (half of them
    uniform over [0, V), V the target's vocabulary, by default the draft
    row's length; half a uniformly chosen prior id when the request has prior
    ids), else gumbel_proposal over the draft row.  The draws come from rng in
    a fixed order, so a workload is a function of its seed."""
    V = np.asarray(z).size if V is None else V
    a, b = rng.random(), rng.random()
    x = gumbel_proposal(rng, z, T)
    if a < odd_share:
        if b < 0.5 and prior is not None and len(prior):
            x = int(prior[rng.integers(0, len(prior))])
        else:
            x = int(rng.integers(0, V))
    return x


def _prior(rng, B, n, V, pool=None):
    if pool is None:
        ids = rng.integers(0, V, size=(B, n), dtype=np.int64).astype(np.int32)
    else:
        # n entries per row drawn from `pool` distinct ids (many repeats)
        ids = np.stack([rng.choice(V, size=pool, replace=False)[rng.integers(0, pool, size=n)]
                        for _ in range(B)]).astype(np.int32)
    offs = (np.arange(B + 1, dtype=np.int64) * n).astype(np.int32)
    return ids.reshape(-1), offs


def worked_example(draft_id=0, D=0.0, seed=0):
    """p = [.2,.5,.3], q = [.6,.3,.1] over tokens A, B, C as fp32 log-probs,
    T = 1, K = 1 ("Speculative Decoding" note, section "Eigenes Beispiel").
    The bonus row (position 1) repeats p."""
    lp = np.log(np.array([0.2, 0.5, 0.3])).astype(np.float32)
    lq = np.log(np.array([0.6, 0.3, 0.1])).astype(np.float32)
    return Workload(
        name="worked_example", dtype="f32",
        target=np.stack([lp, lp])[None], draft=lq[None, None],
        draft_ids=np.array([[draft_id]], dtype=np.int32),
        k_per_row=np.array([1], dtype=np.int32),
        temperature=np.array([1.0], dtype=np.float32), tv_budget=D, seed=seed)


def config1(seed=0, D=0.0, philox_seed=0):
    rng = np.random.default_rng([1, seed])
    K, V, T = 4, 1000, np.float32(0.7)
    t = rng.normal(0.0, 2.0, size=(1, K + 1, V)).astype(np.float32)
    d = (t[:, :K] + rng.normal(0.0, 1.0, size=(1, K, V))).astype(np.float32)
    ids = np.array([[gumbel_proposal(rng, d[0, j], T) for j in range(K)]],
                   dtype=np.int32)
    return Workload("config1", "f32", t, d, ids,
                    np.array([K], dtype=np.int32), np.array([T], np.float32),
                    tv_budget=D, seed=philox_seed)


def config2(call=0, D=0.0):
    """Call c: generator seed c, Philox seed c, offset 0."""
    rng = np.random.default_rng([2, call])
    K, V, T = 8, V_QWEN25, np.float32(0.7)
    t = rng.normal(0.0, 3.0, size=(1, K + 1, V)).astype(np.float32)
    d = (0.8 * t[:, :K] + rng.normal(0.0, 1.5, size=(1, K, V))).astype(np.float32)
    ids = np.array([[gumbel_proposal(rng, d[0, j], T) for j in range(K)]],
                   dtype=np.int32)
    pid, poff = _prior(rng, 1, 64, V)
    return Workload("config2", "f32", t, d, ids,
                    np.array([K], dtype=np.int32), np.array([T], np.float32),
                    rep_penalty=1.1, prior_ids=pid, prior_offsets=poff,
                    tv_budget=D, seed=call)


def _corr_rows(rng, t, c, sigma):
    eps = rng.standard_normal(size=t.shape)
    return c * t + np.sqrt(1.0 - c * c) * sigma * eps


def config3(K=8, call=0, B=1, V=V_QWEN3):
    """Greedy: B independent requests (B calls of batch 1 are the same rows
    as one call of batch B)."""
    rng = np.random.default_rng([3, K, call])
    t = rng.normal(0.0, 3.0, size=(B, K + 1, V)).astype(np.float32)
    dr = _corr_rows(rng, t[:, :K], 0.9, 3.0).astype(np.float32)
    tb, db = f32_to_bf16_bits(t), f32_to_bf16_bits(dr)
    ids = np.argmax(bf16_bits_to_f32(db), axis=-1).astype(np.int32)
    return Workload("config3", "bf16", tb, db, ids,
                    np.full(B, K, dtype=np.int32), np.ones(B, np.float32))


def config4_row(seed, r, K=8, V=V_QWEN25, n_prior=128, odd_share=0.0, V_draft=None,
                T_range=(0.5, 1.0)):
    """One request row of config 4, from its own generator stream."""
    rng = np.random.default_rng([4, seed, r])
    T = np.float32(rng.uniform(*T_range))
    t = rng.normal(0.0, 3.0, size=(K + 1, V)).astype(np.float32)
    dr = _corr_rows(rng, t[:K], 0.9, 3.0).astype(np.float32)
    if V_draft is not None:
        dr = dr[:, :V_draft]
    tb, db = f32_to_bf16_bits(t), f32_to_bf16_bits(dr)
    dl = bf16_bits_to_f32(db)
    prior = rng.integers(0, V, size=n_prior).astype(np.int32)
    ids = np.array([propose(rng, dl[j], T, odd_share, prior, V) for j in range(K)],
                   dtype=np.int32)
    return tb, db, ids, T, prior


def config4(seed=0, B=256, K=8, V=V_QWEN25, n_prior=128, D=0.75,
            philox_seed=0, top_p=0.9, rep_penalty=1.1, odd_share=0.0, V_draft=None,
            T_range=(0.5, 1.0)):
    """The batched workload.  Proposals come from the draft's own sampler
    (odd_share = 0, the measured workload); parity runs add odd proposals.
    V_draft: a draft model with a shorter vocabulary (the pages' Qwen2.5
    0.5B draft has 151936 logits against the 7B target's 152064)."""
    Vd = V if V_draft is None else V_draft
    tb = np.empty((B, K + 1, V), dtype=np.uint16)
    db = np.empty((B, K, Vd), dtype=np.uint16)
    ids = np.empty((B, K), dtype=np.int32)
    T = np.empty(B, dtype=np.float32)
    prior = np.empty((B, n_prior), dtype=np.int32)
    for r in range(B):
        tb[r], db[r], ids[r], T[r], prior[r] = config4_row(seed, r, K, V, n_prior, odd_share,
                                                           V_draft, T_range)
    offs = (np.arange(B + 1, dtype=np.int64) * n_prior).astype(np.int32)
    return Workload("config4", "bf16", tb, db, ids,
                    np.full(B, K, dtype=np.int32), T, top_p=top_p,
                    rep_penalty=rep_penalty, prior_ids=prior.reshape(-1),
                    prior_offsets=offs, tv_budget=D, seed=philox_seed)


def _draft_confidence(z, T):
    """The draft sampler's own confidence in a row (the largest probability
    of softmax(z/T)), used only to pick config 5's K_r as the early-stop rule
    would.  Nothing compares against it: the verify step never computes it,
    and the draft-side confidence kernel is checked against the oracle's
    own routine, not this one."""
    a = np.asarray(z, dtype=np.float64) / T
    return 1.0 / np.exp(a - a.max()).sum()


def config5(seed=0, B=512, K_max=8, V=V_QWEN3, T=0.7, threshold=0.6,
            forced_ragged=False):
    """Ragged K from the early-stop rule: K_r = first 1-based position whose
    top-1 draft probability is < threshold (that token is still verified),
    capped at K_max.  forced_ragged: K_r ~ U{1..K_max} instead (supplement)."""
    T = np.float32(T)
    tb = np.zeros((B, K_max + 1, V), dtype=np.uint16)
    db = np.empty((B, K_max, V), dtype=np.uint16)
    ids = np.empty((B, K_max), dtype=np.int32)
    ks = np.empty(B, dtype=np.int32)
    for r in range(B):
        rng = np.random.default_rng([5, seed, r])
        rho = rng.uniform(0.3, 0.95)
        t = rng.normal(0.0, 3.0, size=(K_max + 1, V)).astype(np.float32)
        dr = _corr_rows(rng, t[:K_max], rho, 3.0).astype(np.float32)
        db[r] = f32_to_bf16_bits(dr)
        dl = bf16_bits_to_f32(db[r])
        ids[r] = [gumbel_proposal(rng, dl[j], T) for j in range(K_max)]
        if forced_ragged:
            k = int(rng.integers(1, K_max + 1))
        else:
            k = K_max
            for j in range(K_max):
                if _draft_confidence(dl[j], T) < threshold:
                    k = j + 1
                    break
        ks[r] = k
        tb[r, :k + 1] = f32_to_bf16_bits(t[:k + 1])
    return Workload("config5b" if forced_ragged else "config5", "bf16", tb, db,
                    ids, ks, np.full(B, T, np.float32), tv_budget=0.0,
                    seed=seed)


def random_case(seed, B=3, K_max=3, V=300, dtype="f32", sigma=2.0, corr=0.8,
                T_range=(0.5, 1.5), top_p=1.0, rep_penalty=1.0, n_prior=0,
                D=0.0, ragged=False, philox_seed=None, flags=0, prior_pool=None,
                odd_share=0.1, V_draft=None):
    """Small generic case for parity sweeps (rows span several tiles when V
    is a few thousand, with a ragged tail when V is not a tile multiple).
    V_draft < V: the draft rows hold the first V_draft logits only (a draft
    model with a shorter vocabulary)."""
    rng = np.random.default_rng([9, seed])
    t = rng.normal(0.0, sigma, size=(B, K_max + 1, V)).astype(np.float32)
    dr = _corr_rows(rng, t[:, :K_max], corr, sigma).astype(np.float32)
    if V_draft is not None:
        dr = np.ascontiguousarray(dr[..., :V_draft])
    tt, dd = _store(t, dtype), _store(dr, dtype)
    dl = _load(dd, dtype)
    T = rng.uniform(*T_range, size=B).astype(np.float32)
    pid = poff = None
    if n_prior:
        pid, poff = _prior(rng, B, n_prior, V, prior_pool)
    ids = np.array([[propose(rng, dl[r, j], T[r], odd_share,
                             None if pid is None else pid[poff[r]:poff[r + 1]], V)
                     for j in range(K_max)] for r in range(B)], dtype=np.int32)
    ks = (rng.integers(0, K_max + 1, size=B) if ragged
          else np.full(B, K_max)).astype(np.int32)
    return Workload("random", dtype, tt, dd, ids, ks, T, top_p=top_p,
                    rep_penalty=rep_penalty, prior_ids=pid, prior_offsets=poff,
                    tv_budget=D, seed=seed if philox_seed is None else philox_seed,
                    flags=flags)


# ---------------------------------------------------------------------------
# Hidden states and LM heads for the fused LM-head + verify path.
# ---------------------------------------------------------------------------

QWEN25_7B_HIDDEN = 3584    # the pages' target model's hidden size
QWEN25_05B_HIDDEN = 896    # the pages' draft model's hidden size


@dataclass
class LmHeadWorkload:
    name: str
    target_hidden: np.ndarray   # uint16 bf16 bits [B][K_max+1][H_t]
    draft_hidden: np.ndarray    # uint16 bf16 bits [B][K_max][H_d]
    target_weight: np.ndarray   # uint16 bf16 bits [V][H_t]
    draft_weight: np.ndarray    # uint16 bf16 bits [V_draft][H_d]
    draft_ids: np.ndarray       # int32 [B][K_max]
    k_per_row: np.ndarray       # int32 [B]
    temperature: np.ndarray     # float32 [B]
    tv_budget: float = 0.0
    seed: int = 0
    offset: int = 0
    flags: int = 0

    @property
    def B(self):
        return self.target_hidden.shape[0]

    @property
    def K_max(self):
        return self.target_hidden.shape[1] - 1

    @property
    def V(self):
        return self.target_weight.shape[0]

    @property
    def V_draft(self):
        return self.draft_weight.shape[0]

    def f32(self, name):
        return bf16_bits_to_f32(getattr(self, name))

    def positions(self):
        return int(np.sum(self.k_per_row))

    def with_(self, **kw):
        return replace(self, **kw)


def _dyadic_bf16(rng, shape, scale_steps, lo_hi=None):
    """Values m * 2^-8 with integer m ~ round(N(0, scale_steps)), |m| <= 255
    (exact in bf16), or small integers in [lo, hi] when lo_hi is given."""
    if lo_hi is not None:
        x = rng.integers(lo_hi[0], lo_hi[1] + 1, size=shape).astype(np.float32)
    else:
        m = np.clip(np.rint(rng.normal(0.0, scale_steps, size=shape)), -255, 255)
        x = (m * 2.0 ** -8).astype(np.float32)
    b = f32_to_bf16_bits(x)
    assert np.array_equal(bf16_bits_to_f32(b), x)
    return b


def lmhead_case(seed, B=4, K_max=3, V=4096, V_draft=None, H_t=256, H_d=64, sigma=3.0,
                T_range=(0.6, 1.0), D=0.0, ragged=False, exact=True, flags=0,
                proposals=True):
    """Hidden states and LM-head weights whose logits have standard deviation
    about sigma; the draft's hidden state is the first H_d components of the
    target's (a smaller model that sees part of the same state) and its head
    is the target's first H_d columns scaled by sqrt(H_t / H_d), so draft
    logits correlate with the target's at about sqrt(H_d / H_t).

    exact=True: hidden components are integers in [-2, 2] and weights are
    multiples of 2^-8 below 1 in magnitude, so every product and every partial
    sum of a logit is exact in fp32 (|sum| < 2^13 for H <= 4096: 21 bits);
    the logits are then exactly the fp64 oracle's whatever the summation
    order.  exact=False: N(0, 1) hidden states and N(0, sigma^2 / H) weights
    rounded to bf16 (the measured workload).

    Draft ids come from the draft model's own sampler: Gumbel-max over its
    logits / T (the draft forward a plain fp64 matmul here), when proposals is
    set; else uniform ids."""
    rng = np.random.default_rng([11, seed])
    Vd = V if V_draft is None else V_draft
    if exact:
        th = _dyadic_bf16(rng, (B, K_max + 1, H_t), None, (-2, 2))
        wt = _dyadic_bf16(rng, (V, H_t), 256.0 * sigma / np.sqrt(2.0 * H_t))
    else:
        th = f32_to_bf16_bits(rng.standard_normal((B, K_max + 1, H_t), dtype=np.float32))
        wt = np.empty((V, H_t), dtype=np.uint16)
        for i0 in range(0, V, 8192):   # in chunks: full-size heads are large
            i1 = min(V, i0 + 8192)
            wt[i0:i1] = f32_to_bf16_bits(
                rng.standard_normal((i1 - i0, H_t), dtype=np.float32) * np.float32(sigma / np.sqrt(H_t)))
    dh = np.ascontiguousarray(th[:, :K_max, :H_d])
    wd_f = bf16_bits_to_f32(wt[:Vd, :H_d]) * np.float32(np.sqrt(H_t / H_d))
    if exact:   # back onto the 2^-8 grid, |m| <= 255
        wd_f = (np.clip(np.rint(wd_f * 256.0), -255, 255) / 256.0).astype(np.float32)
    wd = f32_to_bf16_bits(wd_f)
    T = rng.uniform(*T_range, size=B).astype(np.float32)
    ids = np.empty((B, K_max), dtype=np.int32)
    if proposals and K_max > 0:
        dhf, wdf = bf16_bits_to_f32(dh).astype(np.float64), bf16_bits_to_f32(wd).astype(np.float64)
        for r in range(B):
            z = dhf[r] @ wdf.T
            for j in range(K_max):
                ids[r, j] = gumbel_proposal(rng, z[j], T[r])
    else:
        ids[:] = rng.integers(0, V, size=ids.shape)
    ks = (rng.integers(0, K_max + 1, size=B) if ragged else np.full(B, K_max)).astype(np.int32)
    return LmHeadWorkload("lmhead", th, dh, wt, wd, ids, ks, T, tv_budget=D, seed=seed,
                          flags=flags)
