"""Exact output law of the oracle's sampling verify on tiny inputs.

Uniforms live on the 2^24 grid {k * 2^-24}.  The accept decision at a
position is monotone in u (accepted for small u) and the inverse-CDF draw is
monotone non-decreasing in v, so the law of the oracle's output can be
computed exactly with binary searches over the grid instead of 2^24 calls.
Everything here calls the oracle's public row function; nothing restates its
arithmetic.
"""
import numpy as np

from oracle.verify import verify_sample_row, process_dist, draft_row_over_target

GRID = 1 << 24


def _first_true(pred, lo=0, hi=GRID):
    """Smallest k in [lo, hi] with pred(k) True, for pred monotone F..F T..T
    over [lo, hi) (returns hi when never True)."""
    while lo < hi:
        mid = (lo + hi) // 2
        if pred(mid):
            hi = mid
        else:
            lo = mid + 1
    return lo


class RowModel:
    """A one-row problem: target rows [K+1][V], draft rows [K][V_d] (fp32,
    V_d <= V: the draft's tail tokens have q = 0)."""

    def __init__(self, tgt, drf, prior=(), T=1.0, top_p=1.0, r_pen=1.0, D=0.0,
                 flags=0):
        self.tgt, self.drf = np.asarray(tgt, np.float32), np.asarray(drf, np.float32)
        self.K = self.drf.shape[0]
        self.V = self.tgt.shape[1]
        self.prior, self.T, self.top_p = list(prior), T, top_p
        self.r_pen, self.D, self.flags = r_pen, D, flags

    def run(self, x, u, v):
        return verify_sample_row(self.tgt, self.drf, np.asarray(x), self.K,
                                 self.prior, self.T, self.top_p, self.r_pen,
                                 self.D, np.asarray(u, float), np.asarray(v, float),
                                 self.V, self.flags)

    def q(self, j, prefix):
        """The proposal law at position j given the accepted prefix: the
        oracle's processed draft distribution."""
        pen = list(self.prior) if (self.flags & 2) else list(self.prior) + list(prefix)
        return process_dist(draft_row_over_target(self.drf[j], self.V), pen, self.r_pen,
                            self.T, self.top_p).p

    def law(self):
        """dict: tuple(emitted tokens) -> probability, with x_j ~ q_j."""
        K = self.K
        out = {}

        def draw_law(x, j, u_fixed, weight):
            # position j is where the scan stopped; enumerate v_j
            def tok(k):
                v = np.zeros(K + 1)
                v[j] = k / GRID
                return self.run(x, u_fixed, v).tokens[-1]

            k = 0
            while k < GRID:
                t = tok(k)
                nxt = _first_true(lambda m: tok(m) != t, k, GRID)
                seq = tuple(x[:j]) + (t,)
                out[seq] = out.get(seq, 0.0) + weight * (nxt - k) / GRID
                k = nxt

        def rec(j, x, u_fixed, weight):
            if j == K:
                if self.flags & 1:
                    seq = tuple(x[:K])
                    out[seq] = out.get(seq, 0.0) + weight
                    return
                draw_law(x, K, u_fixed, weight)
                return
            qj = self.q(j, x[:j])
            for a in range(self.V):
                if qj[a] == 0.0:
                    continue
                xx = list(x[:j]) + [a] + [0] * (K - j - 1)

                def accepted(k):
                    u = np.array(u_fixed, float)
                    u[j] = k / GRID
                    return self.run(xx, u, np.zeros(K + 1)).accepted > j

                n_acc = _first_true(lambda k: not accepted(k))
                if n_acc > 0:
                    u = np.array(u_fixed, float)
                    u[j] = 0.0
                    rec(j + 1, xx, u, weight * qj[a] * n_acc / GRID)
                if n_acc < GRID:
                    u = np.array(u_fixed, float)
                    u[j] = (GRID - 1) / GRID
                    draw_law(xx, j, u, weight * qj[a] * (GRID - n_acc) / GRID)

        rec(0, [0] * K, np.zeros(K + 1), 1.0)
        return out


def marginal(law, pos, cond_prefix=None):
    """Law of emitted token at index pos, optionally conditioned on the first
    pos emitted tokens equal to cond_prefix and the sequence continuing."""
    acc = {}
    tot = 0.0
    for seq, pr in law.items():
        if len(seq) <= pos:
            continue
        if cond_prefix is not None and tuple(seq[:pos]) != tuple(cond_prefix):
            continue
        acc[seq[pos]] = acc.get(seq[pos], 0.0) + pr
        tot += pr
    return acc, tot
