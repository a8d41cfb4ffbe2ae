"""Philox4x32-10, written from its published definition.

Source of the definition: Salmon, Moraes, Dror, Shaw, "Parallel random
numbers: as easy as 1, 2, 3" (SC'11), section on the Philox family.  A Philox
round takes a 4-word counter (c0, c1, c2, c3) and a 2-word key (k0, k1),
forms the two 32x32->64 products M0*c0 and M1*c2, and outputs
(hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)).  Between
rounds the key is bumped by the Weyl constants (0x9E3779B9, 0xBB67AE85).
Ten rounds make Philox4x32-10.

The pages are silent on the random source of the verify step (the
"Speculative Decoding" note, section "Eigenes Beispiel", only warns that
algorithms consume randomness differently).  The reading used here: one
Philox block per (row r, position j), key = (seed_lo, seed_hi), counter =
(j, r, offset_lo, offset_hi); word 0 gives the acceptance uniform u_j and word
1 the draw uniform v_j, each as (w >> 8) * 2^-24, which is exact in fp32 and
fp64 and lies in [0, 1).

Parity: pinned against rocRAND's host-callable Philox4x32-10 engine (a third
party library routine of the same published function), see
tests/test_oracle_philox.py.
"""

import numpy as np

M0 = np.uint64(0xD2511F53)
M1 = np.uint64(0xCD9E8D57)
W0 = 0x9E3779B9
W1 = 0xBB67AE85
MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(counter, key):
    """Philox4x32-10 block function.

    counter: uint32 array of shape (..., 4); key: uint32 array of shape (..., 2)
    (broadcastable).  Returns uint32 array of shape (..., 4).
    """
    c = np.asarray(counter, dtype=np.uint64) & MASK32
    k = np.asarray(key, dtype=np.uint64) & MASK32
    c0, c1, c2, c3 = (c[..., i] for i in range(4))
    k0, k1 = k[..., 0], k[..., 1]
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + np.uint64(W0)) & MASK32
            k1 = (k1 + np.uint64(W1)) & MASK32
        p0 = M0 * c0          # < 2^64, exact in uint64
        p1 = M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    out = np.stack([c0, c1, c2, c3], axis=-1)
    return out.astype(np.uint32)


def to_unit(word):
    """Map a uint32 word to [0, 1): (w >> 8) * 2^-24 (exact in fp32/fp64)."""
    w = np.asarray(word, dtype=np.uint64)
    return (w >> np.uint64(8)).astype(np.float64) * (2.0 ** -24)


def uniforms_for(seed, offset, rows, positions):
    """Acceptance and draw uniforms for (row, position) pairs.

    rows, positions: integer arrays of equal shape.  Returns (u, v) float64
    arrays of that shape, from words 0 and 1 of the block at counter
    (position, row, offset_lo, offset_hi) under key (seed_lo, seed_hi).
    """
    rows = np.asarray(rows, dtype=np.uint64)
    positions = np.asarray(positions, dtype=np.uint64)
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    offset = int(offset) & 0xFFFFFFFFFFFFFFFF
    shape = np.broadcast(rows, positions).shape
    ctr = np.empty(shape + (4,), dtype=np.uint64)
    ctr[..., 0] = positions
    ctr[..., 1] = rows
    ctr[..., 2] = offset & 0xFFFFFFFF
    ctr[..., 3] = offset >> 32
    key = np.array([seed & 0xFFFFFFFF, seed >> 32], dtype=np.uint64)
    blk = philox4x32_10(ctr, key)
    return to_unit(blk[..., 0]), to_unit(blk[..., 1])
