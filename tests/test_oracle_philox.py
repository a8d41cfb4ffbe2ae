"""Pins for the oracle's Philox4x32-10 (CPU only).

The pages fix no random source; the oracle's generator is Philox4x32-10 from
its published definition (Salmon et al., SC'11).  It is pinned against
rocRAND's host-callable engine of the same function, an independent library
implementation, and checked for uniformity.
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
from scipy import stats

from oracle.philox import philox4x32_10, to_unit, uniforms_for

HERE = os.path.dirname(os.path.abspath(__file__))


def _rocrand_blocks(tuples):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND pin helper")
    with tempfile.TemporaryDirectory() as td:
        exe = os.path.join(td, "pin")
        subprocess.run([hipcc, "-O1", "-x", "hip", "--offload-arch=gfx950",
                        os.path.join(HERE, "philox_rocrand_pin.cpp"), "-o", exe],
                       check=True, capture_output=True)
        inp = "".join(f"{s} {r} {p} {o}\n" for s, r, p, o in tuples)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True,
                             check=True).stdout
    return np.array([[int(w) for w in ln.split()] for ln in out.strip().splitlines()],
                    dtype=np.uint64)


def test_philox_matches_rocrand():
    rng = np.random.default_rng(123)
    # rocRAND takes the position as an offset in 32-bit outputs (4 per block),
    # so rows stay below 2^30 to keep 4*(pos + row*2^32) inside 64 bits.
    tuples = [(0, 0, 0, 0), (1, 2, 3, 4), (2**64 - 1, 2**30 - 1, 2**32 - 1, 2**64 - 1)]
    for _ in range(200):
        tuples.append((int(rng.integers(0, 2**63)), int(rng.integers(0, 2**30)),
                       int(rng.integers(0, 2**32)), int(rng.integers(0, 2**63))))
    ref = _rocrand_blocks(tuples)
    ctr = np.array([[p, r, o & 0xFFFFFFFF, o >> 32] for s, r, p, o in tuples],
                   dtype=np.uint64)
    key = np.array([[s & 0xFFFFFFFF, s >> 32] for s, r, p, o in tuples],
                   dtype=np.uint64)
    got = philox4x32_10(ctr, key).astype(np.uint64)
    assert np.array_equal(got, ref)


def test_uniform_mapping_exact_and_in_range():
    w = np.array([0, 255, 256, 2**32 - 1], dtype=np.uint64)
    u = to_unit(w)
    assert u[0] == 0.0 and u[1] == 0.0 and u[2] == 2.0 ** -24
    assert u[3] == 1.0 - 2.0 ** -24
    # exact in fp32
    assert np.array_equal(u.astype(np.float32).astype(np.float64), u)


def test_uniforms_are_uniform():
    n = 1 << 20
    rows = np.arange(n) // 16
    pos = np.arange(n) % 16
    u, v = uniforms_for(7, 3, rows, pos)
    assert stats.kstest(u, "uniform").pvalue > 1e-4
    assert stats.kstest(v, "uniform").pvalue > 1e-4
    # u and v are different words of the block
    assert abs(np.corrcoef(u, v)[0, 1]) < 0.01


def test_streams_differ_by_row_position_offset():
    u1, _ = uniforms_for(0, 0, [0, 1, 0], [0, 0, 1])
    u2, _ = uniforms_for(0, 1, [0], [0])
    assert len(set(u1.tolist() + u2.tolist())) == 4
