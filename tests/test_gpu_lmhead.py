"""The verify step fed from hidden states through the LM heads, on the GPU.

The exact workloads (integer hidden states times multiples of 2^-8 as head
weights) have logits that fp32 accumulates exactly in any order, so the
MFMA tile engine's logits equal the oracle's fp64 ones bit for bit and the
fused verify is held to the same bar as the plain one: decisions bit-exact
outside near-ties, statistics within 1e-5.  Gaussian inputs check the tile
engine against the fp64 product within the bound of fp32 summation:
|error| <= (H + 1) 2^-24 sum_k |h_k W_ik|.
"""
import numpy as np
import pytest

import workloads as wl
from parity import compare_greedy, compare_sample

pytestmark = pytest.mark.gpu


def _sdv():
    import speculative_sampling_verify_temp_amd as sdv
    return sdv


def _dev(w):
    import torch

    def bf(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)

    return dict(th=bf(w.target_hidden), dh=bf(w.draft_hidden), wt=bf(w.target_weight),
                wd=bf(w.draft_weight), ids=torch.from_numpy(w.draft_ids).cuda(),
                k=torch.from_numpy(w.k_per_row).cuda(),
                T=torch.from_numpy(np.ascontiguousarray(w.temperature, np.float32)).cuda())


def _args(w, d, sample=True):
    sdv = _sdv()
    if sample:
        return sdv.make_lmhead_args(d["th"], d["wt"], d["ids"], d["dh"], d["wd"], d["k"], d["T"],
                                    w.tv_budget, w.seed, w.offset, w.flags)
    return sdv.make_lmhead_args(d["th"], d["wt"], d["ids"], k_per_row=d["k"], flags=w.flags)


def gpu_lm_sample(w, stats=True):
    import torch
    sdv = _sdv()
    d = _dev(w)
    a = _args(w, d)
    B, K1 = w.B, w.K_max + 1
    acc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    tok = torch.full((B, K1), -7, dtype=torch.int32, device="cuda")
    st = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    sts = torch.full((B, K1, sdv.SD_NSTAT), -7.0, device="cuda") if stats else None
    sdv.lmhead_verify_sample(a, acc, tok, st, sts)
    torch.cuda.synchronize()
    return dict(accepted=acc.cpu().numpy(), tokens=tok.cpu().numpy(),
                status=st.cpu().numpy().astype(np.uint32),
                stats=None if sts is None else sts.cpu().numpy().astype(np.float64))


def gpu_lm_greedy(w):
    import torch
    sdv = _sdv()
    d = _dev(w)
    a = _args(w, d, sample=False)
    B, K1 = w.B, w.K_max + 1
    acc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    tok = torch.full((B, K1), -7, dtype=torch.int32, device="cuda")
    st = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    am = torch.full((B, K1), -7, dtype=torch.int32, device="cuda")
    sdv.lmhead_verify_greedy(a, acc, tok, st, am)
    torch.cuda.synchronize()
    return dict(accepted=acc.cpu().numpy(), tokens=tok.cpu().numpy(),
                status=st.cpu().numpy().astype(np.uint32), argmax=am.cpu().numpy())


def oracle_lm_sample(w, rows=None):
    from oracle import lmhead_verify_sample_ref
    return lmhead_verify_sample_ref(w.f32("target_hidden"), w.f32("draft_hidden"),
                                    w.f32("target_weight"), w.f32("draft_weight"), w.draft_ids,
                                    w.k_per_row, w.temperature, w.tv_budget, w.seed, w.offset,
                                    w.flags, rows=rows)


def oracle_lm_greedy(w, rows=None):
    from oracle import lmhead_verify_greedy_ref
    return lmhead_verify_greedy_ref(w.f32("target_hidden"), w.f32("target_weight"), w.draft_ids,
                                    w.k_per_row, w.flags, rows=rows)


def _used_rows(w):
    for r in range(w.B):
        K = int(w.k_per_row[r])
        for j in range(K + 1):
            yield r, j, j < K


@pytest.mark.parametrize("exact", [True, False])
@pytest.mark.parametrize("shape", [dict(V=1000, V_draft=900, H_t=128, H_d=64, B=3, K_max=2),
                                   dict(V=5003, V_draft=5003, H_t=256, H_d=128, B=5, K_max=3,
                                        ragged=True)],
                         ids=["ragged_tiles", "ragged_k"])
def test_lmhead_logits(shape, exact):
    """The tile engine's logits of every used row against the fp64 product:
    equal on the exact inputs, within the fp32 summation bound otherwise."""
    import torch
    from oracle import lmhead_logits
    sdv = _sdv()
    w = wl.lmhead_case(1700 + shape["V"], exact=exact, proposals=False, **shape)
    d = _dev(w)
    a = _args(w, d)
    ot = torch.full((w.B, w.K_max + 1, w.V), np.nan, device="cuda")
    od = torch.full((w.B, w.K_max, w.V_draft), np.nan, device="cuda")
    sdv.debug_lmhead_logits(a, ot, od)
    torch.cuda.synchronize()
    ot, od = ot.cpu().numpy().astype(np.float64), od.cpu().numpy().astype(np.float64)
    h, W = w.f32("target_hidden"), w.f32("target_weight")
    hd, Wd = w.f32("draft_hidden"), w.f32("draft_weight")
    zt, zd = lmhead_logits(h, W), lmhead_logits(hd, Wd)
    bt = (h.shape[-1] + 1) * 2.0 ** -24 * (np.abs(h) @ np.abs(W).T)
    bd = (hd.shape[-1] + 1) * 2.0 ** -24 * (np.abs(hd) @ np.abs(Wd).T)
    n = 0
    for r, j, has_d in _used_rows(w):
        if exact:
            np.testing.assert_array_equal(ot[r, j], zt[r, j], err_msg=f"target {r},{j}")
            if has_d:
                np.testing.assert_array_equal(od[r, j], zd[r, j], err_msg=f"draft {r},{j}")
        else:
            assert (np.abs(ot[r, j] - zt[r, j]) <= bt[r, j]).all(), (r, j)
            if has_d:
                assert (np.abs(od[r, j] - zd[r, j]) <= bd[r, j]).all(), (r, j)
        n += 1
    assert n > 0


SAMPLE_CASES = [
    dict(B=6, K_max=3, V=1000, V_draft=1000, H_t=128, H_d=64, D=0.0),
    dict(B=6, K_max=3, V=1000, V_draft=930, H_t=128, H_d=64, D=0.3, ragged=True),
    dict(B=5, K_max=4, V=4099, V_draft=4000, H_t=256, H_d=128, D=0.75, T_range=(0.5, 1.0)),
    dict(B=5, K_max=2, V=3001, V_draft=3001, H_t=192, H_d=64, D=1.0),
    dict(B=4, K_max=3, V=2048, V_draft=2048, H_t=128, H_d=128, D=0.2, flags=1),
    dict(B=4, K_max=0, V=777, V_draft=777, H_t=64, H_d=64, D=0.5),
]


@pytest.mark.parametrize("i", range(len(SAMPLE_CASES)))
def test_lmhead_sample_parity(i):
    tot = [0, 0]
    for seed in range(3):
        w = wl.lmhead_case(1800 + 10 * i + seed, **SAMPLE_CASES[i])
        g, o = gpu_lm_sample(w), oracle_lm_sample(w)
        c, f = compare_sample(g, o, w)
        tot[0] += c
        tot[1] += f
    print(f"lmhead sample case {i}: checked {tot[0]}, near-tie {tot[1]}")
    assert tot[0] >= 0.9 * (tot[0] + tot[1])


def test_lmhead_sample_without_stats_skips_tv_when_not_needed():
    """D = 0 without statistics takes no TV pass; the decisions still match."""
    w = wl.lmhead_case(1900, B=8, K_max=3, V=3000, V_draft=2990, H_t=128, H_d=64, D=0.0)
    g, o = gpu_lm_sample(w, stats=False), oracle_lm_sample(w)
    c, f = compare_sample(g, o, w)
    assert c >= 7


def test_lmhead_sample_invalid_requests():
    w = wl.lmhead_case(1910, B=5, K_max=3, V=1000, H_t=64, H_d=64, D=0.4)
    w.k_per_row[0] = 5            # bad K
    w.draft_ids[1, 2] = 1000      # bad draft id
    w.temperature[2] = 0.0        # bad temperature
    w.draft_ids[3, 0] = w.V - 1   # a proposal (valid)
    g, o = gpu_lm_sample(w), oracle_lm_sample(w)
    compare_sample(g, o, w)
    assert list(g["status"][:3]) == [1, 4, 2]


@pytest.mark.parametrize("case", [dict(B=6, K_max=3, V=1000, H_t=128, H_d=64),
                                  dict(B=5, K_max=4, V=4099, H_t=256, H_d=64, ragged=True),
                                  dict(B=4, K_max=2, V=2000, H_t=64, H_d=64, flags=1)],
                         ids=["small", "ragged", "no_bonus"])
def test_lmhead_greedy_parity(case):
    for seed in range(3):
        w = wl.lmhead_case(1950 + seed, **case)
        # make some proposals the target's argmax, so prefixes get accepted
        from oracle import lmhead_logits
        zt = lmhead_logits(w.f32("target_hidden"), w.f32("target_weight"))
        rng = np.random.default_rng(seed)
        for r in range(w.B):
            for j in range(w.K_max):
                if rng.random() < 0.7:
                    w.draft_ids[r, j] = int(np.argmax(zt[r, j]))
        compare_greedy(gpu_lm_greedy(w), oracle_lm_greedy(w), range(w.B))


@pytest.fixture(scope="module")
def qwen_pair():
    """The pages' model pair at full size: target head 152064 x 3584, draft
    head 151936 x 896 (exact inputs)."""
    return wl.lmhead_case(2000, B=12, K_max=8, V=wl.V_QWEN25, V_draft=wl.V_QWEN3,
                          H_t=wl.QWEN25_7B_HIDDEN, H_d=wl.QWEN25_05B_HIDDEN, D=0.0,
                          T_range=(0.6, 0.8))


@pytest.mark.parametrize("D", [0.0, 0.5])
def test_lmhead_full_size_sample(qwen_pair, D):
    w = qwen_pair.with_(tv_budget=D)
    g = gpu_lm_sample(w)
    rows = [0, 3, 7, 11]
    o = oracle_lm_sample(w, rows=rows)
    c, f = compare_sample(g, o, w, rows=rows)
    print(f"lmhead full size D={D}: checked {c}, near-tie {f}, accepted {g['accepted'].tolist()}")
    assert c >= 3
    assert ((g["accepted"] >= 0) & (g["accepted"] <= w.k_per_row)).all()


def test_lmhead_full_size_greedy(qwen_pair):
    w = qwen_pair
    g = gpu_lm_greedy(w)
    rows = [1, 5]
    compare_greedy(g, oracle_lm_greedy(w, rows=rows), rows)
