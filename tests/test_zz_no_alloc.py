"""sd_verify_sample_noalloc against sd_verify_sample, on the GPU.

The no-allocation entry point runs the same kernels with the library's
built-in scratch array as the workspace, so its outputs must equal those of
sd_verify_sample on the same inputs bit for bit.  Two calls in a row, the
second smaller than the first (the array keeps the first call's contents),
on the single-pass path and then the general path.
"""
import numpy as np
import pytest

import workloads as wl
from parity import to_device

pytestmark = pytest.mark.gpu


def _outputs(sdv, w, d, noalloc):
    import torch
    args = sdv.make_args(d["target"], d["draft"], d["draft_ids"], d["k_per_row"],
                         d["temperature"], w.top_p, w.rep_penalty, d["prior_ids"],
                         d["prior_offsets"], w.tv_budget, w.seed, w.offset, w.flags)
    dev = d["target"].device
    B, K1 = args.B, args.K_max + 1
    # sentinel-filled outputs, so an output the call fails to write shows
    acc = torch.full((B,), -7, dtype=torch.int32, device=dev)
    tok = torch.full((B, K1), -7, dtype=torch.int32, device=dev)
    st = torch.full((B,), -7, dtype=torch.int32, device=dev)
    sts = torch.full((B, K1, sdv.SD_NSTAT), -7.0, dtype=torch.float32, device=dev)
    if noalloc:
        sdv.verify_sample_noalloc(args, acc, tok, st, sts)
    else:
        sdv.verify_sample(d["target"], d["draft"], d["draft_ids"], d["k_per_row"],
                          d["temperature"], w.top_p, w.rep_penalty, d["prior_ids"],
                          d["prior_offsets"], w.tv_budget, w.seed, w.offset, w.flags,
                          stats=True, out=dict(accepted=acc, tokens=tok, status=st, stats=sts))
    torch.cuda.synchronize()
    return args, [x.cpu().numpy() for x in (acc, tok, st, sts)]


CASES = [
    ("single_pass", dict(seed=1401, B=64, K_max=8, V=wl.V_QWEN25, dtype="bf16", sigma=3.0, corr=0.9,
                         T_range=(0.5, 1.0), top_p=0.9, rep_penalty=1.1, n_prior=32, D=0.75)),
    ("single_pass_smaller", dict(seed=1402, B=7, K_max=3, V=20011, dtype="bf16", sigma=3.0,
                                 top_p=0.9, D=0.0, ragged=True)),
    ("general", dict(seed=1403, B=12, K_max=4, V=30011, dtype="f32", sigma=3.0, D=0.5,
                     rep_penalty=1.2, n_prior=8)),
    ("general_smaller", dict(seed=1404, B=3, K_max=2, V=999, dtype="f32", D=0.3, top_p=0.8)),
]


def test_noalloc_matches_workspace_entry_point():
    import speculative_sampling_verify_temp_amd as sdv
    for name, kw in CASES:
        print(f"no-alloc case {name}: B={kw['B']} K={kw['K_max']} V={kw['V']} {kw['dtype']}", flush=True)
        w = wl.random_case(**kw)
        d = to_device(w)
        args, got = _outputs(sdv, w, d, noalloc=True)
        assert sdv.workspace_bytes(args) <= sdv.SD_NOALLOC_MAX_WORKSPACE
        _, ref = _outputs(sdv, w, d, noalloc=False)
        for g, r, what in zip(got, ref, ("accepted", "tokens", "status", "stats")):
            assert np.array_equal(g, r), (name, what)
        assert (got[0] >= -1).all() and (got[0] <= w.K_max).all()


def test_noalloc_rejects_calls_beyond_the_scratch_size():
    import torch
    import speculative_sampling_verify_temp_amd as sdv
    w = wl.random_case(1405, B=4, K_max=2, V=64, dtype="f32")
    d = to_device(w)
    args = sdv.make_args(d["target"], d["draft"], d["draft_ids"], d["k_per_row"],
                         d["temperature"])
    args.B = 100000   # host-side size check only: nothing is enqueued
    acc = torch.empty(4, dtype=torch.int32, device="cuda")
    tok = torch.empty((4, 3), dtype=torch.int32, device="cuda")
    with pytest.raises(sdv.SdVerifyError) as e:
        sdv.verify_sample_noalloc(args, acc, tok)
    assert e.value.code == sdv.SD_ESCRATCH
