#!/usr/bin/env python3
"""Throughput of the speculative-sampling verify step on one MI355X.

Workload: 256 requests x K=8 draft positions, V=152064, bf16 logits ~N(0,3^2)
(draft rows correlated 0.9 with the target), per-request temperature
U[0.5,1.0], top-p 0.9, repetition penalty 1.1 over 128 prior ids plus the
draft prefix, TV budget 0.75, Philox per-request streams.  Inputs are seeded,
synthetic and resident in HBM before the timed region.

One step = one sd_verify_sample call over the whole batch, issued as its
phases on torch's current stream so the dominant kernel can be bracketed by
HIP events inside the timed region.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps 100] [--warmup 60] [--no-cpu-baseline]
                    [--copy-probe BYTES]

The default warmup is long on purpose: after an idle spell the first ~40
back-to-back calls run through a clock transient (the dominant kernel takes
up to ~1.25x its sustained time), and the timed steps should see the
sustained rate.  With a shorter --warmup W the bench still runs untimed
steps until SETTLE_STEPS have run in all (the line's settle_steps says how
many it added).

`roofline.traffic` is the dominant kernel's HBM bytes per launch from two
rocprofv3 counter runs (FETCH_SIZE, then WRITE_SIZE) of this script with
--copy-probe, which runs one plain streaming kernel over BYTES (read BYTES,
write BYTES) before the warmup so the same counters can be scaled to the
bytes that kernel is known to move.  `python bench.py --digest-pmc FETCH_CSV WRITE_CSV` turns the two
counter files into the traffic record; the record names a hash of the kernel
sources and is ignored (traffic null) once they change.
"""
import argparse
import csv
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified draft positions/sec at V=152064 + achieved HBM GB/s vs peak"
PEAK_HBM_GBPS = 8000.0
CSRC = os.path.join(ROOT, "speculative_sampling_verify_temp_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_k_pair_fast_256x8_V152064.json")
COPY_KERNEL = "bitwise_not"   # the calibration kernel: reads N bytes, writes N bytes
WORKLOAD = ("256 requests x K=8, V=152064, bf16 logits, T~U[0.5,1], top-p 0.9, "
            "penalty 1.1 (128 prior ids + draft prefix), TV budget 0.75")


# The sources k_pair_fast is built from (the confidence kernel's file is not
# one of them).
# Untimed steps before the timed region, at least (W included).
SETTLE_STEPS = 40

VERIFY_SOURCES = ("sd_verify.hip", "sdv_device.h", "sdv_exact.h")


def source_hash():
    """sha256 over the verify kernels' sources, in name order."""
    h = hashlib.sha256()
    for n in sorted(VERIFY_SOURCES):
        h.update(n.encode())
        h.update(open(os.path.join(CSRC, n), "rb").read())
    return h.hexdigest()


def algorithmic_bytes(kernel, w, accepted=None):
    """Bytes the kernel must move per launch by definition of its work.

    The single-pass kernel and the general row pass read every logit row of
    the call once (the single pass's exact route re-reads the rows of units
    it could not settle: that is extra traffic, not algorithmic bytes); the
    general TV pass reads the 2K draft-position rows of each request; the
    general draw reads, per request, the target and draft row of the first
    rejected position, or the bonus row (accepted: the accepted lengths).
    Otherwise 0.
    """
    import numpy as np
    es = 2 if w.dtype == "bf16" else 4
    if kernel in ("k_pair_fast", "k_row_prepare"):
        return w.logit_bytes()
    if kernel == "k_pair_tv":
        return 2 * w.K_max * w.V * es * w.B
    if kernel == "k_finalize" and accepted is not None:
        rows = np.where(accepted < w.k_per_row, 2, 1)
        return int(rows.sum()) * w.V * es
    return 0


def read_counters(path, counter, kernel):
    """Per-dispatch values of `counter` for the kernels whose name contains
    `kernel` (rocprofv3 counter CSV)."""
    out = []
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] == counter and kernel in row["Kernel_Name"]:
                out.append(float(row["Counter_Value"]))
    if not out:
        raise SystemExit(f"no {counter} records for a kernel named like {kernel!r} in {path}")
    return out


def digest_pmc(fetch_csv, write_csv, copy_bytes, out_path):
    """Traffic record of k_pair_fast from FETCH_SIZE / WRITE_SIZE runs (KiB)."""
    import numpy as np
    med = lambda path, ctr, k: float(np.median(read_counters(path, ctr, k)))  # noqa: E731
    cf, cw = med(fetch_csv, "FETCH_SIZE", COPY_KERNEL), med(write_csv, "WRITE_SIZE", COPY_KERNEL)
    kf = med(fetch_csv, "FETCH_SIZE", "k_pair_fast")
    kw = med(write_csv, "WRITE_SIZE", "k_pair_fast")
    sf, sw = copy_bytes / (cf * 1024.0), copy_bytes / (cw * 1024.0)
    rec = {
        "kernel": "k_pair_fast", "workload": WORKLOAD, "source_sha256": source_hash(),
        "copy_kernel": COPY_KERNEL, "copy_bytes": copy_bytes,
        "copy_fetch_kib": cf, "copy_write_kib": cw,
        "fetch_scale": sf, "write_scale": sw,
        "kernel_fetch_kib": kf, "kernel_write_kib": kw,
        "traffic_bytes": kf * 1024.0 * sf + kw * 1024.0 * sw,
        "commands": [
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_fetch -o run "
            f"-- python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --copy-probe {copy_bytes}",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_write -o run "
            f"-- python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --copy-probe {copy_bytes}",
            f"python3 bench.py --digest-pmc gpurun_out/pmc_fetch/run_counter_collection.csv "
            f"gpurun_out/pmc_write/run_counter_collection.csv --copy-probe {copy_bytes}"],
    }
    with open(out_path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


def measured_traffic(kernel):
    """Counter-derived bytes per launch, or None (no record, other kernel, or
    the kernel sources changed since the counters were taken)."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel") != kernel or rec.get("source_sha256") != source_hash():
        return None
    return rec["traffic_bytes"]


def cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def device_inputs(w, torch, dev):
    """Copy a workload to the device (bf16 as raw 16-bit patterns)."""
    import numpy as np
    t = torch.from_numpy(w.target.view(np.int16)).to(dev).view(torch.bfloat16)
    d = torch.from_numpy(w.draft.view(np.int16)).to(dev).view(torch.bfloat16)

    def i32(x):
        return None if x is None else torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(dev)

    return dict(target=t, draft=d, draft_ids=i32(w.draft_ids), k_per_row=i32(w.k_per_row),
                temperature=torch.from_numpy(w.temperature).to(dev),
                prior_ids=i32(w.prior_ids), prior_offsets=i32(w.prior_offsets))


def cpu_baseline(w, budget_s=12.0):
    """The oracle, as it stands, on a bounded sample of request rows."""
    import oracle
    rows, t0 = [], time.perf_counter()
    tf, df = w.target_f32(), w.draft_f32()
    r = 0
    while r < w.B and (len(rows) < 2 or time.perf_counter() - t0 < budget_s):
        oracle.verify_sample_ref(tf, df, w.draft_ids, w.k_per_row, w.temperature, w.top_p,
                                 w.rep_penalty, w.prior_ids, w.prior_offsets, w.tv_budget,
                                 w.seed, w.offset, w.flags, rows=[r])
        rows.append(r)
        r += 1
    el = time.perf_counter() - t0
    pos = int(sum(int(w.k_per_row[i]) for i in rows))
    return {"value": pos / el, "unit": "positions/s", "cores": 1, "kind": "oracle",
            "sample": f"request rows 0..{len(rows) - 1} ({len(rows)} of {w.B}, {pos} positions) "
                      f"of the same workload in {el:.1f} s, numpy fp64 on one thread of "
                      f"{cpu_model()} ({os.cpu_count()} logical CPUs visible)"}


def _one_thread():
    """Pool initializer: one numpy/BLAS thread per worker process."""
    os.environ["OMP_NUM_THREADS"] = "1"
    os.environ["OPENBLAS_NUM_THREADS"] = "1"


def _oracle_task(task):
    """One request row of the oracle in a worker process (spawned, so it
    shares nothing with a process that touched the GPU); returns its seconds."""
    kind, payload = task
    import oracle
    t0 = time.perf_counter()
    if kind == "sample":
        oracle.verify_sample_ref(*payload)
    elif kind == "greedy":
        oracle.verify_greedy_ref(*payload)
    else:   # warm-up: imports only
        pass
    return time.perf_counter() - t0


def sample_tasks(w):
    """The workload's request rows as one-row oracle calls (row r's arrays
    only; the cost of a row does not depend on its index)."""
    tf, df = w.target_f32(), w.draft_f32()
    for r in range(w.B):
        prior = offs = None
        if w.prior_ids is not None:
            prior = w.prior_ids[w.prior_offsets[r]:w.prior_offsets[r + 1]]
            offs = [0, len(prior)]
        yield ("sample", (tf[r:r + 1], df[r:r + 1], w.draft_ids[r:r + 1], w.k_per_row[r:r + 1],
                          w.temperature[r:r + 1], w.top_p, w.rep_penalty, prior, offs, w.tv_budget,
                          w.seed, w.offset, w.flags)), int(w.k_per_row[r])


def cpu_baseline_all_cores(tasks, unit_per_task="positions", budget_s=12.0, workers=None):
    """The oracle, as it stands, over request rows in a pool of worker
    processes (one numpy thread each), until about budget_s of wall time."""
    import multiprocessing as mp
    n = workers or min(os.cpu_count() or 1, 16)
    ctx = mp.get_context("spawn")
    with ctx.Pool(n, initializer=_one_thread) as pool:
        pool.map(_oracle_task, [("warm", None)] * n)
        t0 = time.perf_counter()
        done = units = 0
        it = iter(tasks)
        pending = []
        while True:
            while len(pending) < 2 * n:
                try:
                    task, u = next(it)
                except StopIteration:
                    break
                pending.append((pool.apply_async(_oracle_task, (task,)), u))
            if not pending:
                break
            res, u = pending.pop(0)
            res.get()
            done += 1
            units += u
            if time.perf_counter() - t0 > budget_s and done >= n:
                break
        el = time.perf_counter() - t0
        pool.terminate()
    return {"value": units / el, "unit": f"{unit_per_task}/s", "cores": n, "kind": "oracle",
            "sample": f"{done} request rows ({units} {unit_per_task}) of the same workload in "
                      f"{el:.1f} s over {n} worker processes (one numpy thread each) on "
                      f"{cpu_model()} ({os.cpu_count()} logical CPUs visible)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="bytes of one plain device copy run before the warmup")
    ap.add_argument("--digest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--confidence", action="store_true",
                    help="time the draft-side confidence step (sd_draft_confidence) instead")
    ap.add_argument("--config", default="4", choices=["4", "4fb", "2", "3", "5", "5b", "lmhead"],
                    help="workload: 4 (default, the measured one), 4fb (T in [1, 1.5]: wide "
                         "nuclei, units the single-pass kernel settles by its exact route), "
                         "2, 3 (greedy), 5, 5b, lmhead (the fused LM-head path)")
    ap.add_argument("--cpu-cores", choices=["all", "one"], default="all",
                    help="cpu_baseline over a pool of worker processes (all) or one thread")
    a = ap.parse_args()
    if a.digest_pmc:
        if a.copy_probe <= 0:
            sys.exit("--digest-pmc needs --copy-probe BYTES (the size the counter runs used)")
        digest_pmc(a.digest_pmc[0], a.digest_pmc[1], a.copy_probe, TRAFFIC_FILE)
        return
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {a.gpus}): the verify step is "
              "data-parallel over requests and this build has no multi-GPU path; "
              "run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if a.confidence:
        confidence_bench(a)
        return
    if a.config in ("2", "3", "5", "5b", "lmhead"):
        {"2": bench_config2, "3": bench_config3, "5": bench_config5, "5b": bench_config5,
         "lmhead": bench_lmhead}[a.config](a)
        return

    import numpy as np
    import torch
    import speculative_sampling_verify_temp_amd as sdv
    import workloads as wl

    t0 = time.perf_counter()
    w = wl.config4(T_range=(1.0, 1.5)) if a.config == "4fb" else wl.config4()
    gen_s = time.perf_counter() - t0
    print(f"[bench] generated workload in {gen_s:.1f} s", file=sys.stderr, flush=True)
    cpu = None
    if not a.no_cpu_baseline:
        # before the GPU is touched: the worker processes start from a clean state
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = (cpu_baseline_all_cores(sample_tasks(w)) if a.cpu_cores == "all"
               else cpu_baseline(w))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = device_inputs(w, torch, dev)
    args = sdv.make_args(d["target"], d["draft"], d["draft_ids"], d["k_per_row"],
                         d["temperature"], w.top_p, w.rep_penalty, d["prior_ids"],
                         d["prior_offsets"], w.tv_budget, w.seed, w.offset, w.flags)
    ws = sdv.alloc_workspace(args, dev)
    acc = torch.empty(w.B, dtype=torch.int32, device=dev)
    tok = torch.empty((w.B, w.K_max + 1), dtype=torch.int32, device=dev)
    st = torch.empty(w.B, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    names = [sdv.phase_kernel(args, ph) for ph in range(3)]
    phases = [ph for ph in range(3) if names[ph] is not None]

    if a.copy_probe > 0:
        # A plain streaming kernel of known traffic (reads and writes
        # copy_probe bytes) for scaling the memory counters; a same-dtype
        # copy_ would go to a DMA engine and dispatch no kernel.
        src = torch.ones(a.copy_probe, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    def step(evs=None):
        for ph in phases:
            if evs is not None:
                evs[ph][0].record(stream)
            sdv.run_phase(args, ws, ph, acc, tok, st, None, stream)
            if evs is not None:
                evs[ph][1].record(stream)

    # W warmup steps, then more untimed steps while fewer than SETTLE_STEPS
    # have run: the clocks' ramp after an idle spell spans ~40 calls, and the
    # timed steps should see the sustained rate whatever W is (reported as
    # settle_steps).
    for _ in range(a.warmup):
        step()
    settle = max(0, SETTLE_STEPS - a.warmup)
    for _ in range(settle):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({a.warmup} steps + {settle} settle steps)", file=sys.stderr, flush=True)

    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    evs = [[[E(), E()] for _ in range(3)] for _ in range(a.steps)]
    start, end = E(), E()
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(a.steps):
        step(evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / a.steps
    phase_ms = {names[ph]: float(np.mean([evs[i][ph][0].elapsed_time(evs[i][ph][1])
                                          for i in range(a.steps)])) for ph in phases}
    status = st.cpu().numpy()
    assert (status & 0xF).sum() == 0, "invalid rows in the bench workload"

    positions = w.positions()
    logit_bytes = w.logit_bytes()
    dom = max(phase_ms, key=phase_ms.get)
    flagged = None
    if names[0] == "k_pair_fast":
        # units the single pass handed to its exact route (records of the last step)
        nfb, why = sdv.fallback_units(args, ws, stream, why=True)
        flagged = why != 0
    nbytes = algorithmic_bytes(dom, w)
    achieved = nbytes / (phase_ms[dom] * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": positions / (ms_step * 1e-3),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "settle_steps": settle,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": WORKLOAD,
                   "B": w.B, "K": w.K_max, "V": w.V, "input_dtype": "bf16",
                   "logit_bytes_per_call": logit_bytes},
        "call_hbm_gbps": logit_bytes / (ms_step * 1e-3) / 1e9,
        "phases_ms": phase_ms,
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": achieved,
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS,
                     "traffic": measured_traffic(dom),
                     "algorithmic_bytes": nbytes},
        "mean_accepted": float(acc.float().mean().item()),
    }
    if a.config == "4fb":
        line["config"]["workload"] = WORKLOAD.replace("T~U[0.5,1]", "T~U[1,1.5]")
    if flagged is not None:
        line["fallback_units"] = int(flagged.sum())
        line["units"] = w.B * (w.K_max + 1)
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


def confidence_bench(a):
    """The draft-side confidence step on the verify workload's draft rows
    (256 requests x 8 rows x V = 152064, bf16): one sd_draft_confidence call
    per step, every draft logit read once."""
    import numpy as np
    import torch
    import speculative_sampling_verify_temp_amd as sdv
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = wl.config4()
    d = device_inputs(w, torch, dev)
    draft, temp = d["draft"], d["temperature"]
    thr = 0.6   # the threshold of the page's run
    stream = torch.cuda.current_stream()
    for _ in range(a.warmup):
        sdv.draft_confidence(draft, temp, thr, stream)
    torch.cuda.synchronize()
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    start, end = E(), E()
    start.record(stream)
    for _ in range(a.steps):
        top1, kout = sdv.draft_confidence(draft, temp, thr, stream)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / a.steps
    # the row kernel alone (no draft-length launch), for its roofline
    k0, k1 = E(), E()
    k0.record(stream)
    for _ in range(a.steps):
        sdv.draft_confidence(draft, temp, thr, stream, lengths=False)
    k1.record(stream)
    torch.cuda.synchronize()
    ms_k = k0.elapsed_time(k1) / a.steps
    rows = w.B * w.K_max
    nbytes = rows * w.V * 2
    achieved = nbytes / (ms_k * 1e-3) / 1e9
    line = {
        "metric": "draft rows scored/sec (top-1 probability), V=152064 bf16",
        "value": rows / (ms * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "draft confidence: 256 requests x 8 draft rows, V=152064, bf16 logits, "
                               "T~U[0.5,1], threshold 0.6",
                   "B": w.B, "K": w.K_max, "V": w.V, "input_dtype": "bf16"},
        "roofline": {"kernel": "k_draft_confidence", "bound": "hbm", "achieved": achieved,
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS,
                     "traffic": None, "algorithmic_bytes": nbytes},
        "kernel_ms": ms_k,
        "mean_k": float(kout.float().mean().item()),
    }
    if not a.no_cpu_baseline:
        import oracle
        df = w.draft_f32()
        t0, n = time.perf_counter(), 0
        while n < rows and (n < 2 or time.perf_counter() - t0 < 10.0):
            r, j = divmod(n, w.K_max)
            oracle.top1_prob(df[r, j], float(w.temperature[r]))
            n += 1
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": n / dt, "unit": "rows/s", "cores": 1, "kind": "oracle",
                                "sample": f"the first {n} draft rows of the same workload in {dt:.1f} s, "
                                          "numpy fp64 on one thread"}
    print(json.dumps(line), flush=True)


# ---------------------------------------------------------------------------
# The other workloads.  Latency-bound ones (a single request) rotate over
# input copies totalling more than 1 GiB, so that no call finds its rows in
# the 256 MB last-level cache; those copies are generated on the device from
# a seeded torch generator with the workload's recipe.
# ---------------------------------------------------------------------------

def _line(metric, value, unit, a, ms, cfg, roof, extra=None, dtype="f32", hib=True):
    line = {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": a.steps,
            "warmup": a.warmup, "ms_per_step": ms, "higher_is_better": hib, "scaling": "weak",
            "vs_baseline": None, "dtype": dtype, "data": "synthetic", "config": cfg,
            "roofline": roof}
    line.update(extra or {})
    return line


def _hbm_roof(kernel, nbytes, ms):
    ach = nbytes / (ms * 1e-3) / 1e9
    return {"kernel": kernel, "bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": ach / PEAK_HBM_GBPS, "traffic": None, "algorithmic_bytes": nbytes}


def _gumbel_ids(torch, rows, T, g):
    """Draft proposals: Gumbel-max over rows / T (rows [..., V])."""
    u = torch.rand(rows.shape, generator=g, device=rows.device).clamp_(1e-20, 1.0)
    return torch.argmax(rows / T - torch.log(-torch.log(u)), dim=-1).to(torch.int32)


def _phase_loop(torch, sdv, argsets, ws, outs, steps, warmup, stream):
    """Run sd_verify_sample phase by phase over the argument sets in turn
    (each set with the phases it needs: a TV budget strictly between 0 and
    1 adds the TV pass); returns (ms per call, {kernel: ms per launch})."""
    import numpy as np
    acc, tok, st = outs
    names = [[sdv.phase_kernel(a_, ph) for ph in range(3)] for a_ in argsets]
    for i in range(warmup):
        for ph in range(3):
            if names[i % len(argsets)][ph] is not None:
                sdv.run_phase(argsets[i % len(argsets)], ws, ph, acc, tok, st, None, stream)
    torch.cuda.synchronize()
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    evs = [[[E(), E()] for _ in range(3)] for _ in range(steps)]
    s0, s1 = E(), E()
    s0.record(stream)
    for i in range(steps):
        for ph in range(3):
            if names[i % len(argsets)][ph] is None:
                continue
            evs[i][ph][0].record(stream)
            sdv.run_phase(argsets[i % len(argsets)], ws, ph, acc, tok, st, None, stream)
            evs[i][ph][1].record(stream)
    s1.record(stream)
    torch.cuda.synchronize()
    ms = s0.elapsed_time(s1) / steps
    times = {}
    for i in range(steps):
        for ph in range(3):
            nm = names[i % len(argsets)][ph]
            if nm is not None:
                times.setdefault(nm, []).append(evs[i][ph][0].elapsed_time(evs[i][ph][1]))
    per = {nm: float(np.mean(v)) for nm, v in times.items()}
    return ms, per


def bench_config2(a):
    """One request, K = 8, V = 152064, fp32, penalty 1.1 over 64 prior ids
    plus the draft prefix, T = 0.7, budgets cycling through 0, 0.5, 0.75, 1:
    one sd_verify_sample per step (the general path), latency."""
    import numpy as np
    import torch
    import speculative_sampling_verify_temp_amd as sdv
    import workloads as wl
    V, K, T = wl.V_QWEN25, 8, 0.7
    cpu = None
    if not a.no_cpu_baseline:
        ws_ = [wl.config2(call=c, D=D) for c in range(16) for D in (0.0, 0.5, 0.75, 1.0)]
        tasks = ((t, u) for w_ in ws_ for t, u in sample_tasks(w_))
        cpu = (cpu_baseline_all_cores(tasks) if a.cpu_cores == "all" else cpu_baseline(ws_[0]))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    per_copy = (2 * K + 1) * V * 4
    nc = max(4, -(-(1 << 30) // per_copy))
    g = torch.Generator(device=dev).manual_seed(2)
    tgt = torch.randn((nc, K + 1, V), generator=g, device=dev) * 3.0
    drf = 0.8 * tgt[:, :K] + 1.5 * torch.randn((nc, K, V), generator=g, device=dev)
    ids = _gumbel_ids(torch, drf, T, g)
    prior = torch.randint(0, V, (nc, 64), generator=g, device=dev, dtype=torch.int32)
    offs = torch.tensor([0, 64], dtype=torch.int32, device=dev)
    temp = torch.full((1,), T, device=dev)
    argsets = []
    for c in range(nc):
        D = (0.0, 0.5, 0.75, 1.0)[c % 4]
        argsets.append(sdv.make_args(tgt[c:c + 1], drf[c:c + 1], ids[c:c + 1], None, temp, 1.0, 1.1,
                                     prior[c], offs, D, c, 0, 0))
    ws = sdv.alloc_workspace(argsets[0], dev)
    outs = (torch.empty(1, dtype=torch.int32, device=dev), torch.empty((1, K + 1), dtype=torch.int32, device=dev),
            torch.empty(1, dtype=torch.int32, device=dev))
    ms, per = _phase_loop(torch, sdv, argsets, ws, outs, a.steps, a.warmup, torch.cuda.current_stream())
    dom = max(per, key=per.get)
    nbytes = per_copy if dom == "k_row_prepare" else 2 * K * V * 4 if dom == "k_pair_tv" else 2 * V * 4
    cfg = {"workload": "1 request x K=8, V=152064, fp32 logits, T=0.7, penalty 1.1 (64 prior ids + "
                       "draft prefix), TV budget cycling 0/0.5/0.75/1", "B": 1, "K": K, "V": V,
           "input_dtype": "f32", "input_copies": nc}
    line = _line(METRIC, K / (ms * 1e-3), "positions/s", a, ms, cfg, _hbm_roof(dom, nbytes, per[dom]),
                 {"phases_ms": per, "latency_us": ms * 1e3})
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


def bench_config3(a):
    """Greedy verify of one request, V = 151936 bf16, K in {1, 2, 4, 8}: one
    sd_verify_greedy per step, latency; value and roofline for K = 8."""
    import torch
    import speculative_sampling_verify_temp_amd as sdv
    import workloads as wl
    V = wl.V_QWEN3
    cpu = None
    if not a.no_cpu_baseline:
        ws_ = [wl.config3(K=8, call=c) for c in range(64)]

        def tasks():
            for w_ in ws_:
                yield ("greedy", (w_.target_f32(), w_.draft_ids, w_.k_per_row)), 8
        cpu = cpu_baseline_all_cores(tasks())
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    res = {}
    stream = torch.cuda.current_stream()
    for K in (1, 2, 4, 8):
        per_copy = (K + 1) * V * 2
        nc = max(4, -(-(1 << 30) // per_copy))
        g = torch.Generator(device=dev).manual_seed(3 + K)
        tgt = (torch.randn((nc, K + 1, V), generator=g, device=dev) * 3.0).to(torch.bfloat16)
        drf = 0.9 * tgt[:, :K].float() + (1 - 0.81) ** 0.5 * 3.0 * torch.randn((nc, K, V), generator=g, device=dev)
        ids = torch.argmax(drf.to(torch.bfloat16).float(), dim=-1).to(torch.int32)
        del drf
        argsets = [sdv.make_args(tgt[c:c + 1], None, ids[c:c + 1]) for c in range(nc)]
        ws = sdv.alloc_workspace(argsets[0], dev)
        acc = torch.empty(1, dtype=torch.int32, device=dev)
        tok = torch.empty((1, K + 1), dtype=torch.int32, device=dev)
        st = torch.empty(1, dtype=torch.int32, device=dev)
        import ctypes
        f = sdv.lib.sd_verify_greedy
        sp = sdv._stream(stream)
        ptrs = [ctypes.c_void_p(x.data_ptr()) for x in (ws, acc, tok, st)]

        def call(i):
            rc = f(ctypes.byref(argsets[i % nc]), ptrs[0], ws.numel(), ptrs[1], ptrs[2], ptrs[3], None, sp)
            assert rc == 0
        for i in range(a.warmup):
            call(i)
        torch.cuda.synchronize()
        E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
        s0, s1 = E(), E()
        s0.record(stream)
        for i in range(a.steps):
            call(i)
        s1.record(stream)
        torch.cuda.synchronize()
        res[K] = (s0.elapsed_time(s1) / a.steps, per_copy, nc)
        del tgt, ids, argsets, ws
        torch.cuda.empty_cache()
    ms, nbytes, nc = res[8]
    cfg = {"workload": "greedy verify, 1 request, V=151936, bf16 logits, draft correlation 0.9, "
                       "K=8 (value) and 1/2/4", "B": 1, "K": 8, "V": V, "input_dtype": "bf16",
           "input_copies": nc}
    line = _line(METRIC, 8 / (ms * 1e-3), "positions/s", a, ms, cfg,
                 _hbm_roof("sd_verify_greedy (k_greedy_partial + k_greedy_final)", nbytes, ms),
                 {"latency_us_by_K": {str(k): v[0] * 1e3 for k, v in res.items()}}, dtype="u32")
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


def bench_config5(a):
    """512 requests, V = 151936 bf16, lossless (D = 0), T = 0.7, no top-p
    (the general path); K_r from the early-stop rule (5) or uniform in 1..8
    (5b)."""
    import numpy as np
    import torch
    import speculative_sampling_verify_temp_amd as sdv
    import workloads as wl
    w = wl.config5(forced_ragged=a.config == "5b")
    cpu = None
    if not a.no_cpu_baseline:
        cpu = cpu_baseline_all_cores(sample_tasks(w)) if a.cpu_cores == "all" else cpu_baseline(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = device_inputs(w, torch, dev)
    args = sdv.make_args(d["target"], d["draft"], d["draft_ids"], d["k_per_row"], d["temperature"],
                         w.top_p, w.rep_penalty, None, None, w.tv_budget, w.seed, w.offset, w.flags)
    ws = sdv.alloc_workspace(args, dev)
    outs = (torch.empty(w.B, dtype=torch.int32, device=dev),
            torch.empty((w.B, w.K_max + 1), dtype=torch.int32, device=dev),
            torch.empty(w.B, dtype=torch.int32, device=dev))
    ms, per = _phase_loop(torch, sdv, [args], ws, outs, a.steps, a.warmup, torch.cuda.current_stream())
    dom = max(per, key=per.get)
    cfg = {"workload": ("512 requests, V=151936, bf16 logits, draft correlation U[0.3,0.95], T=0.7, "
                        "lossless, no top-p, " + ("K_r ~ U{1..8}" if a.config == "5b" else
                                                  "K_r from the early-stop rule (top-1 < 0.6)")),
           "B": w.B, "K_max": w.K_max, "V": w.V, "input_dtype": "bf16",
           "positions": w.positions(), "k_hist": np.bincount(w.k_per_row, minlength=9).tolist(),
           "logit_bytes_per_call": w.logit_bytes()}
    acc_np = outs[0].cpu().numpy()
    line = _line(METRIC, w.positions() / (ms * 1e-3), "positions/s", a, ms, cfg,
                 _hbm_roof(dom, algorithmic_bytes(dom, w, accepted=acc_np), per[dom]),
                 {"phases_ms": per, "call_hbm_gbps": w.logit_bytes() / (ms * 1e-3) / 1e9,
                  "row_pass_roofline": _hbm_roof("k_row_prepare", w.logit_bytes(),
                                                 per["k_row_prepare"])})
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


def bench_lmhead(a):
    """The fused LM-head path at the pages' model sizes: 64 requests x K = 8,
    target head 152064 x 3584, draft head 151936 x 896 (bf16, N(0, 9 / H)
    weights, N(0, 1) hidden states), T ~ U[0.6, 1], lossless (D = 0): one
    sd_lmhead_verify_sample per step; roofline against the dense bf16 MFMA
    peak from the GEMM flops the call must do (every used row against both
    heads, plus the draw's two rows per request)."""
    import torch
    import speculative_sampling_verify_temp_amd as sdv
    import workloads as wl
    B, K = 64, 8
    w = wl.lmhead_case(2100, B=B, K_max=K, V=wl.V_QWEN25, V_draft=wl.V_QWEN3,
                       H_t=wl.QWEN25_7B_HIDDEN, H_d=wl.QWEN25_05B_HIDDEN, D=0.0, exact=False,
                       T_range=(0.6, 1.0))
    cpu = None
    if not a.no_cpu_baseline:
        import oracle
        t0, n = time.perf_counter(), 0
        while n < B and (n < 1 or time.perf_counter() - t0 < 12.0):
            oracle.lmhead_verify_sample_ref(w.f32("target_hidden")[n:n + 1], w.f32("draft_hidden")[n:n + 1],
                                            w.f32("target_weight"), w.f32("draft_weight"),
                                            w.draft_ids[n:n + 1], w.k_per_row[n:n + 1],
                                            w.temperature[n:n + 1], 0.0)
            n += 1
        el = time.perf_counter() - t0
        cpu = {"value": n * K / el, "unit": "positions/s", "cores": os.cpu_count(), "kind": "oracle",
               "sample": f"{n} requests of the same workload in {el:.1f} s (numpy fp64 matmul on its "
                         f"BLAS threads, then the verify oracle) on {cpu_model()}"}
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def bf(x):
        return torch.from_numpy(x.view(__import__("numpy").int16)).to(dev).view(torch.bfloat16)
    th, dh, wt, wd = bf(w.target_hidden), bf(w.draft_hidden), bf(w.target_weight), bf(w.draft_weight)
    ids = torch.from_numpy(w.draft_ids).to(dev)
    T = torch.from_numpy(w.temperature).to(dev)
    args = sdv.make_lmhead_args(th, wt, ids, dh, wd, None, T, 0.0, 7, 0, 0)
    ws = sdv.lmhead_workspace(args, dev)
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    tok = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    st = torch.empty(B, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(a.warmup):
        sdv.lmhead_verify_sample(args, acc, tok, st, None, ws, stream)
    torch.cuda.synchronize()
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    s0, s1 = E(), E()
    s0.record(stream)
    for _ in range(a.steps):
        sdv.lmhead_verify_sample(args, acc, tok, st, None, ws, stream)
    s1.record(stream)
    torch.cuda.synchronize()
    ms = s0.elapsed_time(s1) / a.steps
    Ht, Hd, V, Vd = w.target_hidden.shape[2], w.draft_hidden.shape[2], w.V, w.V_draft
    flops = 2.0 * (B * (K + 1) * V * Ht + B * K * Vd * Hd + B * (V * Ht + Vd * Hd))
    ach = flops / (ms * 1e-3) / 1e12
    cfg = {"workload": "fused LM head + verify: 64 requests x K=8, target head 152064 x 3584, draft "
                       "head 151936 x 896, bf16, lossless, no top-p", "B": B, "K": K, "V": V,
           "V_draft": Vd, "H_target": Ht, "H_draft": Hd, "input_dtype": "bf16"}
    roof = {"kernel": "sd_lmhead_verify_sample (whole call)", "bound": "mfma", "achieved": ach,
            "peak": 2500.0, "unit": "TFLOP/s", "frac": ach / 2500.0, "traffic": None,
            "algorithmic_flops": flops}
    line = _line("verified draft positions/sec from hidden states (fused LM head + verify)",
                 B * K / (ms * 1e-3), "positions/s", a, ms, cfg, roof,
                 {"mean_accepted": float(acc.float().mean().item())}, dtype="bf16")
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
