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
sustained rate.

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
VERIFY_SOURCES = ("sd_verify.hip", "sdv_device.h", "sdv_exact.h")


def source_hash():
    """sha256 over the verify kernels' sources, in name order."""
    h = hashlib.sha256()
    for n in sorted(VERIFY_SOURCES):
        h.update(n.encode())
        h.update(open(os.path.join(CSRC, n), "rb").read())
    return h.hexdigest()


def algorithmic_bytes(kernel, w):
    """Bytes the kernel must move per launch by definition of its work.

    The single-pass kernel and the general row pass read every logit row of
    the call once; the general TV pass reads the 2K draft-position rows of
    each request; the fallback re-read, finalize and draw kernels read no
    logit row unconditionally.
    """
    if kernel in ("k_pair_fast", "k_row_prepare"):
        return w.logit_bytes()
    if kernel == "k_pair_tv":
        return 2 * w.K_max * w.V * 2 * w.B
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
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(dev)

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

    import numpy as np
    import torch
    import speculative_sampling_verify_temp_amd as sdv
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.perf_counter()
    w = wl.config4()
    gen_s = time.perf_counter() - t0
    print(f"[bench] generated workload in {gen_s:.1f} s", file=sys.stderr, flush=True)
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

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({a.warmup} steps)", file=sys.stderr, flush=True)

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
    achieved = algorithmic_bytes(dom, w) / (phase_ms[dom] * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": positions / (ms_step * 1e-3),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
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
                     "algorithmic_bytes": algorithmic_bytes(dom, w)},
        "mean_accepted": float(acc.float().mean().item()),
    }
    if not a.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w)
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


if __name__ == "__main__":
    main()
