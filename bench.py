"""Benchmark of the decode-step sampler on one MI355X.

Workload: the full sampler chain at N=64 rows, V=128,000, fp32 logits --
penalties over 2,048-id histories, temperature, top-k/top-p/min-p on mixed
rows (filtered path), fp32 probs and logprobs materialised, tokens by
Gumbel-max / argmax.  Inputs are seeded synthetic Zipf-biased Gaussian
logits (workloads.py); six buffer sets (593 MB) rotate so every step reads
its logits from HBM rather than the 256 MB Infinity Cache.

A step is one sampler_step call: one kernel launch, with the per-row
records carried in its arguments.  W warm-up steps, then K timed steps between two
device synchronisations (value, ms_per_step).  Then K more steps with the
library's per-launch event pair (hipExtLaunchKernel's start and stop events,
which bracket the kernel itself) give the kernel duration behind the
roofline figures; the events are kept out of the timed steps because they
add a dependency per launch.

Prints one JSON line.  --gpus N > 1 is refused: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sampled rows/sec and achieved HBM GB/s (% peak) at N=64, V=128,000 filtered path"
HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published
N_SETS = 6
# name -> (generator index in workloads.config, temperature override, buffer
# sets: enough that one pass over them exceeds the 256 MB Infinity Cache
# twice; the small Gumbel-only workload is latency-bound and fits anyway,
# description, ablation stage of the full chain or None)
WORKLOADS = {
    "gumbel-small": (1, None, 1, "Gumbel only N=4 V=1024 fp32, ids + probs", None),
    "batch1": (2, None, 16, "batch-1 decode N=1 V=151936 bf16 T=1 (Gumbel), ids", None),
    "batch1-greedy": (2, 0.0, 16, "batch-1 decode N=1 V=151936 bf16 T=0 (greedy), ids", None),
    "mixed": (3, None, 11, "mixed filtered N=32 V=151936 bf16, one greedy row, probs+logprobs", None),
    "full-chain": (4, None, N_SETS, "full sampler chain N=64 V=128000 fp32, filtered path, probs+logprobs", None),
    "large-vocab": (5, None, 2, "large vocab N=512 (128 x 4 forks) V=256000 bf16, top-20 logprobs", None),
    # the per-feature ablation of the full chain: same logits, temperatures,
    # outputs and RNG keys, features added one at a time (the last stage is
    # full-chain itself)
    "ablation-defaults": (4, None, N_SETS, "full-chain ablation N=64 V=128000 fp32: temperature only, "
                          "probs+logprobs", "defaults"),
    "ablation-penalties": (4, None, N_SETS, "full-chain ablation N=64 V=128000 fp32: + penalties, "
                           "probs+logprobs", "penalties"),
    "ablation-min_p": (4, None, N_SETS, "full-chain ablation N=64 V=128000 fp32: + penalties + min_p, "
                       "probs+logprobs", "min_p"),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--workload", default="full-chain", choices=sorted(WORKLOADS),
                    help="full-chain (default): N=64, V=128,000 with every option; the others time the "
                         "remaining synthetic workloads and the full chain's per-feature ablation "
                         "(no CPU baseline)")
    ap.add_argument("--phase-stamps", action="store_true",
                    help="load the library built with the stamps option (decode_step_token_sampler_amd/build.py "
                         "--stamps), run the workload's warm-up and --steps steps one at a time, and print the "
                         "row kernel's phase timeline (first row of each workgroup) as one JSON line")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write the row kernel's HBM traffic per launch (the counter_collection.csv files of "
                         "rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs of this benchmark and of --calibrate-copy) to "
                         + os.path.relpath(os.path.join("profiles", "row_kernel_N64_V128000_traffic.json")) + " and exit")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 256 MiB device copy 10 times (the reference kernel for scaling "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


COPY_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "row_kernel_N64_V128000_traffic.json")
KERNEL_SOURCES = ("decode_step_token_sampler_amd/csrc/sampler_kernel.hip",
                  "decode_step_token_sampler_amd/csrc/sampler_internal.h")


def kernel_digest():
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch from the committed counter runs, or None when the
    kernel sources changed since they were taken (or none were taken)."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha256") != kernel_digest():
        return None
    return t.get("traffic_bytes")


def _counter_means(path, kernel_pred):
    """Mean Counter_Value over the dispatches of the kernels kernel_pred
    accepts in a rocprofv3 counter_collection.csv, and their count."""
    import csv
    vals = []
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if kernel_pred(row["Kernel_Name"]):
                vals.append(float(row["Counter_Value"]))
    if not vals:
        raise SystemExit(f"{path}: no dispatch of the kernel")
    return float(np.mean(vals)), len(vals)


def traffic_summary(fetch_csv, write_csv, cfetch_csv, cwrite_csv):
    """HBM bytes per launch of the row kernel: each counter (KiB per
    dispatch) scaled by what the same counter reads for a plain copy of
    COPY_BYTES (read COPY_BYTES, write COPY_BYTES)."""
    import workloads
    row_k = lambda name: "row_kernel" in name
    copy_k = lambda name: "copyBuffer" in name  # the runtime's device-to-device copy kernel
    fetch, n_f = _counter_means(fetch_csv, row_k)
    write, n_w = _counter_means(write_csv, row_k)
    cfetch, _ = _counter_means(cfetch_csv, copy_k)
    cwrite, _ = _counter_means(cwrite_csv, copy_k)
    f_scale = COPY_BYTES / 1024.0 / cfetch
    w_scale = COPY_BYTES / 1024.0 / cwrite
    traffic = int(round((fetch * f_scale + write * w_scale) * 1024.0))
    out = {"kernel": "row_kernel<float, true>", "workload": "N=64 V=128000 fp32 full chain (bench.py default)",
           "fetch_kib_per_launch": round(fetch, 1), "write_kib_per_launch": round(write, 1),
           "copy_bytes": COPY_BYTES, "copy_fetch_kib": round(cfetch, 1), "copy_write_kib": round(cwrite, 1),
           "fetch_factor": round(f_scale, 4), "write_factor": round(w_scale, 4), "traffic_bytes": traffic,
           "algorithmic_bytes": workloads.config(4).algorithmic_bytes(), "launches_counted": min(n_f, n_w),
           "kernel_sha256": kernel_digest()}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def calibrate_copy():
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 10}))


def host_cpu():
    """The host's CPU model and logical core count."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "logical_cores": os.cpu_count()}


def stream_rates(dev, nbytes=COPY_BYTES, reps=10):
    """Plain device streams in the same run, as context for the roofline:
    a copy (read + write), a read-only reduction and a write-only fill of
    nbytes each, GB/s of bytes moved (best of reps)."""
    import torch
    a = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    out = {}
    for name, fn, moved in (("copy", lambda: b.copy_(a), 2 * nbytes), ("read", lambda: a.sum(), nbytes),
                            ("write", lambda: b.fill_(0.5), nbytes)):
        fn()
        best = None
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        out[name + "_gbs"] = moved / (best * 1e-3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    out["bytes"] = nbytes
    return out


def batch_record(b):
    """The batch fields of the xbrilliance.ai note's cost record ("记录字段"):
    its batch switches, whether rows mix parameters, and the bytes of the two
    fp32 [N, V] outputs (8 N V)."""
    n, V = b.n_rows, b.vocab
    k = np.asarray(b.top_k)
    pen = [x for x in (b.repetition_penalty, b.presence_penalty, b.frequency_penalty) if x is not None]
    params = np.stack([np.asarray(b.temperature, np.float64), np.asarray(b.top_p, np.float64), k.astype(np.float64),
                       np.asarray(b.min_p, np.float64)] + [np.asarray(x, np.float64) for x in pen], axis=1)
    return {
        "num_seqs": n, "vocab_size": V,
        "do_top_p_top_k": bool(np.any(np.asarray(b.top_p) < 1.0) or np.any(k != -1)),
        "do_min_p": bool(np.any(np.asarray(b.min_p) > 0.0)),
        "do_penalties": bool((b.repetition_penalty is not None and np.any(b.repetition_penalty != 1.0))
                             or (b.presence_penalty is not None and np.any(b.presence_penalty != 0.0))
                             or (b.frequency_penalty is not None and np.any(b.frequency_penalty != 0.0))),
        "param_mixed": bool(np.any(params != params[0])),
        "sampling_tensor_bytes": 8 * n * V,
    }


def parity_summary(b, offset, gpu_out):
    """One timed step's GPU outputs against the oracle on its inputs, under
    the parity rules of tests/parity.py (part of the CPU-baseline leg)."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity import compare, run_oracle
    import dataclasses
    b = dataclasses.replace(b, seed=0, offset=offset)
    g = {k: v.cpu().numpy() for k, v in gpu_out.items()}
    r = compare(g, run_oracle(b, n_threads=min(os.cpu_count() or 1, 16)))
    return {"step_offset": offset, "rows": r.rows, "ok": r.ok(), "token_mismatches": len(r.token_mismatch),
            "flagged_rows": r.flagged, "flagged_by_class": r.flagged_by_class,
            "flagged_rows_failed": len(r.flagged_failed), "max_prob_err": r.max_prob_err,
            "max_logprob_err": r.max_logprob_err, "max_logprob_ulps": r.max_logprob_ulps}


def cpu_baseline(batches, budget_s, threads=None):
    """The oracle, as it stands, on whole steps of the same workload (one
    thread per host core, at most 16 -- the host CPU share of one GPU --
    unless threads is given)."""
    import oracle
    if threads is None:
        threads = min(os.cpu_count() or 1, 16)
    rows = 0
    steps = 0
    t0 = time.perf_counter()
    while True:
        b = batches[steps % len(batches)]
        oracle.step(b.logits, dtype=b.dtype, temperature=b.temperature, top_p=b.top_p, top_k=b.top_k,
                    min_p=b.min_p, repetition_penalty=b.repetition_penalty, presence_penalty=b.presence_penalty,
                    frequency_penalty=b.frequency_penalty, history_ids=b.history_ids,
                    history_start=b.history_start, history_len=b.history_len, seed=b.seed, offset=b.offset,
                    want_probs=True, want_logprobs=True, n_threads=threads)
        rows += b.n_rows
        steps += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s:
            break
    return {"value": rows / dt, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": f"{steps} whole steps of the N=64, V=128,000 full-chain workload "
                      f"({rows} rows, {dt:.1f} s, probs and logprobs materialised)",
            "host": dict(host_cpu(), thread_cap=16)}


PHASES = ("start", "row", "loaded", "max", "hist", "x2", "decided", "gathered", "x3", "thresholds", "select",
          "token", "end", "gumbel", "released", "arrived", "g_bound", "g_listed", "listed_n", "row_index",
          "g_batched", "g_rounds", "table", "x3_read", "x3_ranked", "x3_decided",
          "half", "hashed", "transformed")
NOT_TIMES = ("listed_n", "row_index", "g_rounds")


ROW_INDEX_SLOT = 19  # PHASES[19]
ROW_SLOTS = tuple((name, k) for k, name in enumerate(PHASES))
# the streaming kernel's stamps: its own start slot, the rest in slots of
# the row kernel's list
STREAM_SLOTS = (("start", 29), ("row", 1), ("hashed", 27), ("pass_a", 3), ("pass_b", 4), ("ranges", 6),
                ("pass_c", 7), ("sorted", 24), ("decided", 9), ("end", 12), ("row_index", 19))


def row_class(b, r):
    """The cost class of row r of batch b, as the phase table groups rows."""
    t = float(b.temperature[r])
    if 0.0 <= t < 1e-6:
        return "greedy"
    k = int(b.top_k[r])
    topk = k != -1 and k < b.vocab
    topp = float(b.top_p[r]) < 1.0
    minp = float(b.min_p[r]) > 0.0
    if k == 1:
        return "top-1"
    if not (topk or topp or minp):
        return "keep-all"
    return "+".join(n for n, on in (("top-k", topk), ("top-p", topp), ("min-p", minp)) if on)


def phase_by_class(stamps_runs, khz, slots=ROW_SLOTS):
    """Per row class: the median over steps and workgroups of the time since
    the kernel's first stamp at which the workgroups' rows pass each phase
    (us), the largest end time, and the number of distinct rows seen.
    stamps_runs: (stamps, batch) of each step; slots: (phase, slot) pairs,
    the kernel's start first."""
    acc = {}
    s0 = slots[0][1]
    for st, b in stamps_runs:
        used = st[:, s0] != 0
        if not used.any():
            continue
        t0 = float(st[used, s0].min())
        for blk in np.flatnonzero(used):
            r = int(st[blk, ROW_INDEX_SLOT]) - 1
            if r < 0:
                continue
            c = acc.setdefault(row_class(b, r), {"rows": set(), "phases": {}})
            c["rows"].add(r)
            for name, k in slots:
                if st[blk, k] and name != "row_index":
                    v = float(st[blk, k]) if name in NOT_TIMES else (float(st[blk, k]) - t0) * 1e3 / khz
                    c["phases"].setdefault(name, []).append(v)
    out = {}
    for cls, v in sorted(acc.items()):
        ph = v["phases"]
        out[cls] = {"rows": len(v["rows"]),
                    "select_us": float(np.median(ph["select"])) if "select" in ph else None,
                    "end_us": float(np.median(ph["end"])) if "end" in ph else None,
                    "end_max_us": float(np.max(ph["end"])) if "end" in ph else None,
                    "phases_median_us": {name: float(np.median(ph[name])) for name, _ in slots if name in ph}}
    return out


def phase_timeline(stamps_runs, khz, slots=ROW_SLOTS):
    """Per phase: the median over steps of the median and the maximum over
    workgroups of the time since the kernel's first stamp (us), and the
    number of workgroups that passed it.  A phase a row skipped has no
    stamp.  slots: (phase, slot) pairs, the kernel's start first."""
    per = {name: {"median_us": [], "max_us": [], "workgroups": 0} for name, _ in slots}
    s0 = slots[0][1]
    for st, _ in stamps_runs:
        used = st[:, s0] != 0
        if not used.any():
            continue
        t0 = st[used, s0].min()
        for name, k in slots:
            col = st[used, k]
            col = col[col != 0]
            if col.size == 0 or name in NOT_TIMES:
                continue
            us = (col.astype(np.float64) - float(t0)) * 1e3 / khz
            per[name]["median_us"].append(float(np.median(us)))
            per[name]["max_us"].append(float(us.max()))
            per[name]["workgroups"] = int(col.size)
    return {name: {"median_us": float(np.median(v["median_us"])), "max_us": float(np.median(v["max_us"])),
                   "workgroups": v["workgroups"]} for name, v in per.items() if v["median_us"]}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    import torch
    import decode_step_token_sampler_amd as dsts
    import workloads

    dev = torch.device("cuda:0")
    wl = args.workload
    cfg, temp, n_sets, desc, stage = WORKLOADS[wl]
    headline = wl == "full-chain"
    batches = [workloads.config(cfg, set_id=s, step=s, temperature=temp) for s in range(n_sets)]
    if stage is not None:
        batches = [b.ablation(stage) for b in batches]
    b0 = batches[0]
    n, V = b0.n_rows, b0.vocab
    K = b0.top_logprobs
    sets = []
    for b in batches:
        if b.dtype == "bf16":
            L = torch.from_numpy(b.logits.view(np.int16)).view(torch.bfloat16).to(dev)
        else:
            L = torch.from_numpy(b.logits).to(dev)
        out = dict(token_ids=torch.empty(n, dtype=torch.int32, device=dev),
                   row_status=torch.empty(n, dtype=torch.int32, device=dev))
        if b.want_probs:
            out["probs"] = torch.empty(n, V, dtype=torch.float32, device=dev)
        if b.want_logprobs:
            out["logprobs"] = torch.empty(n, V, dtype=torch.float32, device=dev)
        if K:
            out["top_logprob_vals"] = torch.empty(n, K, dtype=torch.float32, device=dev)
            out["top_logprob_ids"] = torch.empty(n, K, dtype=torch.int32, device=dev)
        sets.append(dict(logits=L, out=out,
                         hist=None if b.history_ids is None else torch.from_numpy(b.history_ids).to(dev)))
    torch.cuda.synchronize()
    if args.phase_stamps:
        from decode_step_token_sampler_amd import build as libbuild
        dsts.load_library(libbuild.LIB_STAMPS)
    S = dsts.Sampler(n, V, max_history_per_row=2048, max_top_logprobs=K)

    def step(i):
        b, t = batches[i % n_sets], sets[i % n_sets]
        return S.step(t["logits"], temperature=b.temperature, top_p=b.top_p, top_k=b.top_k, min_p=b.min_p,
                      repetition_penalty=b.repetition_penalty, presence_penalty=b.presence_penalty,
                      frequency_penalty=b.frequency_penalty, history_ids=t["hist"], history_start=b.history_start,
                      history_len=b.history_len, row_stream=b.row_stream, seed=0, offset=i,
                      want_probs=b.want_probs, want_logprobs=b.want_logprobs, top_logprobs=K, out=t["out"])

    if args.phase_stamps:
        runs, khz = [], 0
        for i in range(args.warmup + args.steps):
            r = step(i)
            torch.cuda.synchronize()
            st, khz = dsts.phase_stamps()
            if i >= args.warmup:
                runs.append((st, batches[i % n_sets]))
        slots = STREAM_SLOTS if r["kernel"] == "stream" else ROW_SLOTS
        print(json.dumps({"workload": desc, "path": r["path"], "kernel": r["kernel"] + "_kernel", "steps": args.steps, "clock_khz": khz,
                          "phases_us_since_kernel_start": phase_timeline(runs, khz, slots),
                          "by_row_class": phase_by_class(runs, khz, slots)}), flush=True)
        S.close()
        return
    for i in range(args.warmup):
        r = step(i)
    if headline:
        assert r["path"] == "filtered"
    # the timed steps (no profiling events: they add a dependency per launch)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # then the same number of steps again, each kernel bracketed by the event
    # pair of hipExtLaunchKernel, for the per-launch kernel duration
    S.profile_start(args.steps)
    for i in range(args.steps):
        step(args.warmup + args.steps + i)
    torch.cuda.synchronize()
    kernel_ms = S.profile_stop()
    status = np.concatenate([s["out"]["row_status"].cpu().numpy() for s in sets])
    if np.any(status != 0):
        print(json.dumps({"error": "row status %s" % np.unique(status).tolist()}))
        sys.exit(1)

    # host-only cost of one call on an idle device (the call itself, no sync
    # inside the timed span), as a separate short column
    host_us = []
    for i in range(50):
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        step(i)
        host_us.append((time.perf_counter() - t1) * 1e6)
    torch.cuda.synchronize()
    # synchronised cost of one step (the call and its kernel, device idle before)
    sync_us = []
    for i in range(50):
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        step(i)
        torch.cuda.synchronize()
        sync_us.append((time.perf_counter() - t1) * 1e6)

    # the last step that wrote set 0's outputs (for the parity summary)
    parity_offset = max(i for i in range(50) if i % n_sets == 0)
    streams = stream_rates(dev)
    ms_per_step = wall * 1e3 / args.steps
    rows_per_s = n * args.steps / wall
    alg_bytes = b0.algorithmic_bytes()
    k_avg_ms = float(np.mean(kernel_ms))
    achieved = alg_bytes / (k_avg_ms * 1e-3) / 1e9
    line = {
        "metric": METRIC if headline else "sampled rows/sec and achieved HBM GB/s (%% peak), %s" % desc,
        "value": rows_per_s,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": b0.dtype,
        "data": "synthetic (seeded Zipf-biased Gaussian logits%s; %d rotating sets: %d MB of logits, %d MB "
                "with their outputs)" % (
            ", Zipf(1.1) histories" if b0.history_ids is not None else "", n_sets,
            sum(int(t["logits"].numel() * t["logits"].element_size()) for t in sets) // 10**6,
            sum(int(v.numel() * v.element_size()) for t in sets for v in [t["logits"]] + list(t["out"].values()))
            // 10**6),
        "config": {"workload": desc, "n_rows": n, "vocab": V,
                   "history_per_row": 2048 if b0.history_ids is not None else 0, "path": r["path"],
                   "kernel": r["kernel"] + "_kernel",
                   "algorithmic_bytes_per_step": alg_bytes},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic() if headline else None},
        "kernel_us": {"mean": k_avg_ms * 1e3, "median": float(np.median(kernel_ms)) * 1e3,
                      "p10": float(np.percentile(kernel_ms, 10)) * 1e3,
                      "p90": float(np.percentile(kernel_ms, 90)) * 1e3},
        "step_gbs": alg_bytes / (ms_per_step * 1e-3) / 1e9,
        "host_call_us_median": float(np.median(host_us)),
        "host_call_us_iqr": [float(np.percentile(host_us, 25)), float(np.percentile(host_us, 75))],
        "sync_step_us_median": float(np.median(sync_us)),
        "sync_step_us_iqr": [float(np.percentile(sync_us, 25)), float(np.percentile(sync_us, 75))],
        "stream_gbs": streams,
        "record": batch_record(b0),
    }
    if stage is not None:
        line["config"]["ablation_stage"] = stage
    if not args.no_cpu_baseline and headline:
        line["parity"] = parity_summary(batches[0], parity_offset, sets[0]["out"])
        line["cpu_baseline"] = cpu_baseline(batches, args.cpu_seconds)
        # the same oracle on one host thread (rows are independent, so this
        # is the per-core rate)
        line["cpu_baseline_1thread"] = cpu_baseline(batches, args.cpu_seconds / 3, threads=1)
    print(json.dumps(line), flush=True)
    S.close()


if __name__ == "__main__":
    main()
