#!/usr/bin/env python3
"""Benchmark of batched lossless draft verification on one MI355X.

A step is one svd_select_and_verify call over one batch of synthetic logits
already resident in HBM: row statistics and alpha for every scored row pair,
streak scores and self-selection, the first rejection, and the fp64 residual or
bonus draw.  Prints one JSON line.

Default workload: batched serving (B = 256 prefixes, K = 1, gamma = 8,
V = 152064, bf16 logits, T = 0.7), the workload that measures sustained HBM
bandwidth.  --workload picks another one.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, 8 TB/s
SETTLE_MS = 100.0  # GPU time of untimed warm-up before the timed steps (the clock settles)
METRIC = "verified draft positions/sec and achieved HBM GB/s (V=152064, bf16 logits)"
# sources whose text decides each kernel's memory traffic
KERNEL_SOURCES = {"rowstats": ["svd_device.hpp", "kr_rowstats.hpp"],
                  "rowstats_split": ["svd_device.hpp", "kr_rowstats.hpp"],
                  "rowstats_live": ["svd_device.hpp", "kr_rowstats.hpp"],
                  "pool_stats": ["svd_device.hpp", "kr_rowstats.hpp", "kr_rows.hpp"],
                  "lattice": ["svd_device.hpp", "kr_rowstats.hpp", "kr_cps.hpp"]}
KERNEL_SYMBOL = {"rowstats": "kr_rowstats", "rowstats_split": "kr_rowstats_split",
                 "rowstats_live": "kr_rowstats_live",
                 "pool_stats": "kr_pool_stats",
                 "lattice": "kr_lattice"}


def settle(torch, stream, step, warmup, settle_ms):
    """Untimed warm-up, in the open: at least `warmup` steps, continued until at
    least `settle_ms` of GPU time has passed since the first one, so that the
    timed steps run on a settled clock.  Returns the GPU time and steps spent."""
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    n = 0
    for _ in range(warmup):
        step()
        n += 1
    while True:
        ev1.record(stream)
        ev1.synchronize()
        elapsed = ev0.elapsed_time(ev1)
        if elapsed >= settle_ms or n >= 1_000_000:
            return {"settle_ms": elapsed, "steps": n}
        for _ in range(16):
            step()
            n += 1


def run_env(torch, **seeds) -> dict:
    """What reproduces a line: the device, the software and the seeds."""
    prop = torch.cuda.get_device_properties(0)
    return dict({"gpu": torch.cuda.get_device_name(0), "arch": getattr(prop, "gcnArchName", None),
                 "compute_units": prop.multi_processor_count, "torch": torch.__version__,
                 "hip": getattr(torch.version, "hip", None)}, **seeds)


def time_adl(torch, svd, stream, drafts, sel, L, B, K, G, calls=200):
    """svd_adl_next on a windowed call's inputs and outputs: microseconds per
    call over `calls` calls back to back on the call's stream (after 20 untimed)."""
    dev = drafts.device
    avg = torch.full((B, 2), 256 * G, dtype=torch.int32, device=dev)
    nxt = torch.empty(B, dtype=torch.int32, device=dev)

    def call():
        rc = svd.svd_adl_next(drafts, sel, L, None, -1, B, K, G, 1, G, 4, 2, 64, avg, nxt,
                              stream.cuda_stream)
        if rc != svd.SVD_OK:
            raise svd.SvdError(rc, "svd_adl_next")

    for _ in range(20):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(calls):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    return {"kernel": "kr_adl", "us_per_call": e0.elapsed_time(e1) * 1e3 / calls,
            "calls": calls, "prefixes": B}


def kernel_samples(steps: int) -> int:
    """Steps whose dominant-kernel launches are timed: at least 5, whatever --steps is."""
    return max(5, min(steps, 20))


def time_kernels(torch, tl, fn, kernels, n, warm=3):
    """(ms per kernel, launches per kernel) over n calls of fn, with the timing
    build recording HIP events around the launches of `kernels`.  The first
    `warm` calls go untimed: a kernel's first launch from a library loads its
    code object."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    tl.svd_profile_read()  # clear
    tl.svd_profile_enable(kernels)
    for _ in range(n):
        fn()
    tl.svd_profile_enable(())
    torch.cuda.synchronize()
    return tl.svd_profile_read()


def traffic_file(kernel: str, mode: str = "standard") -> str:
    tag = "" if mode == "standard" else "_" + mode
    return os.path.join(ROOT, "profiles", "%s%s_traffic.json" % (KERNEL_SYMBOL[kernel], tag))


def kernel_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "lossless_draft_verification_verifier_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str, mode: str = "standard"):
    """HBM bytes per launch of a kernel from committed rocprofv3 counter
    summaries, or None when they are missing or the kernel changed since."""
    try:
        with open(traffic_file(kernel, mode)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_hash") != kernel_hash(kernel) or rec.get("workload") != workload:
        return None
    return rec.get("hbm_bytes_per_launch")


def _counter_per_dispatch(run_dir: str, counter: str, name_part: str):
    """Mean over dispatches of one rocprofv3 counter (summed over its
    instances) for the kernels whose name contains name_part."""
    import csv
    import glob
    per = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if row["Counter_Name"] != counter or name_part not in row["Kernel_Name"]:
                    continue
                key = (f, row["Dispatch_Id"])
                per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    if not per:
        raise SystemExit("no %s samples for %s under %s" % (counter, name_part, run_dir))
    return sum(per.values()) / len(per), len(per)


def record_traffic(kernel, workload, mode, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir):
    """Write profiles/<kernel>_traffic.json from four rocprofv3 --pmc runs: FETCH_SIZE
    and WRITE_SIZE of the kernel, and of a plain 1 GiB copy that scales them."""
    sym = KERNEL_SYMBOL[kernel]
    fetch, nf = _counter_per_dispatch(fetch_dir, "FETCH_SIZE", sym + "<")
    write, nw = _counter_per_dispatch(write_dir, "WRITE_SIZE", sym + "<")
    cfetch, _ = _counter_per_dispatch(copy_fetch_dir, "FETCH_SIZE", "copyBuffer")
    cwrite, _ = _counter_per_dispatch(copy_write_dir, "WRITE_SIZE", "copyBuffer")
    copy_kib = COPY_BYTES / 1024.0
    fscale, wscale = cfetch / copy_kib, cwrite / copy_kib
    hbm = (fetch / fscale + write / wscale) * 1024.0
    import workloads as W
    cfg = W.get_config(workload.replace("cps_", "", 1))
    es = 2 if cfg.dtype == "bf16" else 4
    if kernel == "lattice":  # one drafter row per (prefix, position), read once
        alg = cfg.B * cfg.gamma * (cfg.V * es + CPS_MMAX * 8 + 8)
    elif cfg.layout == "pooled":
        rows = pool_rows_read(W.generate_pooled(cfg), mode)
        alg = rows * (cfg.V * es + POOL_STAT_BYTES)
    else:
        alg = bytes_per_row_pair(cfg.V, es, mode) * cfg.B * cfg.K * cfg.gamma
    rec = {"kernel": sym, "workload": workload, "mode": mode, "kernel_hash": kernel_hash(kernel),
           "fetch_kib_per_dispatch": fetch, "write_kib_per_dispatch": write,
           "dispatches": [nf, nw], "copy_fetch_kib": cfetch, "copy_write_kib": cwrite,
           "copy_bytes_each_way": COPY_BYTES, "fetch_scale": fscale, "write_scale": wscale,
           "hbm_bytes_per_launch": hbm, "algorithmic_bytes_per_launch": alg,
           "traffic_over_algorithmic": hbm / alg}
    with open(traffic_file(kernel, mode), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


POOL_STAT_BYTES = 8  # (max, sum) written per pool row


def pool_rows_read(d, mode: str) -> int:
    """Distinct pool rows that scored positions read (the rows kr_pool_stats streams)."""
    import numpy as np
    G = d["drafts"].shape[-1]
    n = len(np.unique(d["p_index"][:, :, :G].cpu().numpy()))
    if mode != "greedy":
        n += len(np.unique(d["q_index"].cpu().numpy()))
    return n


def bytes_per_row_pair(V: int, es: int, mode: str = "standard") -> int:
    """Algorithmic bytes of one scored position: its logit rows (p and q; p
    alone under greedy acceptance), the drafted token, and the 16-byte
    statistics record plus the 4-byte alpha written for it.  (Bonus rows and
    the 12 output bytes per prefix are left out, so the figure is a lower
    bound.)"""
    rows = 1 if mode == "greedy" else 2
    return rows * V * es + 4 + 16 + 4


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads() -> int:
    """Threads for the oracle: the CPUs this process may run on, at most 16 (one
    GPU's share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _oracle_run(d, cfg, seed, mode, pooled, want_beta, threads, nprefix=None):
    """One untuned oracle pass over the batch (or its first nprefix prefixes)."""
    import oracle
    import workloads as W
    cut = (lambda t: t[:nprefix]) if nprefix else (lambda t: t)
    if pooled:
        hp, hq = W.to_host(d["p_pool"]), W.to_host(d["q_pool"])
        pi, qi = W.to_host(cut(d["p_index"])), W.to_host(cut(d["q_index"]))
        hd = W.to_host(cut(d["drafts"]))
        return lambda: oracle.select_and_verify_rows(hp, pi, hq, qi, hd, temp_p=cfg.temp,
                                                     seed=seed, greedy=mode == "greedy",
                                                     nthreads=threads)
    hp, hd = W.to_host(cut(d["p"])), W.to_host(cut(d["drafts"]))
    if mode == "greedy":
        return lambda: oracle.greedy_select_and_verify(hp, hd, temp_p=cfg.temp, seed=seed,
                                                       nthreads=threads)
    hq = W.to_host(cut(d["q"]))
    return lambda: oracle.select_and_verify(hp, hq, hd, temp_p=cfg.temp, seed=seed,
                                            nthreads=threads, want_beta=want_beta)


def _time_oracle(run, seconds):
    reps, dt = 0, 0.0
    while reps == 0 or dt < seconds:
        t0 = time.perf_counter()
        run()
        dt += time.perf_counter() - t0
        reps += 1
    return reps, dt


# single-threaded samples of a batch larger than this many positions take the
# first few prefixes only, and the batch's rate is extrapolated from them
SINGLE_THREAD_MAX_POSITIONS = 4096


def cpu_baseline(d, cfg, seed, mode="standard", pooled=False, seconds=10.0, want_beta=False):
    """The oracle, untuned, timed on the host: the same batch on the host's
    thread share (repeated until about `seconds` of wall time have passed, at
    least once), and on one thread (the whole batch, or its first prefixes when
    the batch is large, then extrapolated to the batch)."""
    threads = host_threads()
    positions = cfg.B * cfg.K * cfg.gamma
    reps, dt = _time_oracle(_oracle_run(d, cfg, seed, mode, pooled, want_beta, threads), seconds)
    per_prefix = cfg.K * cfg.gamma
    n1 = cfg.B
    if positions > SINGLE_THREAD_MAX_POSITIONS:
        n1 = max(1, min(cfg.B, SINGLE_THREAD_MAX_POSITIONS // per_prefix, 4))
    reps1, dt1 = _time_oracle(_oracle_run(d, cfg, seed, mode, pooled, want_beta, 1,
                                          nprefix=n1 if n1 < cfg.B else None), seconds)
    rate1 = n1 * per_prefix * reps1 / dt1
    single = {"value": rate1, "unit": "positions/s", "threads": 1, "seconds": dt1,
              "sample": "%s%d of the %d prefixes (%d positions) %d times, %.1f s wall" % (
                  "" if n1 == cfg.B else "the first ", n1, cfg.B, n1 * per_prefix, reps1, dt1),
              "extrapolated": n1 < cfg.B}
    if n1 < cfg.B:
        single["batch_seconds_extrapolated"] = positions / rate1
    return {"value": positions * reps / dt, "unit": "positions/s", "cores": threads,
            "kind": "oracle",
            "sample": "the full %s batch (%d prefixes, %d positions) %d times, %.1f s wall on %d "
                      "threads" % (cfg.name, cfg.B, positions, reps, dt, threads),
            "seconds": dt, "single_thread": single, "cpu_model": cpu_model(),
            "host_cpus": os.cpu_count(), "threads_note": "the host's CPUs this process may use, "
            "at most 16 (one GPU's share of the host)"}


COPY_BYTES = 1 << 30
# Inputs smaller than this are rotated through copies of themselves, one per
# step, so that no step finds its logits in the 256 MB last-level cache (MALL)
# where the previous one left them.
COLD_BYTES = 1 << 30


def input_copies(nbytes: int) -> int:
    return max(1, min(512, -(-COLD_BYTES // max(nbytes, 1))))


def calibrate_copy(torch, steps):
    """A plain copy of a known number of bytes, to scale the HBM counters."""
    n = COPY_BYTES // 2  # bf16 elements: 1 GiB each way
    x = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(steps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read": 2 * n, "bytes_written": 2 * n,
                      "launches": steps}), flush=True)


CPS_TAU, CPS_MMAX, CPS_BEAM, CPS_LAMBDA = 0.8, 15, 3, 0.5


def cps_cpu_baseline(hq, flu, cfg, seconds=10.0):
    """The lattice and beam oracles, untuned: the prefixes split over the host's
    thread share (each thread runs both oracles on its slice; the oracle's C
    calls release the interpreter lock), and on one thread, each repeated
    until about `seconds` of wall time have passed."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    B, G = hq.shape[0], hq.shape[1]

    def one(sl):
        ol = oracle.cps_lattice(hq[sl], temp_q=cfg.temp, tau=CPS_TAU, m_max=CPS_MMAX)
        oracle.cps_beam(ol, flu[sl], lam=CPS_LAMBDA, beam=CPS_BEAM)

    threads = min(host_threads(), B)
    parts = [slice(i * B // threads, (i + 1) * B // threads) for i in range(threads)]
    with ThreadPoolExecutor(threads) as ex:
        reps, dt = _time_oracle(lambda: list(ex.map(one, parts)), seconds)
    reps1, dt1 = _time_oracle(lambda: one(slice(0, B)), seconds)
    rows = B * G
    return {"value": rows * reps / dt, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": "the %d drafter rows %d times on %d threads (%.1f s), %d times on one "
                      "(%.1f s)" % (rows, reps, threads, dt, reps1, dt1),
            "single_thread": {"value": rows * reps1 / dt1, "seconds": dt1, "reps": reps1},
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}


def bench_cps(args, torch, svd, W):
    """Causal-consistency path search over one drafter row per (prefix, position): the
    shared drafter rows of the shared_marginal workload (B = 16, gamma = 16)."""
    cfg = W.get_config("shared_marginal")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = W.generate_pooled(cfg, device=dev)
    B, G, V = cfg.B, cfg.gamma, cfg.V
    q = d["q_pool"].view(B, G, V)
    g = torch.Generator(device=dev)
    g.manual_seed(cfg.data_seed + 5)
    flu = torch.randn((B, G, CPS_MMAX, CPS_MMAX), generator=g, device=dev) * 0.3
    es = 2 if cfg.dtype == "bf16" else 4
    stream = torch.cuda.current_stream(dev)
    ncopy = input_copies(q.numel() * es)
    qs = [q] + [q.clone() for _ in range(ncopy - 1)]
    calls = [0]

    def step(lib=None):
        qc = qs[calls[0] % ncopy]
        calls[0] += 1
        lat = svd.cps_lattice(qc, temp_q=cfg.temp, tau=CPS_TAU, m_max=CPS_MMAX,
                              stream=stream.cuda_stream, lib=lib)
        return lat, svd.cps_beam(lat, flu, lam=CPS_LAMBDA, beam=CPS_BEAM,
                                 stream=stream.cuda_stream, lib=lib)

    warm = settle(torch, stream, step, args.warmup, args.settle_ms)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        lat, bm = step()
    ev1.record(stream)
    torch.cuda.synchronize()
    tl = svd.timing_library()
    nsamp = kernel_samples(args.steps)
    ms, n = time_kernels(torch, tl, lambda: step(tl), ["lattice"], nsamp)
    ms_all, n_all = time_kernels(torch, tl, lambda: step(tl), "all", min(args.steps, 10))
    ms_step = ev0.elapsed_time(ev1) / args.steps
    li = svd.KERNELS.index("lattice")
    ms_lat = ms[li] / max(n[li], 1)
    rows = B * G
    unit = V * es + CPS_MMAX * 8 + 8
    achieved = unit * rows / (ms_lat * 1e-3) / 1e9
    result = {
        "metric": "drafter rows/s through the causal-consistency path search (V=152064, bf16)",
        "value": rows / (ms_step * 1e-3), "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "settle_ms": warm["settle_ms"], "warmup_steps_run": warm["steps"],
        "config": {"workload": "cps_" + cfg.name, "B": B, "gamma": G, "V": V, "tau": CPS_TAU,
                   "m_max": CPS_MMAX, "beam": CPS_BEAM, "input_copies": ncopy},
        "kernel_ms": {k: ms_all[i] / max(n_all[i], 1) for i, k in enumerate(svd.KERNELS)
                      if n_all[i]},
        "roofline": {"kernel": "kr_lattice", "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic("lattice", "cps_" + cfg.name),
                     "bytes_per_unit": unit, "units_per_launch": rows,
                     "ms_per_launch": ms_lat, "sampled_steps": nsamp},
        "mean_lattice_width": float(lat["n_cand"].float().mean().item()),
        "env": run_env(torch, data_seed=cfg.data_seed, fluency_seed=cfg.data_seed + 5),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cps_cpu_baseline(W.to_host(q), flu.cpu().numpy(), cfg)
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps first (continued until --settle-ms of GPU time)")
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="least GPU time of warm-up before the timed steps, so that they run on "
                         "a settled clock (reported as settle_ms)")
    ap.add_argument("--workload", default="batched_serving")
    ap.add_argument("--mode", choices=("standard", "greedy"), default="standard",
                    help="acceptance rule: standard (alpha = min(1, p/q)) or greedy (alpha = p(x), "
                         "no drafter rows)")
    ap.add_argument("--early-exit", action="store_true",
                    help="K = 1 workloads: stream each prefix's positions only up to its first "
                         "rejection (svd_verify_window); reported apart from the full-streaming line")
    ap.add_argument("--cps", action="store_true",
                    help="time the causal-consistency path search instead (lattice of the "
                         "workload's drafter rows, then a beam of 3; tau 0.8, M_max 15)")
    ap.add_argument("--beta", action="store_true",
                    help="also ask for the overlap mass beta (a second pass over every scored "
                         "row pair; dense workloads, standard rule)")
    ap.add_argument("--vocab-shards", type=int, default=1,
                    help="one GPU's share of a vocabulary-sharded verifier: the workload with "
                         "V / N columns per row (the statistics exchange between shards is not "
                         "part of the step)")
    ap.add_argument("--batch", type=int, default=0,
                    help="the workload with this many prefixes instead of its own B (a sweep of "
                         "batch sizes over one row shape)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of known size (for counter calibration)")
    ap.add_argument("--record-traffic", nargs=4, metavar="DIR",
                    help="write the dominant kernel's traffic record from four rocprofv3 --pmc "
                         "output folders: FETCH_SIZE and WRITE_SIZE of this workload, then of "
                         "--calibrate-copy")
    args = ap.parse_args()
    if args.record_traffic:
        import workloads as W
        if args.cps:
            record_traffic("lattice", "cps_shared_marginal", args.mode, *args.record_traffic)
            return
        kern = "pool_stats" if W.get_config(args.workload).layout == "pooled" else "rowstats"
        record_traffic(kern, args.workload, args.mode, *args.record_traffic)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the verification path shards by prefix with no "
              "exchange, and this benchmark runs on a single GPU (got --gpus %d)"
              % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy:
        calibrate_copy(torch, max(args.steps, 1))
        return

    import lossless_draft_verification_verifier_amd as svd
    import workloads as W

    if args.cps:
        bench_cps(args, torch, svd, W)
        return

    cfg = W.get_config(args.workload)
    if args.vocab_shards > 1:
        import dataclasses
        cfg = dataclasses.replace(cfg, V=cfg.V // args.vocab_shards,
                                  name="%s_vshard%d" % (cfg.name, args.vocab_shards))
    if args.batch > 0:
        import dataclasses
        cfg = dataclasses.replace(cfg, B=args.batch, name="%s_B%d" % (cfg.name, args.batch))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pooled = cfg.layout == "pooled"
    d = W.generate_pooled(cfg, device=dev) if pooled else W.generate(cfg, device=dev)
    B, K, G, V = cfg.B, cfg.K, cfg.gamma, cfg.V
    es = 2 if cfg.dtype == "bf16" else 4
    if pooled:
        NP, NQ = d["p_pool"].shape[0], d["q_pool"].shape[0]
        ws = torch.empty(svd.svd_rows_workspace_bytes(B, K, G, V, NP, NQ), dtype=torch.uint8,
                         device=dev)
    else:
        ws = svd.alloc_workspace(B, K, G, V, dev)
    sel = torch.empty(B, dtype=torch.int32, device=dev)
    L = torch.empty(B, dtype=torch.int32, device=dev)
    tok = torch.empty(B, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    code = svd.SVD_BF16 if cfg.dtype == "bf16" else svd.SVD_F32

    greedy = args.mode == "greedy"
    early = args.early_exit
    if early and (pooled or K != 1):
        sys.exit("--early-exit needs a dense workload with K = 1")
    alpha_out = torch.empty((B, K, G), dtype=torch.float32, device=dev) if early else None
    if args.beta and (early or pooled or greedy):
        sys.exit("--beta needs a dense workload and the standard rule")
    beta_out = torch.empty((B, K, G), dtype=torch.float32, device=dev) if args.beta else None

    # the logits the kernels read, rotated through copies when small
    keys = ("p_pool", "q_pool") if pooled else ("p", "q")
    ncopy = input_copies(sum(d[k].numel() * d[k].element_size() for k in keys))
    ds = [d] + [dict(d, **{k: d[k].clone() for k in keys}) for _ in range(ncopy - 1)]
    calls = [0]

    def step(lib=svd._default):
        d = ds[calls[0] % ncopy]
        calls[0] += 1
        if early:
            rc = lib.svd_verify_window(
                svd.SVD_RULE_GREEDY if greedy else svd.SVD_RULE_STANDARD, d["p"], d["q"],
                d["drafts"], None, -1, 1, code, B, K, G, V, cfg.temp, cfg.temp, cfg.seed, 0, sel,
                L, tok, None, alpha_out, ws, ws.numel(), stream.cuda_stream)
        elif pooled:
            rc = lib.svd_select_and_verify_rows(
                svd.SVD_RULE_GREEDY if greedy else svd.SVD_RULE_STANDARD, d["p_pool"], NP,
                d["p_index"], d["q_pool"], NQ, d["q_index"], d["drafts"], code, B, K, G, V,
                cfg.temp, cfg.temp, cfg.seed, 0, sel, L, tok, None, None, ws, ws.numel(),
                stream.cuda_stream)
        elif greedy:
            rc = lib.svd_greedy_select_and_verify(d["p"], d["drafts"], code, B, K, G, V, cfg.temp,
                                                  cfg.seed, 0, sel, L, tok, None, None, ws,
                                                  ws.numel(), stream.cuda_stream)
        else:
            rc = lib.svd_select_and_verify(d["p"], d["q"], d["drafts"], code, B, K, G, V,
                                           cfg.temp, cfg.temp, cfg.seed, 0, sel, L, tok, None,
                                           None, beta_out, ws, ws.numel(), stream.cuda_stream)
        if rc != svd.SVD_OK:
            raise svd.SvdError(rc, "select_and_verify (%s)" % args.mode)

    warm = settle(torch, stream, step, args.warmup, args.settle_ms)

    # timed region: exactly --steps calls of the product library, between two
    # events on the call's stream; nothing else is recorded inside it
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / args.steps

    # right after it, on the settled clock: the dominant kernel's launches timed
    # with HIP events (recorded by the timing build on the stream the kernel is
    # launched on) in kernel_samples(--steps) more steps of the same inputs
    # (row pairs split into slices stream through kr_rowstats_split instead, and
    # the chunks of an early exit over a live list through kr_rowstats_live)
    tl = svd.timing_library()
    dom = "pool_stats" if pooled else "rowstats"
    timed = [dom] if pooled else ["rowstats", "rowstats_split", "rowstats_live"]
    nsamp = kernel_samples(args.steps)
    ms_kernels, launches = time_kernels(torch, tl, lambda: step(tl), timed, nsamp)
    if not pooled and launches[svd.KERNELS.index("rowstats")] == 0:
        dom = "rowstats_split"
        if launches[svd.KERNELS.index(dom)] == 0:
            dom = "rowstats_live"

    # then a few steps with every kernel timed, for the breakdown
    ms_all, launches_all = time_kernels(torch, tl, lambda: step(tl), "all", min(args.steps, 10))

    positions = B * K * G
    L_host = L.cpu().numpy()
    bonus_rows = int((L_host == G).sum())
    stream_ids = [svd.KERNELS.index(k) for k in timed]
    if early:
        # positions actually streamed (alpha is NaN at the others), over every
        # streaming launch of a step (the first chunk may stream whole rows,
        # the later ones slices of the live rows)
        streamed = int((~torch.isnan(alpha_out)).sum().item())
        stream_ids = [i for i in stream_ids if launches[i]]
        lpd = max(sum(launches[i] for i in stream_ids) / nsamp, 1)
        units = streamed / lpd
        unit_bytes = bytes_per_row_pair(V, es, args.mode)
        rows = 1 if greedy else 2
        alg_bytes_step = streamed * (rows * V * es + 4) + bonus_rows * V * es + B * 12
    elif pooled:
        units = pool_rows_read(d, args.mode)
        unit_bytes = V * es + POOL_STAT_BYTES
        # the pool rows read once, drafts and index tables, bonus rows drawn, outputs
        alg_bytes_step = (units * V * es + positions * (4 + 4 + (0 if greedy else 4)) +
                          bonus_rows * V * es + B * 12)
    else:
        units = positions
        unit_bytes = bytes_per_row_pair(V, es, args.mode)
        rows = 1 if greedy else 2
        alg_bytes_step = positions * (rows * V * es + 4) + bonus_rows * V * es + B * 12
    if early:
        ms_dom = sum(ms_kernels[i] for i in stream_ids) / max(sum(launches[i] for i in stream_ids), 1)
        dom_name = " + ".join(KERNEL_SYMBOL[svd.KERNELS[i]] for i in stream_ids)
    else:
        di = svd.KERNELS.index(dom)
        ms_dom = ms_kernels[di] / max(launches[di], 1)
        dom_name = KERNEL_SYMBOL[dom]
    launch_bytes = unit_bytes * units
    achieved = launch_bytes / (ms_dom * 1e-3) / 1e9
    traffic = None if early else measured_traffic(dom, cfg.name, args.mode)

    result = {
        "metric": METRIC,
        "value": positions / (ms_step * 1e-3),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "settle_ms": warm["settle_ms"],
        "warmup_steps_run": warm["steps"],
        "config": {"workload": cfg.name, "mode": args.mode, "early_exit": early,
                   "B": B, "K": K, "gamma": G, "V": V,
                   "logits": cfg.dtype, "temperature": cfg.temp, "global_batch": B,
                   "parallelism": "single GPU", "input_copies": ncopy,
                   "vocab_shards": args.vocab_shards},
        "achieved_hbm_gbps": alg_bytes_step / (ms_step * 1e-3) / 1e9,
        "hbm_frac_step": alg_bytes_step / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "kernel_ms": {k: ms_all[i] / max(launches_all[i], 1) for i, k in enumerate(svd.KERNELS)
                      if launches_all[i]},
        "roofline": {"kernel": dom_name, "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": traffic, "bytes_per_unit": unit_bytes,
                     "units_per_launch": units, "ms_per_launch": ms_dom,
                     "sampled_steps": nsamp,
                     "timing": "HIP events around the kernel's launches (timing build, same "
                               "kernels) in %d steps right after the timed region" % nsamp},
        "mean_accept_len": float(L_host.mean()),
        "mat": float(L_host.mean() + 1.0),
        "wall_s": wall,
        "env": run_env(torch, data_seed=cfg.data_seed, seed=cfg.seed, row_base=0),
    }
    if early:  # the window controller that follows a windowed call (one thread per prefix)
        result["adl"] = time_adl(torch, svd, stream, d["drafts"], sel, L, B, K, G)
    if args.beta:  # the second pass over every scored row pair (logit bytes of both rows)
        bi = svd.KERNELS.index("beta")
        ms_beta = ms_all[bi] / max(launches_all[bi], 1)
        gbps = positions * 2 * V * es / (ms_beta * 1e-3) / 1e9
        ci = svd.KERNELS.index("beta_combine")  # few row pairs: the slices' sums added
        ms_comb = ms_all[ci] / launches_all[ci] if launches_all[ci] else 0.0
        result["beta"] = {"kernel": "kr_beta", "ms": ms_beta, "achieved": gbps, "unit": "GB/s",
                          "frac": gbps / HBM_PEAK_GBPS, "combine_ms": ms_comb}
        result["config"]["beta"] = True
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(d, cfg, cfg.seed, args.mode, pooled, want_beta=args.beta)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
