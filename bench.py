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
METRIC = "verified draft positions/sec and achieved HBM GB/s (V=152064, bf16 logits)"
# sources whose text decides each kernel's memory traffic
KERNEL_SOURCES = {
    "rowstats": ["svd_device.hpp", "kr_rowstats.hpp"],
    "fused": ["svd_device.hpp", "kr_rowstats.hpp", "kr_select.hpp", "kr_draw.hpp",
              "kr_fused.hpp", "svd_api.hip"],
}
KERNEL_SYMBOL = {"rowstats": "kr_rowstats", "fused": "kr_fused"}


def traffic_file(kernel: str) -> str:
    return os.path.join(ROOT, "profiles", "%s_traffic.json" % KERNEL_SYMBOL[kernel])


def kernel_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "lossless_draft_verification_verifier_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of a kernel from committed rocprofv3 counter
    summaries, or None when they are missing or the kernel changed since."""
    try:
        with open(traffic_file(kernel)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_hash") != kernel_hash(kernel) or rec.get("workload") != workload:
        return None
    return rec.get("hbm_bytes_per_launch")


def bytes_per_row_pair(V: int, es: int) -> int:
    """Algorithmic bytes of one scored row pair: both logit rows, the drafted
    token, and the 16-byte statistics record plus the 4-byte alpha written for
    it.  (Bonus rows and the 12 output bytes per prefix are left out, so the
    figure is a lower bound.)"""
    return 2 * V * es + 4 + 16 + 4


def cpu_baseline(d, cfg, seed):
    import numpy as np  # noqa: F401
    import oracle
    import workloads as W
    threads = max(1, min(16, os.cpu_count() or 1))
    hp, hq, hd = W.to_host(d["p"]), W.to_host(d["q"]), W.to_host(d["drafts"])
    t0 = time.perf_counter()
    oracle.select_and_verify(hp, hq, hd, temp_p=cfg.temp, seed=seed, nthreads=threads)
    dt = time.perf_counter() - t0
    positions = cfg.B * cfg.K * cfg.gamma
    return {"value": positions / dt, "unit": "positions/s", "cores": threads, "kind": "oracle",
            "sample": "the full %s batch (%d prefixes, %d positions), %.2f s wall on %d threads"
                      % (cfg.name, cfg.B, positions, dt, threads),
            "seconds": dt}


def calibrate_copy(torch, steps):
    """A plain copy of a known number of bytes, to scale the HBM counters."""
    n = 1 << 29  # 1 GiB of bf16 each way
    x = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(steps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read": 2 * n, "bytes_written": 2 * n,
                      "launches": steps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="batched_serving")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of known size (for counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the verification path shards by prefix with no "
              "exchange, and multi-GPU runs are not part of this build (got --gpus %d)"
              % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy:
        calibrate_copy(torch, max(args.steps, 1))
        return

    import lossless_draft_verification_verifier_amd as svd
    import workloads as W

    cfg = W.get_config(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = W.generate(cfg, device=dev)
    B, K, G, V = cfg.B, cfg.K, cfg.gamma, cfg.V
    es = 2 if cfg.dtype == "bf16" else 4
    ws = svd.alloc_workspace(B, K, G, V, dev)
    sel = torch.empty(B, dtype=torch.int32, device=dev)
    L = torch.empty(B, dtype=torch.int32, device=dev)
    tok = torch.empty(B, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    code = svd.SVD_BF16 if cfg.dtype == "bf16" else svd.SVD_F32

    def step():
        rc = svd.svd_select_and_verify(d["p"], d["q"], d["drafts"], code, B, K, G, V, cfg.temp,
                                       cfg.temp, cfg.seed, 0, sel, L, tok, None, None, None, ws,
                                       ws.numel(), stream.cuda_stream)
        if rc != svd.SVD_OK:
            raise svd.SvdError(rc, "svd_select_and_verify")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    svd.svd_profile_read()  # clear

    # timed region: K steps, kernel events recorded on the call's stream
    svd.svd_profile_enable(True)
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
    svd.svd_profile_enable(False)
    ms_kernels, launches = svd.svd_profile_read()
    ms_step = ev0.elapsed_time(ev1) / args.steps

    positions = B * K * G
    L_host = L.cpu().numpy()
    bonus_rows = int((L_host == G).sum())
    alg_bytes_step = positions * (2 * V * es + 4) + bonus_rows * V * es + B * 12
    # the dominant kernel: the one with the most time in the timed region
    dom = max(("fused", "rowstats"), key=lambda k: ms_kernels[svd.KERNELS.index(k)])
    di = svd.KERNELS.index(dom)
    ms_dom = ms_kernels[di] / max(launches[di], 1)
    unit_bytes = bytes_per_row_pair(V, es)
    launch_bytes = unit_bytes * positions
    achieved = launch_bytes / (ms_dom * 1e-3) / 1e9
    traffic = measured_traffic(dom, cfg.name)

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
        "config": {"workload": cfg.name, "B": B, "K": K, "gamma": G, "V": V,
                   "logits": cfg.dtype, "temperature": cfg.temp, "global_batch": B,
                   "parallelism": "single GPU"},
        "achieved_hbm_gbps": alg_bytes_step / (ms_step * 1e-3) / 1e9,
        "hbm_frac_step": alg_bytes_step / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "kernel_ms": {k: ms_kernels[i] / max(launches[i], 1) for i, k in enumerate(svd.KERNELS)
                      if launches[i]},
        "roofline": {"kernel": KERNEL_SYMBOL[dom], "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": traffic, "bytes_per_unit": unit_bytes,
                     "units_per_launch": positions},
        "mean_accept_len": float(L_host.mean()),
        "mat": float(L_host.mean() + 1.0),
        "wall_s": wall,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(d, cfg, cfg.seed)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
