#!/usr/bin/env python3
"""Benchmark of the chunked AllGather + bf16 GEMM hot path on one MI355X.

One step = one fused AG-GEMM call (chunk copy, per-chunk flags, rotated persistent MFMA GEMM) on the
8192 x 8192 x 8192 workload: 8 shards of (1024, 8192) bf16 ~N(0,1), B (8192, 8192) bf16 ~N(0,0.02),
comm blocks of 128 rows.  Inputs are resident in HBM before the timed region.  The JSON line also
carries the unfused (gather, then GEMM) and GEMM-only (flags pre-raised) times of the same workload,
the standalone TGATHER bandwidth on its two workloads, the MFMA roofline of the fused kernel, and the
CPU oracle timed on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
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

METRIC = "AG-GEMM bf16 TFLOP/s + gather GB/s (% of peak), fused vs unfused speedup"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target length of the CPU sample")
    return ap.parse_args()


def time_calls(fn, steps, warmup, stream):
    """Average ms per call over `steps` calls after `warmup` calls, HIP events on `stream`."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def recorded_traffic(tag: str, source: str):
    """HBM bytes per launch from a committed counter summary, or None when the kernel source has
    changed since the counters were taken."""
    path = os.path.join(PROFILES, tag + "_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path, encoding="utf-8"):
        if ":" in line and not line.startswith("#"):
            k, _, v = line.partition(":")
            vals[k.strip()] = v.strip()
    sha = hashlib.sha256(open(source, "rb").read()).hexdigest()
    if vals.get("kernel_source_sha256") != sha or "hbm_bytes_per_launch" not in vals:
        return None
    return float(vals["hbm_bytes_per_launch"])


def cpu_baseline(cfg, A, shards, B, target_s):
    """The oracle (as written, not tuned) on a bounded sample: full rows of C, all columns."""
    import numpy as np
    import torch
    import oracle
    u16 = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)
    sh = [u16(s) for s in shards]
    Bn = u16(B)
    rows = 2
    while True:
        ms = np.repeat(np.arange(rows, dtype=np.int64), cfg.Nc)
        ns = np.tile(np.arange(cfg.Nc, dtype=np.int64), rows)
        t0 = time.perf_counter()
        oracle.ag_gemm_at(sh, Bn, ms, ns)
        dt = time.perf_counter() - t0
        if dt >= target_s or rows >= cfg.M:
            break
        rows = min(cfg.M, max(rows * 2, int(rows * target_s / max(dt, 1e-3) * 1.05)))
    flops = 2.0 * rows * cfg.Nc * cfg.K
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "%d full rows x %d columns of C of the %s workload (%.1f s)" % (rows, cfg.Nc, cfg.name, dt)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (N shards live on one "
              "MI355X); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import allgather_gemm_amd as ag
    import workloads

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    cfg = workloads.AG_SQUARE
    A, shards, B = workloads.make_ag_gemm(cfg)
    sd = [s.to(dev) for s in shards]
    Bd = B.to(dev)
    C = torch.empty((cfg.M, cfg.Nc), dtype=torch.bfloat16, device=dev)
    a_gath = torch.empty((cfg.M, cfg.K), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    fused = lambda: ag.ag_gemm(sd, Bd, cfg.cb, C=C, a_out=a_gath)
    ms_fused = time_calls(fused, args.steps, args.warmup, stream)
    rc, info = ag.check()
    if rc != ag.AG_OK:
        print("fused call reported %s %s" % (ag.status_str(rc), info), file=sys.stderr)
        sys.exit(1)
    ms_unfused = time_calls(lambda: ag.ag_gemm(sd, Bd, cfg.cb, C=C, mode="unfused", a_out=a_gath),
                            args.steps, args.warmup, stream)
    ms_gemm_only = time_calls(lambda: ag.ag_gemm(sd, Bd, cfg.cb, C=C, mode="gemm_only", a_out=a_gath),
                              args.steps, args.warmup, stream)
    tflops = cfg.flops / (ms_fused * 1e-3) / 1e12

    # standalone TGATHER on its two workloads
    gathers = {}
    for tg in (workloads.TG_FP16, workloads.TG_RAGGED):
        shs = [s.to(dev) for s in workloads.make_tgather(tg.N, tg.D, tg.H, tg.W, tg.dtype, seed=tg.seed)]
        dst = torch.empty((tg.D[0], tg.D[1], tg.D[2], tg.N * tg.H, tg.W), dtype=tg.dtype, device=dev)
        vr = tg.valid_rows or tg.H
        vc = tg.valid_cols or tg.W
        ms = time_calls(lambda: ag.tgather(shs, vr, vc, dst=dst), args.steps, args.warmup, stream)
        gbs = 2.0 * tg.payload_bytes / (ms * 1e-3) / 1e9
        gathers[tg.name] = {"ms": round(ms, 5), "GB/s": round(gbs, 1),
                            "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                            "valid_rows": vr, "valid_cols": vc}
        del shs, dst

    gemm_src = os.path.join(ROOT, "allgather_gemm_amd", "csrc", "ag_gemm.hip")
    traffic = recorded_traffic("gemm_fused_8192", gemm_src)
    roofline = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic}

    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_fused, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded randn/rand, shapes of the configured workloads)",
        "config": {"workload": cfg.name + " fused", "M": cfg.M, "K": cfg.K, "Nc": cfg.Nc,
                   "shards": cfg.N, "comm_block_rows": cfg.cb, "local_rank": 0},
        "roofline": roofline,
        "schedules": {
            "fused_ms": round(ms_fused, 5), "unfused_ms": round(ms_unfused, 5),
            "gemm_only_ms": round(ms_gemm_only, 5),
            "fused_vs_unfused_speedup": round(ms_unfused / ms_fused, 4),
            "gemm_only_tflops": round(cfg.flops / (ms_gemm_only * 1e-3) / 1e12, 2),
        },
        "tgather": gathers,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, A, shards, B, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
