#!/usr/bin/env python3
"""Benchmark of the chunked AllGather + bf16 GEMM hot path on one MI355X.

One step = one fused AG-GEMM call (chunk copy by a copy kernel on a second stream beside the rotated
persistent MFMA GEMM, per-chunk flags, waiting tiles copy too) on the 8192 x 8192 x 8192 workload:
8 shards of (1024, 8192) bf16 ~N(0,1),
B (8192, 8192) bf16 ~N(0,0.02), comm blocks of 128 rows.  Inputs are resident in HBM before the
timed region.  The headline is K back-to-back steps; the GEMM kernel inside them is timed with HIP
events the library records around its launch, on its stream, which gives the roofline figure.

Besides the headline the JSON line carries, per the fused AllGather+MatMul article's reporting list
(section 性能结果与适用边界: warm-up, statistic, baseline, effective bandwidth, utilisation):
  * every schedule of the square workload -- fused with each producer, unfused (gather, then GEMM),
    GEMM-only (flags raised beforehand) and the plain GEMM alone -- as median / p10 / p90 of
    individually timed calls, cold (a 1 GiB read evicts L2 and the MALL before every call) and hot;
  * the MLP-up (16384 x 14336 x 4096) and ragged (4000 x 28672 x 8192) workloads the same way;
  * GEMM + ReduceScatter (one rank's share of the square workload split over 8 ranks), fused and
    serial;
  * FP8 inputs (E4M3 A and B, bf16 C) on the square workload, its schedules as above, the GEMM
    kernel against the 5 PFLOP/s dense fp8 peak;
  * TGATHER on its two workloads, cold and hot, as GB/s of algorithmic traffic;
  * the shader clock sampled while fused calls run back to back;
  * the CPU oracle timed on a bounded sample of the square workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--reps R] [--no-cpu-baseline]
       python bench.py --headline-only ...   (headline steps only, for kernel traces and counters)
       python bench.py --tgather-only ...    (TGATHER workloads only, likewise)
       python bench.py --rs-only ...         (GEMM + ReduceScatter only, likewise)
       python bench.py --fp8-only ...        (FP8-input square workload only, likewise)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import shutil
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "AG-GEMM bf16 TFLOP/s + gather GB/s (% of peak), fused vs unfused speedup"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA, published
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
MFMA_FLOPS_PER_CLK = 256 * 4 * 1024   # CUs x SIMDs x dense bf16 flops per SIMD per clock
PROFILES = os.path.join(ROOT, "profiles")
GEMM_SRC = os.path.join(ROOT, "allgather_gemm_amd", "csrc", "ag_gemm.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30,
                    help="untimed steps first: the clock settles only after a few dozen calls")
    ap.add_argument("--reps", type=int, default=50, help="individually timed calls per schedule statistic")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target length of the CPU sample")
    ap.add_argument("--headline-only", action="store_true",
                    help="only the headline steps (plus one calibration copy): for rocprofv3 runs")
    ap.add_argument("--workload", default="ag_gemm_8192x8192x8192",
                    help="with --headline-only: the AG-GEMM workload of the steps (a name from workloads.py)")
    ap.add_argument("--mode", default="fused", choices=("fused", "fused_in_kernel", "unfused", "plain_gemm"),
                    help="with --headline-only: the schedule of the steps (fused_in_kernel: the fused "
                         "schedule with the GEMM's own workgroups copying)")
    ap.add_argument("--tgather-only", action="store_true",
                    help="only TGATHER on its two workloads, --steps calls each: for rocprofv3 runs")
    ap.add_argument("--fp8-only", action="store_true",
                    help="only the FP8-input square workload, --steps fused calls: for rocprofv3 runs")
    ap.add_argument("--rs-only", action="store_true",
                    help="only GEMM + ReduceScatter, --steps fused then --steps serial calls: for rocprofv3 runs")
    return ap.parse_args()


def pct(xs, q):
    xs = sorted(xs)
    if not xs:
        return None
    i = min(len(xs) - 1, max(0, int(round(q * (len(xs) - 1)))))
    return xs[i]


def stats(ms_list):
    return {"median_ms": round(pct(ms_list, 0.5), 5), "p10_ms": round(pct(ms_list, 0.1), 5),
            "p90_ms": round(pct(ms_list, 0.9), 5)}


class Scrubber:
    """Reads 1 GiB so that neither L2 nor the 256 MB MALL holds anything of the next call's data.
    Reading (not writing) leaves no dirty lines behind, whose write-back would otherwise land inside
    the timed call; the last call's own dirty lines are written back during the scrub."""

    def __init__(self, torch, dev):
        self.buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        self.out = torch.empty((), dtype=torch.float32, device=dev)
        self.torch = torch

    def __call__(self):
        self.torch.amax(self.buf, dim=0, out=self.out)


def time_each(torch, fn, reps, warmup, stream, scrub=None, events=False):
    """Individually event-timed calls.  Returns (call ms list, GEMM-kernel ms list or None)."""
    for _ in range(warmup):
        fn(None)
    torch.cuda.synchronize()
    calls, kernels = [], []
    for _ in range(reps):
        if scrub is not None:
            scrub()
        # keep the GPU busy while the host enqueues the call, so host latency stays out of the window
        torch.cuda._sleep(100000)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        k = None
        if events:
            k = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            k[0].record(stream)     # materialise the events before the library records them
            k[1].record(stream)
        e0.record(stream)
        fn(k)
        e1.record(stream)
        e1.synchronize()
        calls.append(e0.elapsed_time(e1))
        if k is not None:
            kernels.append(k[0].elapsed_time(k[1]))
    return calls, (kernels if events else None)


class ClockSampler:
    """Samples the GFX clock from amd-smi (or rocm-smi) in a thread while work runs."""

    def __init__(self, period=0.05):
        self.period = period
        self.samples = []
        self.stop_flag = False
        self.cmd = None
        if shutil.which("amd-smi"):
            self.cmd = ["amd-smi", "metric", "-g", "0", "--clock", "--json"]
        elif shutil.which("rocm-smi"):
            self.cmd = ["rocm-smi", "-d", "0", "--showclocks", "--json"]

    @staticmethod
    def _parse(text):
        # amd-smi: {"clock": {"gfx_0": {"clk": {"value": 2100, "unit": "MHz"}, ...}}} (layouts vary);
        # rocm-smi: {"card0": {"sclk clock speed:": "(2100Mhz)", ...}}
        try:
            data = json.loads(text)
        except ValueError:
            return None
        found = []

        def walk(node, path):
            if isinstance(node, dict):
                for k, v in node.items():
                    walk(v, path + [str(k).lower()])
            elif isinstance(node, list):
                for v in node:
                    walk(v, path)
            else:
                p = "/".join(path)
                if ("gfx" in p or "sclk" in p) and "min" not in p and "max" not in p and "lock" not in p.split("/")[-1]:
                    m = re.search(r"(\d+(?:\.\d+)?)", str(node))
                    if m and ("value" in path[-1] or "sclk" in p or path[-1] == "clk"):
                        found.append(float(m.group(1)))

        walk(data, [])
        vals = [v for v in found if 100.0 <= v <= 5000.0]
        return max(vals) if vals else None

    def run(self):
        while not self.stop_flag:
            try:
                out = subprocess.run(self.cmd, capture_output=True, text=True, timeout=5).stdout
                v = self._parse(out)
                if v is not None:
                    self.samples.append(v)
            except Exception:
                pass
            time.sleep(self.period)

    def __enter__(self):
        if self.cmd:
            self.th = threading.Thread(target=self.run, daemon=True)
            self.th.start()
        return self

    def __exit__(self, *exc):
        self.stop_flag = True
        if self.cmd:
            self.th.join(timeout=10)

    def result(self):
        if not self.samples:
            return None
        return {"source": self.cmd[0], "samples": len(self.samples),
                "mean_mhz": round(sum(self.samples) / len(self.samples), 1),
                "min_mhz": min(self.samples), "max_mhz": max(self.samples)}


def recorded_traffic(tag: str):
    """HBM bytes per launch from a committed counter summary of the current kernel source, or None."""
    path = os.path.join(PROFILES, tag + "_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path, encoding="utf-8"):
        if ":" in line and not line.startswith("#"):
            k, _, v = line.partition(":")
            vals[k.strip()] = v.strip()
    sha = hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()
    if vals.get("kernel_source_sha256") != sha or "hbm_bytes_per_launch" not in vals:
        return None
    return float(vals["hbm_bytes_per_launch"])


def ag_cus(torch) -> int:
    return torch.cuda.get_device_properties(0).multi_processor_count


def cpu_baseline(cfg, shards, B, target_s):
    """The oracle as it stands (naive ascending-k loop, gcc -O3, no -march, OpenMP) on a bounded
    sample: full rows of C, every column."""
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
    threads = oracle.num_threads()
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "%d full rows x %d columns of C of the %s workload (%.1f s; oracle built gcc -O3 "
                      "-fopenmp -ffp-contract=off, no -march)" % (rows, cfg.Nc, cfg.name, dt)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the N shards live on one "
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

    def fp8_inputs():
        fcfg = workloads.AG_SQUARE_FP8
        fA, fsh, fB = workloads.make_ag_gemm_fp8(fcfg)
        fsd = [t.to(dev) for t in fsh]
        fBd = fB.to(dev)
        fC = torch.empty((fcfg.M, fcfg.Nc), dtype=torch.bfloat16, device=dev)
        fa = torch.empty((fcfg.M, fcfg.K), dtype=torch.uint8, device=dev)
        fkw = {"in_dtype": "fp8_e4m3", "out_scale": 1.0 / math.sqrt(fcfg.K)}
        torch.cuda.synchronize()
        return fcfg, fsd, fBd, fC, fa, fkw

    if args.fp8_only:
        fcfg, fsd, fBd, fC, fa, fkw = fp8_inputs()
        kev8 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for k in kev8:      # torch creates an event when it first records it
            k[0].record(stream)
            k[1].record(stream)
        for _ in range(args.warmup):
            ag.ag_gemm(fsd, fBd, fcfg.cb, C=fC, a_out=fa, **fkw)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            ag.ag_gemm(fsd, fBd, fcfg.cb, C=fC, a_out=fa, gemm_events=kev8[i], **fkw)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        kms = sum(k[0].elapsed_time(k[1]) for k in kev8) / args.steps
        print(json.dumps({"fp8_only": True, "workload": fcfg.name, "ms_per_step": round(ms, 5),
                          "gemm_kernel_ms": round(kms, 5),
                          "kernel_TFLOP/s": round(fcfg.flops / (kms * 1e-3) / 1e12, 2)}), flush=True)
        return

    if args.rs_only:
        rcfg = workloads.RS_SQUARE
        rA, rB, rrecv = workloads.make_gemm_rs(rcfg)
        rAd, rBd = rA.to(dev), rB.to(dev)
        rrd = [None if t is None else t.to(dev) for t in rrecv]
        rP = torch.empty((rcfg.M, rcfg.Nc), dtype=torch.bfloat16, device=dev)
        rout = torch.empty((rcfg.H, rcfg.Nc), dtype=torch.bfloat16, device=dev)
        out = {}
        for name, fused in (("fused", True), ("unfused", False)):
            for _ in range(args.warmup):
                ag.gemm_rs(rAd, rBd, rrd, rcfg.local, P=rP, out=rout, fused=fused)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(args.steps):
                ag.gemm_rs(rAd, rBd, rrd, rcfg.local, P=rP, out=rout, fused=fused)
            e1.record(stream)
            torch.cuda.synchronize()
            out[name + "_ms_per_call"] = round(e0.elapsed_time(e1) / args.steps, 5)
        print(json.dumps({"rs_only": True, "workload": rcfg.name, **out}), flush=True)
        return

    if args.tgather_only:
        out = {}
        for tg in (workloads.TG_FP16, workloads.TG_RAGGED):
            shs = [s.to(dev) for s in workloads.make_tgather(tg.N, tg.D, tg.H, tg.W, tg.dtype, seed=tg.seed)]
            dst = torch.empty((tg.D[0], tg.D[1], tg.D[2], tg.N * tg.H, tg.W), dtype=tg.dtype, device=dev)
            vr, vc = tg.valid_rows or tg.H, tg.valid_cols or tg.W
            for _ in range(args.warmup):
                ag.tgather(shs, vr, vc, dst=dst)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(args.steps):
                ag.tgather(shs, vr, vc, dst=dst)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / args.steps
            out[tg.name] = {"ms_per_call": round(ms, 5), "payload_bytes": tg.payload_bytes,
                            "GB/s": round(2 * tg.payload_bytes / (ms * 1e-3) / 1e9, 1)}
            del shs, dst
        print(json.dumps({"tgather_only": True, **out}), flush=True)
        return

    def load(cfg):
        A, shards, B = workloads.make_ag_gemm(cfg)
        sd = [s.to(dev) for s in shards]
        Bd = B.to(dev)
        C = torch.empty((cfg.M, cfg.Nc), dtype=torch.bfloat16, device=dev)
        a_gath = torch.empty((cfg.M, cfg.K), dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()
        return A, shards, B, sd, Bd, C, a_gath

    cfg = workloads.AG_SQUARE
    mode = "fused"
    if args.headline_only:
        # a rocprofv3 run of another workload or schedule: the same steps, nothing else
        cfg = workloads.AG_CONFIGS[args.workload]
        mode = args.mode
    A, shards, B, sd, Bd, C, a_gath = load(cfg)
    if mode == "plain_gemm":
        a_gath.copy_(A.to(dev))   # the plain GEMM reads the gathered A as its input
    step_kw = {"producer": "in_kernel"} if mode == "fused_in_kernel" else {"mode": mode}

    # headline: K back-to-back fused steps, the GEMM kernel of each timed by the library's events
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for k in kev:
        k[0].record(stream)
        k[1].record(stream)
    for _ in range(args.warmup):
        ag.ag_gemm(sd, Bd, cfg.cb, C=C, a_out=a_gath, **step_kw)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        ag.ag_gemm(sd, Bd, cfg.cb, C=C, a_out=a_gath, gemm_events=kev[i], **step_kw)
    end.record(stream)
    torch.cuda.synchronize()
    ms_fused = start.elapsed_time(end) / args.steps
    gemm_kernel_ms = sum(k[0].elapsed_time(k[1]) for k in kev) / args.steps
    rc, info = ag.check()
    if rc != ag.AG_OK:
        print("fused call reported %s %s" % (ag.status_str(rc), info), file=sys.stderr)
        sys.exit(1)
    tflops = cfg.flops / (ms_fused * 1e-3) / 1e12
    kernel_tflops = cfg.flops / (gemm_kernel_ms * 1e-3) / 1e12

    # how long the fused GEMM's tiles waited on chunk flags: 10 more calls, outside the timed steps
    wst = torch.zeros(4, dtype=torch.int64, device=dev)
    nw = 10 if mode in ("fused", "fused_in_kernel") else 0
    for _ in range(nw):
        ag.ag_gemm(sd, Bd, cfg.cb, C=C, a_out=a_gath, wait_stats=wst, **step_kw)
    torch.cuda.synchronize()
    nw = max(nw, 1)
    ticks, waits, copied, skipped = (int(v) for v in wst.cpu().tolist())
    grid = min(ag_cus(torch), ((cfg.M + 255) // 256) * ((cfg.Nc + 255) // 256))
    fused_waits = {
        "calls": nw, "workgroups": grid,
        "wait_us_per_call_summed_over_workgroups": round(ticks / 100.0 / nw, 2),
        "wait_us_per_workgroup_per_call": round(ticks / 100.0 / nw / grid, 3),
        "waits_per_call": waits / nw, "tiles_skipping_the_wait_per_call": skipped / nw,
        "pieces_copied_by_waiting_tiles_per_call": copied / nw,
        "pieces_per_call": cfg.N * ((cfg.H + cfg.cb - 1) // cfg.cb) * ((cfg.cb * cfg.K * 2 + 16383) // 16384),
    }
    if mode not in ("fused", "fused_in_kernel"):
        fused_waits = None

    if args.headline_only:
        # one copy of known size, for scaling the memory counters of a profiled run: 256 MiB read
        # and written once each, with the caches evicted first so that every byte comes from HBM
        shs = [torch.ones((4096, 4096), dtype=torch.float16, device=dev) for _ in range(8)]
        dst = torch.empty((8 * 4096, 4096), dtype=torch.float16, device=dev)
        Scrubber(torch, dev)()
        ag.tgather(shs, 4096, 4096, dst=dst)
        torch.cuda.synchronize()
        print(json.dumps({"headline_only": True, "workload": cfg.name, "mode": mode,
                          "ms_per_step": round(ms_fused, 5),
                          "gemm_kernel_ms": round(gemm_kernel_ms, 5), "TFLOP/s": round(tflops, 2),
                          "fused_waits": fused_waits,
                          "calibration_copy_bytes_each_way": 8 * 4096 * 4096 * 2}), flush=True)
        return

    scrub = Scrubber(torch, dev)
    reps, warm = args.reps, 3

    def schedule_stats(cfg, sd, Bd, C, a_gath, modes):
        out = {}
        for name, kw in modes:
            fn = lambda k, kw=kw: ag.ag_gemm(sd, Bd, cfg.cb, C=C, a_out=a_gath, gemm_events=k, **kw)
            cold, kcold = time_each(torch, fn, reps, warm, stream, scrub=scrub, events=True)
            hot, khot = time_each(torch, fn, reps, warm, stream, scrub=None, events=True)
            rc, info = ag.check()
            if rc != ag.AG_OK:
                print("%s reported %s %s" % (name, ag.status_str(rc), info), file=sys.stderr)
                sys.exit(1)
            ent = {"cold": stats(cold), "hot": stats(hot),
                   "gemm_kernel_cold_median_ms": round(pct(kcold, 0.5), 5),
                   "gemm_kernel_hot_median_ms": round(pct(khot, 0.5), 5)}
            ent["cold_tflops"] = round(cfg.flops / (ent["cold"]["median_ms"] * 1e-3) / 1e12, 2)
            ent["hot_tflops"] = round(cfg.flops / (ent["hot"]["median_ms"] * 1e-3) / 1e12, 2)
            out[name] = ent
        fu, un = out["fused"]["cold"]["median_ms"], out["unfused"]["cold"]["median_ms"]
        out["fused_vs_unfused_speedup_cold"] = round(un / fu, 4)
        out["fused_vs_unfused_speedup_hot"] = round(out["unfused"]["hot"]["median_ms"] /
                                                    out["fused"]["hot"]["median_ms"], 4)
        return out

    modes_sq = [("fused", {}), ("fused_in_kernel", {"producer": "in_kernel"}),
                ("fused_copy_engine", {"producer": "copy_engine"}), ("unfused", {"mode": "unfused"}),
                ("gemm_only", {"mode": "gemm_only"}), ("plain_gemm", {"mode": "plain_gemm"})]
    # gathered A for the GEMM-only / plain modes
    ag.ag_gemm(sd, Bd, cfg.cb, C=C, a_out=a_gath, mode="unfused")
    sched = schedule_stats(cfg, sd, Bd, C, a_gath, modes_sq)

    # the shader clock while fused calls run back to back (about two seconds)
    with ClockSampler() as clk:
        t_end = time.time() + 2.0
        while time.time() < t_end:
            for _ in range(20):
                ag.ag_gemm(sd, Bd, cfg.cb, C=C, a_out=a_gath)
            torch.cuda.synchronize()
    sclk = clk.result()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, shards, B, args.cpu_seconds)
    del A, shards, B, sd, Bd, C, a_gath
    torch.cuda.empty_cache()

    # the other two AG-GEMM workloads
    other = {}
    modes_o = [("fused", {}), ("unfused", {"mode": "unfused"}), ("gemm_only", {"mode": "gemm_only"}),
               ("plain_gemm", {"mode": "plain_gemm"})]
    for ocfg in (workloads.AG_MLP_UP, workloads.AG_RAGGED):
        _, _, _, osd, oBd, oC, oa = load(ocfg)
        ag.ag_gemm(osd, oBd, ocfg.cb, C=oC, a_out=oa, mode="unfused")
        other[ocfg.name] = schedule_stats(ocfg, osd, oBd, oC, oa, modes_o)
        del osd, oBd, oC, oa
        torch.cuda.empty_cache()

    # FP8 inputs on the square workload: E4M3 A and B, bf16 C = A B^T / sqrt(K)
    fcfg, fsd, fBd, fC, fa, fkw = fp8_inputs()
    ag.ag_gemm(fsd, fBd, fcfg.cb, C=fC, a_out=fa, mode="unfused", **fkw)
    fp8_in = schedule_stats(fcfg, fsd, fBd, fC, fa, [(n, {**kw, **fkw}) for n, kw in modes_o])
    for name in ("fused", "unfused", "gemm_only", "plain_gemm"):
        kms = fp8_in[name]["gemm_kernel_hot_median_ms"]
        fp8_in[name]["gemm_kernel_hot_tflops"] = round(fcfg.flops / (kms * 1e-3) / 1e12, 2)
        fp8_in[name]["gemm_kernel_hot_frac_of_fp8_peak"] = round(fcfg.flops / (kms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4)
    fp8_in["config"] = {"workload": fcfg.name, "M": fcfg.M, "K": fcfg.K, "Nc": fcfg.Nc, "shards": fcfg.N,
                        "comm_block_rows": fcfg.cb, "inputs": "fp8_e4m3", "C": "bf16",
                        "out_scale": fkw["out_scale"], "peak_tflops": PEAK_FP8_TFLOPS}
    del fsd, fBd, fC, fa
    torch.cuda.empty_cache()

    # GEMM + ReduceScatter, one rank's share, on the square workload split over 8 ranks
    rcfg = workloads.RS_SQUARE
    rA, rB, rrecv = workloads.make_gemm_rs(rcfg)
    rAd, rBd = rA.to(dev), rB.to(dev)
    rrd = [None if t is None else t.to(dev) for t in rrecv]
    rP = torch.empty((rcfg.M, rcfg.Nc), dtype=torch.bfloat16, device=dev)
    rout = torch.empty((rcfg.H, rcfg.Nc), dtype=torch.bfloat16, device=dev)
    rs = {}
    for name, fused in (("fused", True), ("unfused", False)):
        fn = lambda k, fused=fused: ag.gemm_rs(rAd, rBd, rrd, rcfg.local, P=rP, out=rout, fused=fused)
        cold, _ = time_each(torch, fn, reps, warm, stream, scrub=scrub)
        hot, _ = time_each(torch, fn, reps, warm, stream)
        rs[name] = {"cold": stats(cold), "hot": stats(hot)}
        rs[name]["cold_tflops"] = round(rcfg.flops / (rs[name]["cold"]["median_ms"] * 1e-3) / 1e12, 2)
    rc, info = ag.check()
    if rc != ag.AG_OK:
        print("gemm_rs reported %s %s" % (ag.status_str(rc), info), file=sys.stderr)
        sys.exit(1)
    rs["fused_vs_unfused_speedup_cold"] = round(rs["unfused"]["cold"]["median_ms"] / rs["fused"]["cold"]["median_ms"], 4)
    rs["fused_vs_unfused_speedup_hot"] = round(rs["unfused"]["hot"]["median_ms"] / rs["fused"]["hot"]["median_ms"], 4)
    rs["config"] = {"workload": rcfg.name, "M": rcfg.M, "K_per_rank": rcfg.K, "Nc": rcfg.Nc, "ranks": rcfg.N,
                    "local_rank": rcfg.local}
    del rAd, rBd, rrd, rP, rout
    torch.cuda.empty_cache()

    # standalone TGATHER on its two workloads
    gathers = {}
    for tg in (workloads.TG_FP16, workloads.TG_RAGGED):
        shs = [s.to(dev) for s in workloads.make_tgather(tg.N, tg.D, tg.H, tg.W, tg.dtype, seed=tg.seed)]
        dst = torch.empty((tg.D[0], tg.D[1], tg.D[2], tg.N * tg.H, tg.W), dtype=tg.dtype, device=dev)
        vr = tg.valid_rows or tg.H
        vc = tg.valid_cols or tg.W
        fn = lambda k: ag.tgather(shs, vr, vc, dst=dst)
        cold, _ = time_each(torch, fn, reps, warm, stream, scrub=scrub)
        hot, _ = time_each(torch, fn, reps, warm, stream)
        ent = {"cold": stats(cold), "hot": stats(hot), "valid_rows": vr, "valid_cols": vc}
        for k in ("cold", "hot"):
            gbs = 2.0 * tg.payload_bytes / (ent[k]["median_ms"] * 1e-3) / 1e9
            ent[k + "_GB/s"] = round(gbs, 1)
            ent[k + "_frac_of_hbm_peak"] = round(gbs / PEAK_HBM_GBS, 4)
        gathers[tg.name] = ent
        del shs, dst

    traffic = recorded_traffic("gemm_fused_8192")
    roofline = {"bound": "mfma", "achieved": round(kernel_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(kernel_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "kernel": "gemm_fused_kernel", "kernel_ms": round(gemm_kernel_ms, 5),
                "flops_per_launch": cfg.flops}
    if sclk:
        peak_at_clock = MFMA_FLOPS_PER_CLK * sclk["mean_mhz"] * 1e6 / 1e12
        roofline["peak_at_sampled_sclk"] = round(peak_at_clock, 1)
        roofline["frac_at_sampled_sclk"] = round(kernel_tflops / peak_at_clock, 4)

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
                   "shards": cfg.N, "comm_block_rows": cfg.cb, "local_rank": 0, "producer": "side_stream"},
        "roofline": roofline,
        "fused_waits": fused_waits,
        "schedules": sched,
        "workloads": other,
        "tgather": gathers,
        "gemm_reduce_scatter": rs,
        "fp8_inputs": fp8_in,
        "sclk": sclk,
        "protocol": {"reps": reps, "warmup_per_statistic": warm,
                     "cold": "1 GiB read (torch amax) before every timed call", "statistic": "median, p10, p90"},
    }
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
