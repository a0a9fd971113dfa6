"""Benchmark of the FP8 block-scaled GEMM on one MI355X.

One step = the dense decode/prefill sweep over DeepSeek-V3-like projection shapes: M in
{64, 128, 4096} x (N, K) in {(2112,7168), (24576,1536), (32768,512), (7168,16384), (4096,7168),
(7168,2048)} -- 18 GEMMs, each D[M,N] bf16 = A[M,K] e4m3 (1x128 fp32 scales) . B[N,K]^T e4m3
(128x128 fp32 scales).  Inputs are synthetic, seeded, quantised from N(0,1) and resident in HBM
before timing; consecutive GEMMs use different buffers (about 1.3 GB per step), so each GEMM's
operands are not left in the 256 MB last-level cache by the previous one.

Prints ONE JSON line: value = aggregate FP8 TFLOP/s of the sweep (total flop / total time),
per-shape TFLOP/s and GB/s with their roofline fractions, the roofline of the dominant kernel
measured with HIP events on the launch stream, the grouped (MoE) configurations, and the CPU
oracle timed on a bounded sample on the host's cores.
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

PEAK_FP8_TFLOPS = 5000.0       # MI355X dense FP8 MFMA (AMD published)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E (AMD published)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-grouped", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU-oracle sample time")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (--gpus %d requested)"
              % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import fp8_block_scaled_x128_amd as fg
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    fg.init()

    # ---- inputs: all 18 sweep cases resident on the device -----------------------------------
    t0 = time.time()
    cases = []
    b_cache = {}
    for nki, (N, K) in enumerate(W.SWEEP_NK):
        for mi, M in enumerate(W.SWEEP_M):
            a_seed, b_seed = W.sweep_seeds(mi, nki)
            if nki not in b_cache:
                rng_b = np.random.default_rng(b_seed)
                Bq, sbq = W.quantize_128x128(W.normal(rng_b, (N, K)))
                b_cache[nki] = (torch.from_numpy(Bq).to(dev), torch.from_numpy(sbq).to(dev), Bq, sbq)
            Bd, sbd, Bq, sbq = b_cache[nki]
            Aq, saq = W._acts(np.random.default_rng(a_seed), M, K)
            cases.append(dict(M=M, N=N, K=K, A=torch.from_numpy(Aq).to(dev),
                              sa=torch.from_numpy(np.ascontiguousarray(saq.T)).to(dev),
                              B=Bd, sb=sbd, D=torch.empty((M, N), dtype=torch.bfloat16, device=dev),
                              hostA=Aq, hostsa=saq, hostB=Bq, hostsb=sbq))
    # interleave M values so that no two consecutive GEMMs share a weight matrix
    order = sorted(range(len(cases)), key=lambda i: (W.SWEEP_M.index(cases[i]["M"]), i))
    cases = [cases[i] for i in order]
    log("inputs ready in %.1f s" % (time.time() - t0))

    stream = torch.cuda.current_stream(dev)

    def run_case(c):
        fg.gemm_nt(c["A"], c["sa"], c["B"], c["sb"], out=c["D"], stream=stream)

    configs = []
    for c in cases:
        run_case(c)
        configs.append(fg.last_config())
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        for c in cases:
            run_case(c)
    torch.cuda.synchronize()

    # ---- timed region: K steps, HIP events around every launch on the launch stream ----------
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in cases] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(args.steps):
        for i, c in enumerate(cases):
            ev[s][i][0].record(stream)
            run_case(c)
            ev[s][i][1].record(stream)
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    ms_per_step = 1e3 * t_total / args.steps

    per = []
    total_flop = 0
    kern_time = {}
    kern_flop = {}
    kern_bytes = {}
    for i, c in enumerate(cases):
        ms = float(np.mean([ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(args.steps)]))
        flop, byts = W.dense_work(c["M"], c["N"], c["K"])
        total_flop += flop
        tf = flop / (ms * 1e-3) / 1e12
        gbs = byts / (ms * 1e-3) / 1e9
        kname = configs[i].split(" split=")[0]
        kern_time[kname] = kern_time.get(kname, 0.0) + ms
        kern_flop[kname] = kern_flop.get(kname, 0) + flop
        kern_bytes[kname] = kern_bytes.get(kname, 0) + byts
        ai = flop / byts
        bound = "mfma" if ai * PEAK_HBM_GBS * 1e9 > PEAK_FP8_TFLOPS * 1e12 else "hbm"
        per.append(dict(M=c["M"], N=c["N"], K=c["K"], us=round(ms * 1e3, 2), tflops=round(tf, 1),
                        gbs=round(gbs, 1), frac_mfma=round(tf / PEAK_FP8_TFLOPS, 4),
                        frac_hbm=round(gbs / PEAK_HBM_GBS, 4), roof=bound, config=configs[i]))
    sum_kernel_ms = sum(p["us"] for p in per) / 1e3
    value = total_flop / (sum_kernel_ms * 1e-3) / 1e12

    dom = max(kern_time, key=kern_time.get)
    dom_launches = sum(1 for i in range(len(cases)) if configs[i].split(" split=")[0] == dom)
    dom_avg_us = kern_time[dom] / dom_launches * 1e3
    ach = kern_flop[dom] / (kern_time[dom] * 1e-3) / 1e12
    roofline = dict(bound="mfma", achieved=round(ach, 1), peak=PEAK_FP8_TFLOPS, unit="TFLOP/s",
                    frac=round(ach / PEAK_FP8_TFLOPS, 4), traffic=None, kernel=dom,
                    launches_per_step=dom_launches, avg_launch_us=round(dom_avg_us, 2),
                    flop_per_launch=kern_flop[dom] // dom_launches)

    # ---- grouped (MoE) configurations ----------------------------------------------------------
    grouped = {}
    if not args.no_grouped:
        grouped = bench_grouped(fg, W, torch, dev, stream)

    # ---- CPU oracle on a bounded sample of the same workload ----------------------------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cases, args.cpu_seconds)

    line = {
        "metric": "FP8 TFLOPS and HBM GB/s per shape (dense, contiguous, masked) on 1 MI355X",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3",
        "data": "synthetic: seeded N(0,1) fp32 quantised to e4m3 (A 1x128, B 128x128 fp32 scales)",
        "config": {"workload": "dense FP8 NT GEMM sweep, M in {64,128,4096} x (N,K) in "
                               "{(2112,7168),(24576,1536),(32768,512),(7168,16384),(4096,7168),(7168,2048)}, "
                               "18 GEMMs per step, bf16 out",
                   "gemms_per_step": len(cases), "flop_per_step": total_flop,
                   "kernel_ms_per_step": round(sum_kernel_ms, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "per_shape": per,
        "grouped": grouped,
    }
    print(json.dumps(line), flush=True)


def bench_grouped(fg, W, torch, dev, stream, reps=10):
    out = {}
    for name, make in (("contiguous_cfg2", W.config2), ("contiguous_cfg3", W.config3),
                       ("masked_cfg4", W.config4)):
        t0 = time.time()
        w = make()
        A, B, sb = (torch.from_numpy(x).to(dev) for x in (w.A, w.B, w.sb))
        sa = torch.from_numpy(np.ascontiguousarray(np.swapaxes(w.sa, -1, -2))).to(dev)  # K-block-major
        N, K = w.B.shape[1], w.B.shape[2]
        if name.startswith("contiguous"):
            idx = torch.from_numpy(w.m_indices).to(dev)
            D = torch.empty((w.A.shape[0], N), dtype=torch.bfloat16, device=dev)
            call = lambda: fg.grouped_contiguous(A, sa, B, sb, idx, out=D, stream=stream)
            counts = [int(np.sum(w.m_indices == g)) for g in range(w.B.shape[0])]
            flop, byts = W.grouped_work(counts, N, K, index_bytes=4 * w.A.shape[0])
        else:
            mm = torch.from_numpy(w.masked_m).to(dev)
            D = torch.empty((w.A.shape[0], w.A.shape[1], N), dtype=torch.bfloat16, device=dev)
            call = lambda: fg.grouped_masked(A, sa, B, sb, mm, w.expected_m, out=D, stream=stream)
            counts = [int(x) for x in w.masked_m]
            flop, byts = W.grouped_work(counts, N, K, index_bytes=4 * len(counts))
        call()
        cfg = fg.last_config()
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        es = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in es:
            e0.record(stream)
            call()
            e1.record(stream)
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in es]))
        tf = flop / (ms * 1e-3) / 1e12
        gbs = byts / (ms * 1e-3) / 1e9
        out[name] = dict(us=round(ms * 1e3, 1), tflops=round(tf, 1), gbs=round(gbs, 1),
                         frac_mfma=round(tf / PEAK_FP8_TFLOPS, 4), frac_hbm=round(gbs / PEAK_HBM_GBS, 4),
                         valid_rows=int(sum(counts)), config=cfg)
        log("%s: %.1f us, %.1f TFLOP/s, %.1f GB/s (%s) [inputs %.1f s]" % (name, ms * 1e3, tf, gbs, cfg,
                                                                            time.time() - t0))
        del A, sa, B, sb, D
        torch.cuda.empty_cache()
    return out


def cpu_baseline(cases, target_s):
    """The CPU oracle (as it stands) on rows 0..r-1 of every sweep case, r sized so the whole
    sample takes about target_s seconds on this host."""
    import oracle

    nth = oracle.num_threads(0)
    probe = cases[0]
    t0 = time.perf_counter()
    oracle.gemm_nt(probe["hostA"][:1], probe["hostsa"][:1], probe["hostB"], probe["hostsb"])
    t_probe = time.perf_counter() - t0
    per_row_all = t_probe * sum(c["N"] * c["K"] for c in cases) / (probe["N"] * probe["K"])
    rows = int(max(1, min(64, target_s / max(per_row_all, 1e-9))))
    flop = 0
    t0 = time.perf_counter()
    for c in cases:
        r = min(rows, c["M"])
        oracle.gemm_nt(c["hostA"][:r], c["hostsa"][:r], c["hostB"], c["hostsb"])
        flop += 2 * r * c["N"] * c["K"]
    dt = time.perf_counter() - t0
    log("cpu oracle: %d rows of each case, %.1f GFLOP in %.1f s on %d threads" % (rows, flop / 1e9, dt, nth))
    return dict(value=round(flop / dt / 1e12, 6), unit="TFLOP/s", cores=nth, kind="oracle",
                sample="first %d rows of each of the 18 sweep GEMMs (all N, all K), %.1f GFLOP, %.1f s"
                       % (rows, flop / 1e9, dt))


if __name__ == "__main__":
    main()
