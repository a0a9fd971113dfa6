"""Benchmark of the FP8 block-scaled GEMM on one MI355X.

One step = the dense decode/prefill sweep over DeepSeek-V3-like projection shapes: M in
{64, 128, 4096} x (N, K) in {(2112,7168), (24576,1536), (32768,512), (7168,16384), (4096,7168),
(7168,2048)} -- 18 GEMMs, each D[M,N] bf16 = A[M,K] e4m3 (1x128 fp32 scales) . B[N,K]^T e4m3
(128x128 fp32 scales).  Inputs are synthetic, seeded, quantised from N(0,1) and resident in HBM
before timing.

Launch path: each step's 18 library calls are captured once into a HIP graph (the launch
stream's split-K workspace is created first, by fp8gemm_prepare_stream, and never moves) and the
graph is replayed; R copies of every operand set rotate between steps and between the launches
of the per-shape graphs, so no GEMM finds its operands in the 256 MB last-level cache.
Graph outputs are checked bit for bit against eager calls before timing.

Prints ONE JSON line:
  value        aggregate FP8 TFLOP/s of the sweep = flop per step / wall-clock time per step
               (K graph replays between two device synchronisations)
  per_shape    per GEMM: average launch time from HIP events around per-shape graphs of R
               launches (on the launch stream), TFLOP/s, GB/s and roofline fractions
  roofline     the dominant kernel (largest share of the step's time): algorithmic flop per
               launch / average launch time, against the 5.0 PFLOP/s dense FP8 peak
  grouped      the contiguous and masked MoE configurations (context, not part of value)
  quantize_1x128  the bf16 -> E4M3 1x128 activation quantiser on the contiguous configuration's
               activations (32768 x 7168) and the masked decode configuration's, with its own
               HBM roofline (context, not part of value)
  moe_expert_chain  one DeepSeek-V3-sized MoE expert layer on the masked decode configuration's
               groups: first grouped GEMM, SwiGLU + requantisation, second grouped GEMM
               (context, not part of value)
  cpu_baseline the CPU oracle on a bounded sample of the same workload on this host's cores
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0       # MI355X dense FP8 MFMA (AMD published)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E (AMD published)
COPIES = 4                     # rotated operand copies


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-grouped", action="store_true")
    p.add_argument("--no-library-reference", action="store_true",
                   help="skip the context leg timing the vendor library's plain FP8 GEMM")
    p.add_argument("--cpu-seconds", type=float, default=20.0, help="target CPU-oracle sample time")
    p.add_argument("--counters", action="store_true",
                   help="launch every kernel the benchmark times (the 18 sweep GEMMs, the grouped "
                        "configurations, the quantiser) COUNTER_REPS times each, eagerly, then a 1 GiB copy "
                        "(run under rocprofv3 --pmc, one pass per counter group)")
    p.add_argument("--trace-summary", nargs=2, metavar=("TRACE_DIR", "BENCH_JSON"),
                   help="turn the rocprofv3 --kernel-trace output folder of a benchmark run and that run's "
                        "JSON line into profiles/kernel_stats_*_bench.txt (dispatches per leg by the leg markers)")
    p.add_argument("--counter-summary", nargs="+", metavar="PASS_DIR",
                   help="turn the rocprofv3 --pmc output folders of --counters runs (one per pass) into "
                        "the per-family summaries profiles/counters_*.txt and " + TRAFFIC_FILE)
    return p.parse_args()


TRAFFIC_FILE = os.path.join("profiles", "traffic_dense_256x256_m4096_sweep.txt")
COPY_BYTES = 1 << 30           # calibration copy: reads and writes this many bytes


KERNEL_SOURCES = ("fp8gemm_tiled.h", "fp8gemm_device.h", "fp8gemm_args.h", "fp8gemm_kernels.hip",
                  "stream_kernels.hip", "quantize_kernels.hip", "fp8gemm_internal.h")


def kernel_source_hash():
    """Hash of every source that makes a GPU kernel the counters and traces cover (the tiled
    kernel's body, helpers, argument block and instantiation table, the masked decode kernel and
    the quantisers), stamped into each profile summary."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, "fp8_block_scaled_x128_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def read_traffic():
    """Measured HBM traffic per launch of the dominant kernel from the committed counter summary,
    or None when there is none or the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, TRAFFIC_FILE)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith(" "):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return int(vals["traffic_bytes_per_launch"].split()[0])
    except (KeyError, ValueError):
        return None


COUNTER_FILES = ("counters_dense_prefill.txt", "counters_dense_decode.txt", "counters_grouped.txt",
                 "counters_quantize.txt")


def leg_key(label):
    """The key a counter summary's leg label and a benchmark leg share: 'dense 64x2112x7168',
    'contiguous cfg2', 'masked cfg4', 'masked fp8xfp4 cfg4', 'quantize_1x128 32768x7168'."""
    words = label.split()
    if words[0] == "dense" or words[0].startswith("quantize"):
        return " ".join(words[:2])
    return " ".join(w for w in words[:3] if not re.match(r"^\d+x\d+$", w))


def read_leg_traffic():
    """Measured HBM bytes per call of every leg in the committed counter summaries (calibrated
    FETCH_SIZE + WRITE_SIZE), keyed by leg_key; a summary taken on other kernel sources is
    skipped."""
    out = {}
    h = kernel_source_hash()
    for fname in COUNTER_FILES:
        path = os.path.join(ROOT, "profiles", fname)
        if not os.path.exists(path):
            continue
        lines = open(path).read().splitlines()
        if not any(l.startswith("kernel_source_sha256_16:") and l.split(":", 1)[1].strip() == h for l in lines):
            continue
        label = None
        for line in lines:
            if line and not line.startswith(" ") and "[" in line:
                label = line.split("[")[0].strip()
            m = re.search(r"hbm_MB ([0-9.]+)", line)
            if label and line.startswith("    derived:") and m:
                out[leg_key(label)] = int(float(m.group(1)) * 1e6)
    return out


def main():
    args = parse()
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.trace_summary:
        trace_summary(*args.trace_summary)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (--gpus %d requested)"
              % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import fp8_block_scaled_x128_amd as fg
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    fg.init()
    stream = torch.cuda.Stream(dev)
    fg.prepare_stream(stream)           # the split-K workspace, before any capture

    # ---- inputs: all 18 sweep cases resident on the device, COPIES copies each -----------------
    t0 = time.time()
    cases = []
    b_host = {}
    for nki, (N, K) in enumerate(W.SWEEP_NK):
        a_seed, b_seed = W.sweep_seeds(0, nki)
        rng_b = np.random.default_rng(b_seed)
        b_host[nki] = W.quantize_128x128(W.normal(rng_b, (N, K)))
    for mi, M in enumerate(W.SWEEP_M):          # M outer: consecutive GEMMs use other weights
        for nki, (N, K) in enumerate(W.SWEEP_NK):
            a_seed, _ = W.sweep_seeds(mi, nki)
            Aq, saq = W.acts(np.random.default_rng(a_seed), M, K)
            Bq, sbq = b_host[nki]
            base = dict(A=torch.from_numpy(Aq).to(dev),
                        sa=torch.from_numpy(np.ascontiguousarray(saq.T)).to(dev),   # [K/128, M]
                        B=torch.from_numpy(Bq).to(dev), sb=torch.from_numpy(sbq).to(dev))
            copies = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(COPIES - 1)]
            for c in copies:
                c["D"] = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            cases.append(dict(M=M, N=N, K=K, copies=copies, hostA=Aq, hostsa=saq, hostB=Bq, hostsb=sbq))
    torch.cuda.synchronize()            # operands (and their copies) are made on the default stream
    log("inputs ready in %.1f s" % (time.time() - t0))

    def call(case, r):
        c = case["copies"][r]
        fg.gemm_nt(c["A"], c["sa"], c["B"], c["sb"], out=c["D"], stream=stream)

    if args.counters:
        counters_run(fg, W, torch, dev, stream, cases, call)
        return

    # ---- eager reference outputs and launch configurations ------------------------------------
    mark_leg(torch, stream, "sweep")
    launch_cfgs = []
    with torch.cuda.stream(stream):
        for case in cases:
            for r in range(COPIES):
                call(case, r)
            launch_cfgs.append(fg.last_config())
    stream.synchronize()
    eager = [[c["D"].clone() for c in case["copies"]] for case in cases]

    # ---- graphs: one per step copy, one per shape (COPIES launches) --------------------------
    step_graphs = []
    for r in range(COPIES):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for case in cases:
                call(case, r)
        step_graphs.append(g)
    shape_graphs = []
    for case in cases:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for r in range(COPIES):
                call(case, r)
        shape_graphs.append(g)

    def replay(g):
        with torch.cuda.stream(stream):
            g.replay()

    # graph replays must reproduce the eager outputs bit for bit
    for case in cases:
        for c in case["copies"]:
            c["D"].zero_()
    for r in range(COPIES):
        replay(step_graphs[r])
    stream.synchronize()
    for i, case in enumerate(cases):
        for r in range(COPIES):
            if not torch.equal(case["copies"][r]["D"], eager[i][r]):
                raise RuntimeError("graph replay differs from eager output (case %d copy %d)" % (i, r))

    flush = torch.ones(256 * 1024 * 1024, dtype=torch.float32, device=dev)    # 1 GiB, read only
    sink = torch.zeros(1, device=dev)

    def read_flush():
        with torch.cuda.stream(stream):
            sink.add_(flush.sum())

    # ---- timed region: K steps --------------------------------------------------------------
    for s in range(args.warmup):
        replay(step_graphs[s % COPIES])
    stream.synchronize()
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    e_start.record(stream)
    for s in range(args.steps):
        replay(step_graphs[s % COPIES])
    e_end.record(stream)
    stream.synchronize()
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    ms_per_step = 1e3 * t_total / args.steps
    gpu_ms_per_step = e_start.elapsed_time(e_end) / args.steps
    gpu_state = sample_gpu_state()          # right after the timed steps, the part still warm

    # ---- per-shape launch times: HIP events around per-shape graphs on the launch stream -------
    reps = 5
    per = []
    total_flop = 0
    kern_time, kern_flop, kern_launch = {}, {}, {}
    # one untimed pass over every shape first: whichever shape is timed first after the step loop
    # measures slow (20 against 14 us on 64x2112x7168, 89 against 77 us on 4096x7168x2048)
    mark_leg(torch, stream, "sweep_per_shape")
    for i in range(len(cases)):
        read_flush()
        replay(shape_graphs[i])
    stream.synchronize()
    for i, case in enumerate(cases):
        ts = []
        for _ in range(reps):
            read_flush()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            replay(shape_graphs[i])
            e1.record(stream)
            stream.synchronize()
            ts.append(e0.elapsed_time(e1) / COPIES)
        ms = float(np.mean(ts))
        flop, byts = W.dense_work(case["M"], case["N"], case["K"])
        total_flop += flop
        tf = flop / (ms * 1e-3) / 1e12
        gbs = byts / (ms * 1e-3) / 1e9
        kname = launch_cfgs[i].split(" split=")[0]
        kern_time[kname] = kern_time.get(kname, 0.0) + ms
        kern_flop[kname] = kern_flop.get(kname, 0) + flop
        kern_launch[kname] = kern_launch.get(kname, 0) + 1
        bound = "mfma" if flop / byts * PEAK_HBM_GBS * 1e9 > PEAK_FP8_TFLOPS * 1e12 else "hbm"
        per.append(dict(M=case["M"], N=case["N"], K=case["K"], us=round(ms * 1e3, 2), tflops=round(tf, 1),
                        gbs=round(gbs, 1), frac_mfma=round(tf / PEAK_FP8_TFLOPS, 4),
                        frac_hbm=round(gbs / PEAK_HBM_GBS, 4), roof=bound, config=launch_cfgs[i]))
    value = total_flop / (ms_per_step * 1e-3) / 1e12

    dom = max(kern_time, key=kern_time.get)
    ach = kern_flop[dom] / (kern_time[dom] * 1e-3) / 1e12
    traffic = read_traffic() if dom.startswith("nt tile=256x256") else None
    roofline = dict(bound="mfma", achieved=round(ach, 1), peak=PEAK_FP8_TFLOPS, unit="TFLOP/s",
                    frac=round(ach / PEAK_FP8_TFLOPS, 4), traffic=traffic, kernel=dom,
                    launches_per_step=kern_launch[dom],
                    avg_launch_us=round(kern_time[dom] / kern_launch[dom] * 1e3, 2),
                    flop_per_launch=kern_flop[dom] // kern_launch[dom],
                    share_of_step=round(kern_time[dom] / sum(kern_time.values()), 3))

    read_floor = bench_read_floor(torch, dev, stream, per, read_flush, reps)
    library = {} if args.no_library_reference else bench_library_reference(torch, dev, stream, per, read_flush, reps)
    specialized = bench_specialized(fg, torch, stream, cases, per, replay, read_flush, reps)

    grouped = {}
    if not args.no_grouped:
        del flush
        grouped = bench_grouped(fg, W, torch, dev, stream, cpu=not args.no_cpu_baseline)
    quantize = bench_quantize(fg, W, torch, dev, stream)
    moe = {} if args.no_grouped else bench_moe_chain(fg, W, torch, dev, stream, cpu=not args.no_cpu_baseline)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cases, eager, args.cpu_seconds)

    # measured HBM bytes per call of each leg, from the committed counter summaries of the same
    # kernel sources (None where there is none)
    leg_traffic = read_leg_traffic()
    for q in per:
        q["traffic"] = leg_traffic.get("dense %dx%dx%d" % (q["M"], q["N"], q["K"]))
    for name, g in grouped.items():
        g["traffic"] = leg_traffic.get(name.replace("_", " "))
    if "dense_32768x7168" in quantize:
        quantize["dense_32768x7168"]["roofline"]["traffic"] = leg_traffic.get("quantize_1x128 32768x7168")

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
                   "gpu_ms_per_step": round(gpu_ms_per_step, 4), "launch": "hip graph replay",
                   "operand_copies": COPIES},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "per_shape": per,
        "grouped": grouped,
        "quantize_1x128": quantize,
        "moe_expert_chain": moe,
        "specialized": specialized,
        "read_floor": read_floor,
        "library_reference": library,
        "gpu_state": gpu_state,
        "traffic_note": "traffic: HBM bytes per call (calibrated FETCH_SIZE + WRITE_SIZE) from profiles/counters_*.txt "
                        "taken on the same kernel sources; null where none match",
    }
    print(json.dumps(line), flush=True)


COUNTER_REPS = 3
# kernels of the library, as rocprofv3 names their dispatches
LIB_KERNELS = ("fp8gemm_kernel", "fp8gemm_masked_decode_kernel", "quantize_1x128_kernel")


def counter_legs():
    """(label, family, flop, bytes) of every leg of a --counters run, in launch order: the 18 sweep
    GEMMs, the grouped configurations 2, 3, 4 and 4 with MXFP4 weights, the activation quantiser
    (32768 x 7168).  Each leg is launched COUNTER_REPS times."""
    import workloads as W
    legs = []
    for M in W.SWEEP_M:
        for N, K in W.SWEEP_NK:
            flop, byts = W.dense_work(M, N, K)
            legs.append(("dense %dx%dx%d" % (M, N, K), "dense_decode" if M <= 128 else "dense_prefill", flop, byts))
    c2 = [7782] * 4
    legs.append(("contiguous cfg2 4x8192 N=4096 K=7168", "grouped") + W.grouped_work(c2, 4096, 7168, 4 * 32768))
    c3 = W.config3_counts()
    legs.append(("contiguous cfg3 8x4096 N=7168 K=2048", "grouped") + W.grouped_work(c3, 7168, 2048, 4 * 32768))
    c4 = [int(x) for x in W.config4_masked_m()]
    legs.append(("masked cfg4 16x256 N=4096 K=7168", "grouped") + W.grouped_work(c4, 4096, 7168, 4 * 16))
    legs.append(("masked fp8xfp4 cfg4 16x256 N=4096 K=7168", "grouped") +
                W.grouped_fp4_work(c4, 4096, 7168, 4 * 16))
    legs.append(("quantize_1x128 32768x7168", "quantize", 0, W.quantize_work(W.QUANT_M, W.QUANT_K)))
    return legs


def counters_run(fg, W, torch, dev, stream, cases, call):
    """Eager launches for hardware-counter passes: every leg of counter_legs() COUNTER_REPS times,
    each after a read-only cache flush (a reduction), then an elementwise copy (dst = src + 0) of
    COPY_BYTES COUNTER_REPS times, the calibration of the traffic counters.  Prints the launch
    order with each launch's configuration."""
    flush = torch.ones(256 * 1024 * 1024, dtype=torch.float32, device=dev)
    sink = torch.zeros((), device=dev)
    order = []

    def run(label, f):
        for r in range(COUNTER_REPS):
            torch.sum(flush, dim=0, out=sink)   # read-only flush: a reduction, no elementwise kernel
            f(r)
            order.append((label, fg.last_config()))

    with torch.cuda.stream(stream):
        for case in cases:
            run("dense %dx%dx%d" % (case["M"], case["N"], case["K"]), lambda r, case=case: call(case, r % COPIES))
    stream.synchronize()
    for label, make in (("contiguous cfg2 4x8192 N=4096 K=7168", W.config2),
                        ("contiguous cfg3 8x4096 N=7168 K=2048", W.config3),
                        ("masked cfg4 16x256 N=4096 K=7168", W.config4),
                        ("masked fp8xfp4 cfg4 16x256 N=4096 K=7168", W.config4_fp4)):
        w = make()
        A, B, sb = (torch.from_numpy(x).to(dev) for x in (w.A, w.B, w.sb))
        sa = torch.from_numpy(np.ascontiguousarray(np.swapaxes(w.sa, -1, -2))).to(dev)
        N = w.B.shape[1]
        with torch.cuda.stream(stream):
            if label.startswith("contiguous"):
                idx = torch.from_numpy(w.m_indices).to(dev)
                D = torch.empty((w.A.shape[0], N), dtype=torch.bfloat16, device=dev)
                run(label, lambda r: fg.grouped_contiguous(A, sa, B, sb, idx, out=D, stream=stream))
            else:
                mm = torch.from_numpy(w.masked_m).to(dev)
                D = torch.empty((w.A.shape[0], w.A.shape[1], N), dtype=torch.bfloat16, device=dev)
                f = fg.fp8fp4_grouped_masked if "fp8xfp4" in label else fg.grouped_masked
                run(label, lambda r: f(A, sa, B, sb, mm, w.expected_m, out=D, stream=stream))
        stream.synchronize()
        del A, B, sb, sa, D, w
        torch.cuda.empty_cache()
    bits = W.activations_bf16(W.QUANT_M, W.QUANT_K, seed=31)
    X = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
    codes = torch.empty((W.QUANT_M, W.QUANT_K), dtype=torch.float8_e4m3fn, device=dev)
    scales = torch.empty((W.QUANT_K // 128, W.QUANT_M), dtype=torch.float32, device=dev)
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    with torch.cuda.stream(stream):
        run("quantize_1x128 32768x7168", lambda r: fg.quantize_1x128(X, codes=codes, scales=scales, stream=stream))
        # the calibration copy: the last elementwise kernels of the run (read and write COPY_BYTES)
        for r in range(COUNTER_REPS):
            torch.add(src, 0.0, out=dst)
            order.append(("copy %d" % COPY_BYTES, ""))
    stream.synchronize()
    print(json.dumps({"counter_launches": order}), flush=True)


def _pass_rows(folder):
    """{dispatch id: (kernel name, {counter: value})} from one rocprofv3 --pmc csv output folder
    (values summed over the dimensions rocprofv3 reports them in; GRBM counters, which count
    cycles per XCD, take the maximum instead)."""
    import csv
    import glob
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % folder)
    per = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            key = int(r["Dispatch_Id"])
            name, vals = per.setdefault(key, (r["Kernel_Name"], {}))
            c, v = r["Counter_Name"], float(r["Counter_Value"])
            vals[c] = max(vals.get(c, v), v) if c.startswith("GRBM_") else vals.get(c, 0.0) + v
    return per


def _short_kernel(name):
    for k in LIB_KERNELS:
        if k in name:
            i = name.index(k)
            j = name.find(">", i)
            return name[i:j + 1] if j > 0 else k
    return name


def counter_summary(folders):
    """Per leg of counter_legs(): the median over its COUNTER_REPS dispatches of every counter the
    passes collected, with derived figures where the counters allow:
      HBM traffic  = FETCH_SIZE and WRITE_SIZE (KiB) scaled by what they count for the calibration
                     copy of COPY_BYTES, against the leg's algorithmic bytes;
      MFMA busy    = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x CUs x 4 SIMDs);
      FP8 MFMA work = SQ_INSTS_VALU_MFMA_MOPS_F8 x 512 flop, against the leg's algorithmic flop;
      wait share   = SQ_WAIT_ANY / SQ_WAVE_CYCLES; TA busy = TA_BUSY_avr / GRBM_GUI_ACTIVE.
    Writes profiles/counters_<family>.txt per family and the dominant kernel's traffic file."""
    legs = counter_legs()
    lib, copies = [], []
    merged = {}
    for folder in folders:
        for key, (name, vals) in _pass_rows(folder).items():
            m = merged.setdefault(key, [name, {}])
            m[1].update(vals)
    for key in sorted(merged):
        name, vals = merged[key]
        if any(k in name for k in LIB_KERNELS):
            lib.append((name, vals))
        elif "elementwise" in name.lower():
            copies.append(vals)
    if len(lib) != COUNTER_REPS * len(legs):
        raise SystemExit("%d library dispatches found, %d expected" % (len(lib), COUNTER_REPS * len(legs)))
    cal = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        v = [x[c] for x in copies[-COUNTER_REPS:] if c in x]
        if v:
            cal[c] = COPY_BYTES / (float(np.median(v)) * 1024.0)
    cus = 256
    rows = []
    for i, (label, family, flop, byts) in enumerate(legs):
        part = lib[i * COUNTER_REPS:(i + 1) * COUNTER_REPS]
        names = {n for n, _ in part}
        med = {c: float(np.median([v[c] for _, v in part if c in v])) for c in part[0][1]}
        d = {}
        if "FETCH_SIZE" in med and "WRITE_SIZE" in med and len(cal) == 2:
            t = med["FETCH_SIZE"] * 1024 * cal["FETCH_SIZE"] + med["WRITE_SIZE"] * 1024 * cal["WRITE_SIZE"]
            d["hbm_MB"] = t / 1e6
            d["alg_MB"] = byts / 1e6
            d["hbm/alg"] = t / byts
        gui = med.get("GRBM_GUI_ACTIVE")
        if "MfmaUtil" in med:
            d["mfma_busy"] = med["MfmaUtil"] / 100.0
        elif "SQ_VALU_MFMA_BUSY_CYCLES" in med and gui:
            d["mfma_busy"] = med["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * cus * 4)
        if "SQ_INSTS_VALU_MFMA_MOPS_F8" in med and flop:
            d["mfma_flop/alg"] = med["SQ_INSTS_VALU_MFMA_MOPS_F8"] * 512 / flop
        if med.get("SQ_WAVE_CYCLES") and "SQ_WAIT_ANY" in med:
            d["wait_share"] = med["SQ_WAIT_ANY"] / med["SQ_WAVE_CYCLES"]
        if gui and "TA_BUSY_avr" in med:
            d["ta_busy"] = med["TA_BUSY_avr"] / gui
        if gui and "TD_BUSY_avr" in med:
            d["td_busy"] = med["TD_BUSY_avr"] / gui
        if gui and "SQ_LDS_IDX_ACTIVE" in med:
            d["lds_active"] = med["SQ_LDS_IDX_ACTIVE"] / (gui * cus)
        if gui and "SQ_LDS_BANK_CONFLICT" in med:
            d["lds_bank_conflict"] = med["SQ_LDS_BANK_CONFLICT"] / (gui * cus)
        if "VALUBusy" in med:
            d["valu_busy"] = med["VALUBusy"] / 100.0
        rows.append((label, family, sorted(_short_kernel(n) for n in names), med, d, byts))
    src = kernel_source_hash()
    for family in sorted({r[1] for r in rows}):
        path = os.path.join(ROOT, "profiles", "counters_%s.txt" % family)
        with open(path, "w") as f:
            f.write("Hardware counters of the %s legs (rocprofv3 --pmc; median of %d eager launches per leg, each "
                    "after a read-only 1 GiB buffer read)\n" % (family.replace("_", " "), COUNTER_REPS))
            f.write("command (one per counter group): rocprofv3 --pmc <counters> --output-format csv -d <dir> "
                    "-- python3 bench.py --counters\n")
            f.write("summary: python3 bench.py --counter-summary <dir> [<dir> ...]\n")
            f.write("kernel_source_sha256_16: %s\n" % src)
            for c, fct in sorted(cal.items()):
                f.write("%s calibration: factor %.4f (bytes of a %d-byte copy / bytes counted)\n" % (c, fct, COPY_BYTES))
            f.write("derived (GRBM_GUI_ACTIVE: cycles of the busiest XCD): hbm = calibrated FETCH_SIZE + WRITE_SIZE; "
                    "mfma_busy = MfmaUtil / 100 (MFMA busy cycles over all SIMDs / (GRBM_GUI_ACTIVE x SIMDs)); "
                    "mfma_flop/alg = SQ_INSTS_VALU_MFMA_MOPS_F8 x 512 / algorithmic flop; wait_share = SQ_WAIT_ANY / "
                    "SQ_WAVE_CYCLES; ta_busy, td_busy = TA_BUSY_avr, TD_BUSY_avr / GRBM_GUI_ACTIVE; lds_active, "
                    "lds_bank_conflict = SQ_LDS_IDX_ACTIVE, SQ_LDS_BANK_CONFLICT / (GRBM_GUI_ACTIVE x %d CUs); "
                    "valu_busy = VALUBusy / 100\n" % cus)
            for label, fam, kern, med, d, byts in rows:
                if fam != family:
                    continue
                f.write("%s  [%s]\n" % (label, ", ".join(kern)))
                f.write("    derived: %s\n" % "  ".join("%s %.3f" % (k, v) for k, v in d.items()))
                f.write("    raw: %s\n" % "  ".join("%s %.6g" % (k, v) for k, v in sorted(med.items())))
        print(open(path).read())
    # the dominant kernel's traffic per launch (read by the benchmark's roofline.traffic)
    dom = [r for r in rows if r[2] == [DOMINANT_KERNEL] and "hbm_MB" in r[4]]
    if dom:
        per_launch = int(round(np.mean([r[4]["hbm_MB"] for r in dom]) * 1e6))
        with open(os.path.join(ROOT, TRAFFIC_FILE), "w") as f:
            f.write("HBM traffic of the dense 256x256 kernel on the M=4096 sweep shapes (rocprofv3 --pmc)\n")
            f.write("command (per counter): rocprofv3 --pmc <FETCH_SIZE | WRITE_SIZE> --output-format csv -d <dir> "
                    "-- python3 bench.py --counters\n")
            f.write("summary: python3 bench.py --counter-summary <dir> [<dir> ...]\n")
            f.write("kernel_source_sha256_16: %s\n" % src)
            for c, fct in sorted(cal.items()):
                f.write("%s_copy_calibration: factor %.4f\n" % (c, fct))
            for r in dom:
                f.write("  %-28s traffic %7.1f MB  algorithmic %6.1f MB  ratio %.2f\n"
                        % (r[0], r[4]["hbm_MB"], r[4]["alg_MB"], r[4]["hbm/alg"]))
            f.write("traffic_bytes_per_launch: %d   (mean over the %d shapes run by %s)\n"
                    % (per_launch, len(dom), DOMINANT_KERNEL))
        print(open(os.path.join(ROOT, TRAFFIC_FILE)).read())


DOMINANT_KERNEL = "fp8gemm_kernel<256, 256, 4, 2, 2, 0, 0, 0>"


READ_WGS = (256, 512, 1024, 2048)
READ_DEPTHS = (8, 16)


def bench_read_floor(torch, dev, stream, per, read_flush, reps):
    """The read floor of every decode-sized sweep GEMM (M <= 128): a plain streaming read
    (libreadprobe.so: contiguous 16-byte loads, 8 or 16 in flight per thread, 256-2048
    workgroups, the best of these) of the GEMM's algorithmic byte count, timed like the GEMMs:
    HIP events on the launch stream around a graph of COPIES launches that each read another
    buffer copy, after a read-only 1 GiB buffer read.  Adds read_floor_us and frac_read_floor
    (read time / GEMM time) to the per-shape rows."""
    import ctypes
    lib = probe_lib()
    rows = [p for p in per if p["M"] <= 128]
    if not rows:
        return {}
    nbytes = [(-(-W_bytes(p) // 16)) * 16 for p in rows]
    bufs = [torch.empty(max(nbytes), dtype=torch.uint8, device=dev) for _ in range(COPIES)]
    for b in bufs:
        b.fill_(1)
    sink = torch.zeros(max(READ_WGS), dtype=torch.int32, device=dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    t0 = time.time()
    out = []
    mark_leg(torch, stream, "read_floor")
    for p, nb in zip(rows, nbytes):
        best = None
        for wgs in READ_WGS:
            for depth in READ_DEPTHS:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    for b in bufs:
                        if lib.read_probe(b.data_ptr(), nb, wgs, depth, sink.data_ptr(), sp) != 0:
                            raise RuntimeError("read_probe launch failed")
                replay_on(stream, g)
                stream.synchronize()
                ts = []
                for _ in range(reps):
                    read_flush()
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    replay_on(stream, g)
                    e1.record(stream)
                    stream.synchronize()
                    ts.append(e0.elapsed_time(e1) / COPIES)
                us = float(np.mean(ts)) * 1e3
                if best is None or us < best[0]:
                    best = (us, wgs, depth)
                del g
        p["read_floor_us"] = round(best[0], 2)
        p["frac_read_floor"] = round(best[0] / p["us"], 4)
        out.append(dict(M=p["M"], N=p["N"], K=p["K"], bytes=nb, read_us=round(best[0], 2),
                        read_frac_hbm=round(nb / (best[0] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                        gemm_us=p["us"], frac_read_floor=p["frac_read_floor"], wgs=best[1], depth=best[2]))
    log("read floor of %d decode shapes in %.1f s: GEMM time / read time %s" % (
        len(rows), time.time() - t0, " ".join("%.2f" % (1.0 / r["frac_read_floor"]) for r in out)))
    del bufs
    return dict(method="plain streaming read of each shape's algorithmic bytes (best of %s workgroups x %s "
                       "loads in flight), timed as the GEMMs" % (list(READ_WGS), list(READ_DEPTHS)),
                per_shape=out)


def _kernel_label(name):
    """A dispatch's kernel name without its return type and trailing parameter list."""
    name = name.strip()
    if name.startswith("void "):
        name = name[5:]
    if name.endswith(")"):
        depth = 0
        for i in range(len(name) - 1, -1, -1):
            depth += {")": 1, "(": -1}.get(name[i], 0)
            if depth == 0:
                return name[:i].rstrip()
    return name


def trace_dispatches(folder):
    """[(start ns, end ns, kernel label, workgroups)] of every dispatch in one rocprofv3
    --kernel-trace csv output folder, in start order."""
    import csv
    import glob
    files = glob.glob(os.path.join(folder, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit("no kernel_trace.csv under %s" % folder)
    out = []
    for f in files:
        for r in csv.DictReader(open(f)):
            grid = int(r.get("Grid_Size_X") or r.get("Grid_Size") or 0)
            wg = max(1, int(r.get("Workgroup_Size_X") or r.get("Workgroup_Size") or 1))
            # grid in work-items (a multiple of the workgroup size), else already in workgroups
            wgs = grid // wg if grid >= wg and grid % wg == 0 else grid
            out.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), _kernel_label(r["Kernel_Name"]), wgs))
    out.sort()
    return out


def legs_of(dispatches):
    """{leg: [(label, duration us)]} of the library dispatches (kernels in namespace fp8gemm),
    attributed to the leg of the last marker before them (mark_leg)."""
    legs = {}
    cur = None
    for t0, t1, label, wgs in dispatches:
        if label.endswith("read_probe_kernel<4>") and 1 <= wgs <= len(LEGS):
            cur = LEGS[wgs - 1]
            legs.setdefault(cur, [])
        elif cur is not None and label.startswith("fp8gemm::"):
            legs[cur].append((label, (t1 - t0) * 1e-3))
    return legs


def _stats(ds):
    a = np.array(ds, dtype=np.float64)
    return len(a), float(a.mean()), float(a.min()), float(a.max()), float(a.sum())


TRACE_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run -- "
             "python3 bench.py --steps 5 --warmup 2 > <bench json>")
TRACE_SUMMARY_CMD = "python3 bench.py --trace-summary <dir> <bench json>"


def trace_summary(folder, bench_json):
    """Kernel durations per leg of a benchmark run under rocprofv3 --kernel-trace, beside the
    run's own HIP-event figures (its JSON line): writes profiles/kernel_stats_dense_sweep_bench.txt
    (the sweep's kernels, and the dominant kernel's rocprofv3 average against the benchmark's
    avg_launch_us), profiles/kernel_stats_grouped_moe_bench.txt and
    profiles/kernel_stats_quantize_1x128_bench.txt."""
    line = None
    for ln in open(bench_json):
        ln = ln.strip()
        if ln.startswith("{"):
            line = json.loads(ln)
    if line is None:
        raise SystemExit("no JSON line in %s" % bench_json)
    legs = legs_of(trace_dispatches(folder))
    missing = [l for l in LEGS if l not in legs]
    if missing:
        raise SystemExit("the trace has no marker for legs %s" % missing)
    head = ("command: %s\nsummary: %s\nsource hash of the kernels: %s\n"
            % (TRACE_CMD, TRACE_SUMMARY_CMD, kernel_source_hash()))

    def table(rows):
        by = {}
        for label, us in rows:
            by.setdefault(label, []).append(us)
        out = ["%-78s %6s %10s %10s %10s %12s" % ("kernel", "calls", "avg us", "min us", "max us", "total us")]
        for label, ds in sorted(by.items(), key=lambda kv: -sum(kv[1])):
            n, avg, mn, mx, tot = _stats(ds)
            out.append("%-78s %6d %10.2f %10.2f %10.2f %12.1f" % (label, n, avg, mn, mx, tot))
        return "\n".join(out) + "\n"

    # ---- dense sweep ---------------------------------------------------------------------------
    rf = line["roofline"]
    dom = "fp8gemm::" + DOMINANT_KERNEL
    if not rf["kernel"].startswith("nt tile=256x256 waves=4x2 stages=2"):
        raise SystemExit("the run's dominant kernel (%s) is not %s" % (rf["kernel"], DOMINANT_KERNEL))
    timed = [us for label, us in legs["sweep_per_shape"] if label == dom]
    everywhere = [us for leg in ("sweep", "sweep_per_shape") for label, us in legs[leg] if label == dom]
    with open(os.path.join(ROOT, "profiles", "kernel_stats_dense_sweep_bench.txt"), "w") as f:
        f.write("Kernel durations of the dense sweep legs of one benchmark run (rocprofv3 --kernel-trace --stats)\n")
        f.write(head)
        f.write("workload: the 18-GEMM dense sweep (M in {64,128,4096} x (N,K) in {(2112,7168),(24576,1536),"
                "(32768,512),(7168,16384),(4096,7168),(7168,2048)}); template arguments BM, BN, waves M, waves N,\n"
                "stages, layout (0 dense), N, K (N and K nonzero: the kernels specialised at run time).\n\n")
        for leg, what in (("sweep", "eager reference calls, graph checks, warm-up and the timed steps (graph replays)"),
                          ("sweep_per_shape", "per-shape graphs of 4 launches: one untimed pass, then 5 timed"),
                          ("specialized", "the same shapes with the kernels specialised to N and K")):
            f.write("leg %s: %s\n" % (leg, what))
            f.write(table(legs[leg]) + "\n")
        n, avg, mn, mx, _ = _stats(timed)
        f.write("dominant kernel %s (%s):\n" % (DOMINANT_KERNEL, rf["kernel"]))
        f.write("  rocprofv3, per-shape leg: %d dispatches, average %.2f us (min %.2f, max %.2f)\n" % (n, avg, mn, mx))
        n2, avg2, _, _, _ = _stats(everywhere)
        f.write("  rocprofv3, every sweep dispatch of it: %d, average %.2f us\n" % (n2, avg2))
        f.write("  bench.py, same run (HIP events around the per-shape graphs): avg_launch_us %.2f over %d launches "
                "per step, achieved %.1f TFLOP/s (frac %.4f of %.0f)\n"
                % (rf["avg_launch_us"], rf["launches_per_step"], rf["achieved"], rf["frac"], rf["peak"]))
        f.write("  ratio bench / rocprofv3 (per-shape leg): %.4f\n" % (rf["avg_launch_us"] / avg))
        f.write("\nper-shape figures of the same run (bench.py):\n")
        for p in line["per_shape"]:
            f.write("  %5d x %5d x %5d  %8.2f us  %7.1f TFLOP/s  %7.1f GB/s  %s\n"
                    % (p["M"], p["N"], p["K"], p["us"], p["tflops"], p["gbs"], p["config"]))
    # ---- grouped, MoE and quantiser legs ------------------------------------------------------------
    bench_us = {}
    for k, v in (line.get("grouped") or {}).items():
        bench_us[k] = (v["us"], v["config"])
    for k, v in (line.get("moe_expert_chain") or {}).items():
        bench_us["moe_" + k] = (v["us"], v["config"])
    for k, v in (line.get("quantize_1x128") or {}).items():
        bench_us["quantize_" + k] = (v["us"], v["config"])
    for fname, title, names in (
            ("kernel_stats_grouped_moe_bench.txt", "the grouped, FP8 x FP4 and MoE-chain legs",
             ("contiguous_cfg2", "contiguous_cfg3", "masked_cfg4", "masked_fp8xfp4_cfg4", "moe_chain",
              "moe_first_layer", "moe_swiglu_quantize", "moe_second_layer")),
            ("kernel_stats_quantize_1x128_bench.txt", "the 1x128 activation quantiser legs",
             ("quantize_dense_32768x7168", "quantize_masked_16x256x7168"))):
        with open(os.path.join(ROOT, "profiles", fname), "w") as f:
            f.write("Kernel durations of %s of one benchmark run (rocprofv3 --kernel-trace --stats)\n" % title)
            f.write(head)
            f.write("per leg: every library dispatch after the leg's marker (the leg's first eager call, then its "
                    "graph: one untimed replay and the timed ones); bench us = the same run's HIP-event time per "
                    "call.\n\n")
            for leg in names:
                us, cfg = bench_us.get(leg, (float("nan"), ""))
                f.write("leg %s: bench %.2f us per call (%s)\n" % (leg, us, cfg))
                f.write(table(legs[leg]) + "\n")
    print("wrote profiles/kernel_stats_{dense_sweep,grouped_moe,quantize_1x128}_bench.txt; dominant kernel: "
          "rocprofv3 %.2f us, bench %.2f us" % (avg, rf["avg_launch_us"]))


def sample_gpu_state():
    """Shader and memory clocks, power and temperature as rocm-smi reports them (one sample, taken
    by the caller right after a timed region), or the reason there is none.  Context only: under a
    matrix-core load the shader clock sits below the 2.4 GHz behind the published peaks."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--showpower", "--showtemp", "--json"],
                           capture_output=True, text=True, timeout=30)
        data = json.loads(r.stdout)
    except Exception as e:      # no tool, no JSON, or a time-out: the benchmark goes on without it
        return {"unavailable": str(e)[:200]}
    out = {}
    for card, vals in data.items():
        if not isinstance(vals, dict):
            continue
        keep = {k.strip(" :"): v for k, v in vals.items()
                if any(w in k.lower() for w in ("sclk", "mclk", "fclk", "power", "temperature"))}
        if keep:
            out[card] = keep
    return out or {"unavailable": "rocm-smi printed no clock, power or temperature fields"}


_PROBE = {}


def probe_lib():
    """libreadprobe.so (the streaming-read kernel of the read floor and of the leg markers)."""
    import ctypes
    if "lib" not in _PROBE:
        lib = ctypes.CDLL(os.path.join(ROOT, "fp8_block_scaled_x128_amd", "libreadprobe.so"))
        lib.read_probe.restype = ctypes.c_int
        lib.read_probe.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.c_void_p]
        _PROBE["lib"] = lib
    return _PROBE["lib"]


# the benchmark's legs in run order; mark_leg puts the start of each into a kernel trace
LEGS = ("sweep", "sweep_per_shape", "read_floor", "specialized", "contiguous_cfg2", "contiguous_cfg3",
        "masked_cfg4", "masked_fp8xfp4_cfg4", "quantize_dense_32768x7168", "quantize_masked_16x256x7168",
        "moe_chain", "moe_first_layer", "moe_swiglu_quantize", "moe_second_layer", "moe_setup",
        "library_reference")


def mark_leg(torch, stream, name):
    """Mark the start of leg `name` in a kernel trace: one read_probe launch on the launch stream,
    4 loads deep (the read floor uses 8 and 16), with (leg number + 1) workgroups, that reads 16
    bytes.  Every library dispatch after it (in start order) belongs to its leg."""
    import ctypes
    if "buf" not in _PROBE:
        _PROBE["buf"] = torch.zeros(64, dtype=torch.int32, device=torch.device("cuda", torch.cuda.current_device()))
    buf = _PROBE["buf"]
    rc = probe_lib().read_probe(buf.data_ptr(), 16, LEGS.index(name) + 1, 4, buf[16:].data_ptr(),
                                ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise RuntimeError("leg marker launch failed")


def bench_library_reference(torch, dev, stream, per, read_flush, reps):
    """Context, not part of value: the vendor library's plain FP8 GEMM (torch._scaled_mm, served by
    hipBLASLt) on the prefill shapes (M >= 1024), with one fp32 scale per tensor and with one per
    row of A and column of B, timed as the sweep GEMMs (HIP events on the launch stream around a
    graph of COPIES launches on rotated operand copies, after a read-only 1 GiB buffer read).  It
    computes a coarser-scaled product -- no 128-wide K blocks, no per-block promotion -- so it is
    a ceiling for what this machine's matrix cores reach on an FP8 GEMM of the same shape, not
    the same operation.  Operands are random E4M3 values; outputs are not compared."""
    rows = [p for p in per if p["M"] >= 1024]
    out = []
    t0 = time.time()
    mark_leg(torch, stream, "library_reference")
    for p in rows:
        M, N, K = p["M"], p["N"], p["K"]
        g = torch.Generator(device=dev).manual_seed(M + N + K)
        ops = [((torch.randn(M, K, device=dev, generator=g) * 0.5).to(torch.float8_e4m3fn),
                (torch.randn(N, K, device=dev, generator=g) * 0.5).to(torch.float8_e4m3fn)) for _ in range(COPIES)]
        one = torch.ones((), device=dev)
        sa_row, sb_col = torch.ones(M, 1, device=dev), torch.ones(1, N, device=dev)
        torch.cuda.synchronize()
        row = dict(M=M, N=N, K=K, us_this=p["us"])
        for kind, sa, sb in (("per_tensor", one, one), ("per_row_col", sa_row, sb_col)):
            def call(r, sa=sa, sb=sb):
                a, b = ops[r]
                torch._scaled_mm(a, b.t(), scale_a=sa, scale_b=sb, out_dtype=torch.bfloat16)
            try:
                with torch.cuda.stream(stream):
                    for r in range(COPIES):
                        call(r)
                stream.synchronize()
            except RuntimeError as e:
                row[kind] = "unavailable: %s" % str(e).splitlines()[0][:100]
                continue
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=stream):
                for r in range(COPIES):
                    call(r)
            read_flush()
            replay_on(stream, gr)
            stream.synchronize()
            ts = []
            for _ in range(reps):
                read_flush()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                replay_on(stream, gr)
                e1.record(stream)
                stream.synchronize()
                ts.append(e0.elapsed_time(e1) / COPIES)
            us = float(np.mean(ts)) * 1e3
            row[kind + "_us"] = round(us, 2)
            row[kind + "_frac_mfma"] = round(2 * M * N * K / (us * 1e-6) / 1e12 / PEAK_FP8_TFLOPS, 4)
            del gr
        out.append(row)
        del ops
    torch.cuda.synchronize()
    if out:
        log("library FP8 GEMM (per-tensor scales) on %d prefill shapes in %.1f s: this kernel / library %s" % (
            len(out), time.time() - t0,
            " ".join("%.2f" % (r["us_this"] / r["per_tensor_us"]) for r in out if "per_tensor_us" in r)))
    return dict(what="torch._scaled_mm (hipBLASLt), E4M3 x E4M3 -> bf16, one scale per tensor / per row and "
                     "column: a coarser-scaled GEMM without 128-wide block promotion (context only)",
                per_shape=out)


def W_bytes(p):
    import workloads as W
    return W.dense_work(p["M"], p["N"], p["K"])[1]


def replay_on(stream, g):
    import torch
    with torch.cuda.stream(stream):
        g.replay()


def bench_specialized(fg, torch, stream, cases, per, replay, read_flush, reps):
    """The 18 sweep shapes with the tiled kernel built at run time for each (N, K): compile + load
    time of each kernel, then the same per-shape timing as the table kernels (HIP events around
    a graph of COPIES launches after a read-only 1 GiB buffer read), outputs checked bit for bit
    against the table kernel's with the same schedule (whole tiles)."""
    t0 = time.time()
    rows = []
    mark_leg(torch, stream, "specialized")
    for i, case in enumerate(cases):
        compile_ms = fg.specialize_nt(case["M"], case["N"], case["K"])
        # the specialised kernels keep whole tiles: their reference is the table kernel with the
        # same schedule (stream-K off), which shares their arithmetic order
        c0 = case["copies"][0]
        os.environ["FP8GEMM_STREAMK"] = "0"
        try:
            with torch.cuda.stream(stream):
                fg.gemm_nt(c0["A"], c0["sa"], c0["B"], c0["sb"], out=c0["D"], stream=stream)
            stream.synchronize()
        finally:
            os.environ.pop("FP8GEMM_STREAMK", None)
        ref = c0["D"].clone()

        def call(r, case=case):
            c = case["copies"][r]
            fg.gemm_nt_specialized(c["A"], c["sa"], c["B"], c["sb"], out=c["D"], stream=stream)

        with torch.cuda.stream(stream):
            call(0)
        stream.synchronize()
        if not torch.equal(case["copies"][0]["D"], ref):
            raise RuntimeError("specialized kernel differs from the table kernel (case %d)" % i)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for r in range(COPIES):
                call(r)
        replay(g)                        # untimed, as for the table kernels
        stream.synchronize()
        ts = []
        for _ in range(reps):
            read_flush()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            replay(g)
            e1.record(stream)
            stream.synchronize()
            ts.append(e0.elapsed_time(e1) / COPIES)
        us = float(np.mean(ts)) * 1e3
        rows.append(dict(M=case["M"], N=case["N"], K=case["K"], us_table=per[i]["us"], us_specialized=round(us, 2),
                         speedup=round(per[i]["us"] / us, 4), compile_ms=round(compile_ms, 1)))
        del g
    sp = [r["speedup"] for r in rows]
    geo = float(np.exp(np.mean(np.log(sp))))
    log("specialized kernels: geomean speedup %.3f over the table kernels, compile %.0f ms total (%.1f s)" % (
        geo, sum(r["compile_ms"] for r in rows), time.time() - t0))
    return dict(geomean_speedup=round(geo, 4), compile_ms_total=round(sum(r["compile_ms"] for r in rows), 1),
                per_shape=rows)


GROUPED_CALLS = 3      # calls per timed graph of the grouped configurations (at least one per copy)


ROTATE_BYTES = 600 * 1000 * 1000   # operand copies rotate over more than the 256 MB memory-side cache


def copies_for(nbytes, cap=4):
    """Operand copies so that the copies a graph rotates through exceed the memory-side cache."""
    return int(min(cap, max(1, -(-ROTATE_BYTES // max(1, nbytes)))))


def grouped_oracle_sample(name, w, got, target_rows=64):
    """The CPU oracle (as it stands) beside a grouped leg, on a bounded sample of the same
    workload: the first rows of the first two groups (contiguous: of the first group), all N and
    K.  Returns the oracle's rate in TFLOP/s; the sample's outputs are compared with the GPU's
    (`got`, the leg's output as bf16 bits), and a mismatch fails the run."""
    import oracle

    nth = oracle.num_threads(0)
    t0 = time.perf_counter()
    if name.startswith("contiguous"):
        rows = np.nonzero(w.m_indices == 0)[0][:4 * target_rows]
        ref, _ = oracle.grouped_contiguous(w.A[rows], w.sa[rows], w.B[:1], w.sb[:1], w.m_indices[rows])
        flop = 2 * rows.size * w.B.shape[1] * w.A.shape[1]
        what = "the first %d rows of group 0" % rows.size
        dt = time.perf_counter() - t0
        par = check_sample(got[rows], ref, name)
    else:
        G = 2
        mm = np.minimum(w.masked_m[:G], target_rows).astype(np.int32)
        args = (w.A[:G, :target_rows], w.sa[:G, :target_rows], w.B[:G], w.sb[:G], mm)
        ref, valid = (oracle.grouped_masked_fp4 if "fp4" in name else oracle.grouped_masked)(*args)
        flop = 2 * int(mm.sum()) * w.B.shape[1] * w.A.shape[2]
        what = "the first %d valid rows of groups 0 and 1" % int(mm.sum())
        dt = time.perf_counter() - t0
        v = valid.astype(bool)
        par = check_sample(got[:G, :target_rows][v], ref[v], name)
    return dict(value=round(flop / dt / 1e12, 6), unit="TFLOP/s", cores=nth, kind="oracle",
                sample="%s, all N and K: %.2f GFLOP in %.2f s (operand decode included)" % (what, flop / 1e9, dt),
                parity_vs_gpu=par)


def bench_grouped(fg, W, torch, dev, stream, reps=10, cpu=False):
    """Grouped configurations 2-4 and configuration 4 with MXFP4 weights: HIP events on the launch
    stream around a graph of calls after a read-only 1 GiB buffer read, divided by the calls; the
    calls rotate over operand copies (together over 600 MB), so none reads an operand another
    call left in the caches."""
    out = {}
    for name, make in (("contiguous_cfg2", W.config2), ("contiguous_cfg3", W.config3),
                       ("masked_cfg4", W.config4), ("masked_fp8xfp4_cfg4", W.config4_fp4)):
        t0 = time.time()
        w = make()
        base = dict(A=torch.from_numpy(w.A).to(dev), B=torch.from_numpy(w.B).to(dev),
                    sb=torch.from_numpy(w.sb).to(dev),
                    sa=torch.from_numpy(np.ascontiguousarray(np.swapaxes(w.sa, -1, -2))).to(dev))  # K-block-major
        nbytes = sum(t.numel() * t.element_size() for t in base.values())
        ncopy = copies_for(nbytes)
        ops = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(ncopy - 1)]
        N, K = w.B.shape[1], w.A.shape[-1]
        if name.startswith("contiguous"):
            idx = torch.from_numpy(w.m_indices).to(dev)
            for o in ops:
                o["D"] = torch.empty((w.A.shape[0], N), dtype=torch.bfloat16, device=dev)
            call = lambda o: fg.grouped_contiguous(o["A"], o["sa"], o["B"], o["sb"], idx, out=o["D"], stream=stream)
            counts = [int(np.sum(w.m_indices == g)) for g in range(w.B.shape[0])]
            flop, byts = W.grouped_work(counts, N, K, index_bytes=4 * w.A.shape[0])
        else:
            mm = torch.from_numpy(w.masked_m).to(dev)
            for o in ops:
                o["D"] = torch.empty((w.A.shape[0], w.A.shape[1], N), dtype=torch.bfloat16, device=dev)
            f = fg.fp8fp4_grouped_masked if "fp4" in name else fg.grouped_masked
            call = lambda o, f=f: f(o["A"], o["sa"], o["B"], o["sb"], mm, w.expected_m, out=o["D"], stream=stream)
            counts = [int(x) for x in w.masked_m]
            work = W.grouped_fp4_work if "fp4" in name else W.grouped_work
            flop, byts = work(counts, N, K, index_bytes=4 * len(counts))
        calls = max(GROUPED_CALLS, ncopy)
        torch.cuda.synchronize()        # operand copies are made on the default stream
        mark_leg(torch, stream, name)
        with torch.cuda.stream(stream):
            call(ops[0])
        cfg = fg.last_config()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for r in range(calls):
                call(ops[r % ncopy])
        flush = torch.ones(256 * 1024 * 1024, dtype=torch.float32, device=dev)
        sink = torch.zeros(1, device=dev)
        with torch.cuda.stream(stream):      # untimed: a graph's first replay measures slow
            sink.add_(flush.sum())
            g.replay()
        stream.synchronize()
        ts = []
        for _ in range(reps):
            with torch.cuda.stream(stream):
                sink.add_(flush.sum())
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                g.replay()
                e1.record(stream)
            stream.synchronize()
            ts.append(e0.elapsed_time(e1) / calls)
        ms = float(np.mean(ts))
        tf = flop / (ms * 1e-3) / 1e12
        gbs = byts / (ms * 1e-3) / 1e9
        out[name] = dict(us=round(ms * 1e3, 1), tflops=round(tf, 1), gbs=round(gbs, 1),
                         frac_mfma=round(tf / PEAK_FP8_TFLOPS, 4), frac_hbm=round(gbs / PEAK_HBM_GBS, 4),
                         valid_rows=int(sum(counts)), operand_copies=ncopy, config=cfg)
        if cpu:
            got = ops[0]["D"].view(torch.int16).cpu().numpy().view(np.uint16)
            out[name]["cpu_oracle"] = grouped_oracle_sample(name, w, got)
        log("%s: %.1f us, %.1f TFLOP/s, %.1f GB/s (%s) [%d copies, inputs %.1f s]" % (
            name, ms * 1e3, tf, gbs, cfg, ncopy, time.time() - t0))
        del ops, base, flush, g
        torch.cuda.empty_cache()
    return out


MOE_CALLS = 4          # calls per timed graph of the MoE legs (at least one per copy)


def moe_oracle_sample(e, rows_per_group=32, G=2):
    """The CPU oracle (as it stands) beside the MoE leg: the whole expert layer (first GEMM,
    SwiGLU + requantisation, second GEMM) for the first valid rows of the first two groups."""
    import oracle

    nth = oracle.num_threads(0)
    I = e.W2.shape[2]
    mm = np.minimum(e.masked_m[:G], rows_per_group).astype(np.int32)
    r = rows_per_group
    t0 = time.perf_counter()
    y, _ = oracle.grouped_masked(e.A[:G, :r], e.sa[:G, :r], e.W1[:G], e.s1[:G], mm)
    codes, sh, _ = oracle.swiglu_quantize_1x128(y.reshape(G * r, 2 * I))
    oracle.grouped_masked(codes.reshape(G, r, I), sh.reshape(G, r, -1), e.W2[:G], e.s2[:G], mm)
    dt = time.perf_counter() - t0
    H = e.A.shape[2]
    flop = 2 * int(mm.sum()) * (2 * I * H + H * I)
    return dict(value=round(flop / dt / 1e12, 6), unit="TFLOP/s", cores=nth, kind="oracle",
                sample="the expert layer for the first %d valid rows of groups 0 and 1: %.2f GFLOP in %.2f s "
                       "(operand decode included)" % (int(mm.sum()), flop / 1e9, dt))


def bench_moe_chain(fg, W, torch, dev, stream, reps=5, cpu=False):
    """One DeepSeek-V3-sized MoE expert layer on the masked decode configuration's groups (16
    groups, M_max 256, about 64 valid rows each, H = 7168, I = 2048): the first grouped GEMM
    (N = 4096, K = 7168), SwiGLU + requantisation, the second grouped GEMM (N = 7168, K = 2048),
    through the single chain entry point, and each step alone.  HIP events on the launch stream
    around a graph of calls after a read-only 1 GiB buffer read, divided by the calls; the calls of
    a step rotate over copies of its weights and buffers (together over 600 MB, at most 4), so the
    GEMM steps never read weights another call left in the caches (the SwiGLU step's 34 MB input
    copies stay below that).  HBM roofline on the algorithmic bytes (both layers' weights dominate)."""
    t0 = time.time()
    e = W.moe_config4()
    G, M_max, H = e.A.shape
    I = e.W2.shape[2]
    A = torch.from_numpy(e.A).to(dev)
    sa = torch.from_numpy(np.ascontiguousarray(np.swapaxes(e.sa, -1, -2))).to(dev)
    mm = torch.from_numpy(e.masked_m).to(dev)
    w0 = dict(W1=torch.from_numpy(e.W1).to(dev), s1=torch.from_numpy(e.s1).to(dev),
              W2=torch.from_numpy(e.W2).to(dev), s2=torch.from_numpy(e.s2).to(dev))

    def buffers():
        return dict(Y1=torch.empty((G, M_max, 2 * I), dtype=torch.bfloat16, device=dev),
                    Hq=torch.empty((G, M_max, I), dtype=torch.float8_e4m3fn, device=dev),
                    sh=torch.empty((G, I // 128, M_max), dtype=torch.float32, device=dev),
                    out=torch.empty((G, M_max, H), dtype=torch.bfloat16, device=dev))

    nb = lambda *ts: sum(t.numel() * t.element_size() for t in ts)
    counts = [int(x) for x in e.masked_m]
    rows = sum(counts)
    steps = {   # name: (bytes one call reads of weights and inputs, call on copy c)
        "chain": (nb(*w0.values()),
                  lambda c: fg.moe_expert_masked(A, sa, c["W1"], c["s1"], c["W2"], c["s2"], mm, e.expected_m,
                                                 out=c["out"], workspace=(c["Y1"], c["Hq"], c["sh"]), stream=stream)),
        "first_layer": (nb(w0["W1"], w0["s1"]),
                        lambda c: fg.grouped_masked(A, sa, c["W1"], c["s1"], mm, e.expected_m, out=c["Y1"], stream=stream)),
        "swiglu_quantize": (W.swiglu_quantize_work(rows, I),
                            lambda c: fg.swiglu_quantize_1x128_masked(c["Y1"], mm, codes=c["Hq"], scales=c["sh"],
                                                                      stream=stream)),
        "second_layer": (nb(w0["W2"], w0["s2"]),
                         lambda c: fg.grouped_masked(c["Hq"], c["sh"], c["W2"], c["s2"], mm, e.expected_m, out=c["out"],
                                                     stream=stream)),
    }
    work = {"chain": W.moe_expert_work(counts, H, I, G),
            "first_layer": W.grouped_work(counts, 2 * I, H, index_bytes=4 * G),
            "swiglu_quantize": (0, W.swiglu_quantize_work(rows, I)),
            "second_layer": W.grouped_work(counts, H, I, index_bytes=4 * G)}
    flush = torch.ones(256 * 1024 * 1024, dtype=torch.float32, device=dev)
    sink = torch.zeros(1, device=dev)
    res = {}
    copies = [dict(w0, **buffers())]
    for name, (nbytes, call) in steps.items():
        ncopy = copies_for(nbytes)
        while len(copies) < ncopy:
            copies.append(dict({k: v.clone() for k, v in w0.items()}, **buffers()))
        # every copy's buffers hold the previous step's results of that copy (chain order)
        torch.cuda.synchronize()        # weight copies are made on the default stream
        mark_leg(torch, stream, "moe_setup")
        with torch.cuda.stream(stream):
            for c in copies[:ncopy]:
                steps["chain"][1](c)
        stream.synchronize()
        mark_leg(torch, stream, "moe_" + name)      # the step's own launches follow
        with torch.cuda.stream(stream):
            call(copies[0])
        stream.synchronize()
        cfg = fg.last_config()
        calls = max(MOE_CALLS, ncopy)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for r in range(calls):
                call(copies[r % ncopy])
        with torch.cuda.stream(stream):      # untimed: a graph's first replay measures slow
            sink.add_(flush.sum())
            g.replay()
        stream.synchronize()
        ts = []
        for _ in range(reps):
            with torch.cuda.stream(stream):
                sink.add_(flush.sum())
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                g.replay()
                e1.record(stream)
            stream.synchronize()
            ts.append(e0.elapsed_time(e1) / calls)
        ms = float(np.mean(ts))
        flop, byts = work[name]
        gbs = byts / (ms * 1e-3) / 1e9
        res[name] = dict(us=round(ms * 1e3, 1), bytes=byts, gbs=round(gbs, 1),
                         frac_hbm=round(gbs / PEAK_HBM_GBS, 4), operand_copies=ncopy, config=cfg)
        if flop:
            res[name]["tflops"] = round(flop / (ms * 1e-3) / 1e12, 1)
        log("moe %s: %.1f us, %.1f GB/s (%s) [%d copies]" % (name, ms * 1e3, gbs, cfg, ncopy))
        del g
    res["chain"]["valid_rows"] = rows
    res["chain"]["shape"] = "G=%d M_max=%d H=%d I=%d" % (G, M_max, H, I)
    if cpu:
        res["chain"]["cpu_oracle"] = moe_oracle_sample(e)
    log("moe chain leg done in %.1f s" % (time.time() - t0))
    del A, sa, mm, w0, copies, flush
    torch.cuda.empty_cache()
    return res


QUANT_LAUNCHES = 16    # launches per timed graph of the quantiser (two operand copies alternate)


def bench_quantize(fg, W, torch, dev, stream, reps=5):
    """The 1x128 activation quantiser on the contiguous MoE configuration's activations
    (32768 x 7168 bf16) and on the masked decode configuration's (16 groups x 256 rows, about
    64 valid per group), against the HBM roofline: algorithmic bytes = 2 (bf16 in) + 1 (code
    out) per element + 4 per 128-element scale, over the average launch time.  Launch times come
    from HIP events on the launch stream around a graph of QUANT_LAUNCHES launches that alternate
    between two copies of every operand (940 MB of input for the dense case, well past the 256 MB
    last-level cache), after reading a 1 GiB buffer."""
    import oracle

    out = {}
    M, K = W.QUANT_M, W.QUANT_K
    t0 = time.time()
    bits = W.activations_bf16(M, K, seed=31)
    X0 = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
    Xs = [X0, X0.clone()]
    codes = [torch.empty((M, K), dtype=torch.float8_e4m3fn, device=dev) for _ in range(2)]
    scales = [torch.empty((K // 128, M), dtype=torch.float32, device=dev) for _ in range(2)]
    mm = W.config4_masked_m()
    G, M_max = len(mm), 256
    Xm = [x[:G * M_max].view(G, M_max, K) for x in Xs]
    mm_dev = torch.from_numpy(mm).to(dev)
    codes_m = [torch.empty((G, M_max, K), dtype=torch.float8_e4m3fn, device=dev) for _ in range(2)]
    scales_m = [torch.empty((G, K // 128, M_max), dtype=torch.float32, device=dev) for _ in range(2)]
    flush = torch.ones(256 * 1024 * 1024, dtype=torch.float32, device=dev)
    sink = torch.zeros(1, device=dev)

    def dense(i):
        fg.quantize_1x128(Xs[i], codes=codes[i], scales=scales[i], stream=stream)

    def masked(i):
        fg.quantize_1x128_masked(Xm[i], mm_dev, codes=codes_m[i], scales=scales_m[i], stream=stream)

    legs = (("dense_32768x7168", dense, W.quantize_work(M, K)),
            ("masked_16x256x7168", masked, W.quantize_work(int(mm.sum()), K)))
    for name, call, byts in legs:
        mark_leg(torch, stream, "quantize_" + name)
        with torch.cuda.stream(stream):
            call(0)
            call(1)
        cfg = fg.last_config()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(QUANT_LAUNCHES):
                call(i % 2)
        with torch.cuda.stream(stream):      # untimed: a graph's first replay measures slow
            sink.add_(flush.sum())
            g.replay()
        stream.synchronize()
        ts = []
        for _ in range(reps):
            with torch.cuda.stream(stream):
                sink.add_(flush.sum())
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                g.replay()
                e1.record(stream)
            stream.synchronize()
            ts.append(e0.elapsed_time(e1) / QUANT_LAUNCHES)
        ms = float(np.mean(ts))
        gbs = byts / (ms * 1e-3) / 1e9
        out[name] = dict(us=round(ms * 1e3, 2), bytes=byts, gbs=round(gbs, 1),
                         frac_hbm=round(gbs / PEAK_HBM_GBS, 4), config=cfg,
                         launches_per_graph=QUANT_LAUNCHES)
        log("quantize %s: %.2f us per launch, %.1f GB/s (%s)" % (name, ms * 1e3, gbs, cfg))
        del g
    # the product of the timed launches must equal the oracle's on a sample of rows
    rows = np.arange(0, M, 977)
    ref_c, ref_s = oracle.quantize_1x128(bits[rows])
    idx = torch.from_numpy(rows).to(dev)
    for i in range(2):
        got_c = codes[i].view(torch.uint8)[idx].cpu().numpy()
        got_s = scales[i][:, idx].cpu().numpy().T
        if not (np.array_equal(got_c, ref_c) and np.array_equal(got_s, ref_s)):
            raise RuntimeError("quantiser output differs from the oracle on sampled rows")
    d = out["dense_32768x7168"]
    d["roofline"] = dict(bound="hbm", achieved=d["gbs"], peak=PEAK_HBM_GBS, unit="GB/s",
                         frac=d["frac_hbm"], traffic=None)
    # the oracle on a bounded sample of the same matrix (context)
    nth = oracle.num_threads(0)
    r = min(M, 8192)
    t1 = time.perf_counter()
    oracle.quantize_1x128(bits[:r])
    dt = time.perf_counter() - t1
    d["cpu_oracle"] = dict(value=round(W.quantize_work(r, K) / dt / 1e9, 3), unit="GB/s", cores=nth,
                           sample="first %d rows of the 32768 x 7168 matrix in %.2f s" % (r, dt))
    log("quantiser legs done in %.1f s" % (time.time() - t0))
    del Xs, Xm, codes, scales, codes_m, scales_m, flush
    torch.cuda.empty_cache()
    return out


def check_sample(got_bits, ref_bits, what):
    """GPU outputs against the oracle's on the same outputs: |gpu - ref| <= 2^-7 |ref| +
    1e-3 rms(ref) per element (rms over the sample).  Raises on a mismatch, so a bench run whose
    outputs are wrong fails; returns the count, bit-equal share and worst error / tolerance."""
    f = lambda b: (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    g, r = f(got_bits).ravel(), f(ref_bits).ravel()
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    lim = 2.0 ** -7 * np.abs(r) + 1e-3 * rms
    err = np.abs(g - r)
    bad = int(np.sum(~(err <= lim)))
    if bad:
        raise RuntimeError("%s: %d of %d GPU outputs differ from the oracle beyond the tolerance" % (what, bad, r.size))
    return dict(outputs=int(r.size), bit_equal=round(float(np.mean(g == r)), 6),
                max_err_over_tolerance=round(float(np.max(err / np.maximum(lim, 1e-300))), 4) if r.size else 0.0)


def cpu_baseline(cases, eager, target_s):
    """The CPU oracle (as it stands) on rows 0..r-1 of every sweep case, r sized so the whole
    sample takes about target_s seconds on this host; the oracle's rows of the reported sample
    are compared with the GPU's outputs of the same rows (the run fails on a mismatch)."""
    import oracle

    nth = oracle.num_threads(0)
    # the oracle spreads rows over its threads: probe with two rows per thread
    probe = max(cases, key=lambda c: c["M"])
    pr = min(probe["M"], 2 * nth)
    t0 = time.perf_counter()
    oracle.gemm_nt(probe["hostA"][:pr], probe["hostsa"][:pr], probe["hostB"], probe["hostsb"])
    t_probe = (time.perf_counter() - t0) / pr
    per_row_all = t_probe * sum(c["N"] * c["K"] for c in cases) / (probe["N"] * probe["K"])
    rows = int(max(1, min(4096, target_s / max(per_row_all, 1e-9))))

    def run(rows):
        flop, refs = 0, []
        t0 = time.perf_counter()
        for c in cases:
            r = min(rows, c["M"])
            refs.append(oracle.gemm_nt(c["hostA"][:r], c["hostsa"][:r], c["hostB"], c["hostsb"]))
            flop += 2 * r * c["N"] * c["K"]
        return flop, time.perf_counter() - t0, refs

    flop, dt, refs = run(rows)
    # the probe also pays the per-call decode of B, so the first sample can fall short of the
    # target: resize once from the measured time (the reported sample is the second)
    if dt < 0.6 * target_s and rows < 4096:
        rows = int(max(1, min(4096, rows * target_s / dt)))
        flop, dt, refs = run(rows)
    log("cpu oracle: %d rows of each case, %.1f GFLOP in %.1f s on %d threads" % (rows, flop / 1e9, dt, nth))
    import torch
    checked = []
    for c, ref, outs in zip(cases, refs, eager):
        got = outs[0][:ref.shape[0]].view(torch.int16).cpu().numpy().view(np.uint16)
        checked.append(check_sample(got, ref, "%dx%dx%d" % (c["M"], c["N"], c["K"])))
    n = sum(x["outputs"] for x in checked)
    parity = dict(outputs=n, bit_equal=round(sum(x["bit_equal"] * x["outputs"] for x in checked) / n, 6),
                  max_err_over_tolerance=max(x["max_err_over_tolerance"] for x in checked), within_tolerance=True)
    log("cpu oracle sample vs GPU outputs: %d outputs within tolerance, %.4f bit-equal" % (n, parity["bit_equal"]))
    return dict(value=round(flop / dt / 1e12, 6), unit="TFLOP/s", cores=nth, kind="oracle",
                sample="first %d rows (at most M) of each of the 18 sweep GEMMs, all N and K: %.1f GFLOP in %.1f s"
                       % (rows, flop / 1e9, dt), parity_vs_gpu=parity)


if __name__ == "__main__":
    main()
