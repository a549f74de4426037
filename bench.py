#!/usr/bin/env python3
"""Throughput of FP32 SGEMM C = A.B on one MI355X.

A step is one call of ``sgemm`` (every kernel the default plan enqueues) on
the workload's seeded synthetic inputs, already resident in HBM.  The default
workload is M = N = K = 4096 with A, B i.i.d. uniform on [-1, 1).

Prints one JSON line with the throughput (TFLOP/s, 2MNK per step), the
roofline of the dominant kernel (its time per step from two HIP events on the
launch stream around the timed steps; for a plan of one launch per step that
is the kernel's own launch time plus the gap to the next launch, for a plan of
several launches it covers all of them), against the FP32 matrix-core peak,
the median and minimum of launches timed one by one after a cache flush
(`flushed`), and the host oracle's throughput on a bounded sample of the same
workload and on the 256^3 workload (all host threads and one thread).
"""
import argparse
import hashlib
import json
import os
import re
import statistics
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP32_TFLOPS = 157.3        # MI355X dense FP32 (vector and matrix), 256 CU x 2.4 GHz x 256 FLOP/clk
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E
METRIC = "FP32 SGEMM TFLOPS at M=N=K=4096 and % of MI355X FP32 peak"
DEFAULT_WORKLOAD = "sgemm_4096"


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--path", default="auto")
    ap.add_argument("--tile", type=int, default=-1)
    ap.add_argument("--split-k", type=int, default=0)
    ap.add_argument("--decomposition", default="auto")
    ap.add_argument("--pack", default="auto", choices=["auto", "never", "always"])
    ap.add_argument("--row-tail", default="auto", choices=["auto", "never", "always"],
                    help="run the last 1-32 rows of M through the skinny kernel (planner default: auto)")
    ap.add_argument("--tile-order", default="xcd", choices=["xcd", "plain"],
                    help="matrix-core tile order: XCD-aware (default) or plain row-major, for comparison")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target host time of the oracle sample (0 = skip the CPU baseline)")
    ap.add_argument("--flush-mib", type=int, default=1024,
                    help="size of the buffer read (or written) before each flushed launch")
    ap.add_argument("--flush-launches", type=int, default=50,
                    help="launches timed one by one after a cache flush (0 = none)")
    ap.add_argument("--probe-seconds", type=float, default=1.5,
                    help="untimed steps before the timed region while rocm-smi samples the clocks (0 = none)")
    return ap.parse_args()


def algorithmic(w):
    flops = 2 * w.M * w.N * w.K
    bytes_ = 4 * (w.M * w.K + w.K * w.N + w.M * w.N)
    return flops, bytes_


def source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_key, digest):
    """HBM traffic per launch from the committed counter summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as fh:
            db = json.load(fh)
    except (OSError, ValueError):
        return None
    rec = db.get(kernel_key)
    if not rec or rec.get("source_digest") != digest:
        return None
    return rec.get("bytes_per_launch")


def sample_clocks(stop, out):
    """rocm-smi readings (shader clock in MHz, package power in W) until stop is set."""
    while not stop.is_set():
        try:
            r = subprocess.run(["rocm-smi", "--showclocks", "--showpower"], capture_output=True, text=True,
                               timeout=5)
        except (OSError, subprocess.SubprocessError):
            return
        m = re.search(r"sclk clock level: \d+: \((\d+)Mhz\)", r.stdout)
        if m:
            out["sclk_mhz"].append(int(m.group(1)))
        m = re.search(r"Package Power \(W\): ([0-9.]+)", r.stdout)
        if m:
            out["power_w"].append(float(m.group(1)))


def cpu_oracle_small(threads_all):
    """The oracle on the 256^3 workload: median of 3 runs on all host threads
    and on one thread (TFLOP/s)."""
    import oracle
    import workloads
    w = workloads.CONFIGS["sgemm_256"]
    An, Bn = w.a().numpy(), w.b().numpy()
    out = {}
    for threads in (threads_all, 1):
        oracle.set_num_threads(threads)
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            oracle.sgemm(An, Bn)
            ts.append(time.perf_counter() - t0)
        out[f"threads_{threads}"] = {"value": 2 * w.M * w.N * w.K / statistics.median(ts) / 1e12,
                                     "unit": "TFLOP/s", "ms_median": statistics.median(ts) * 1e3}
    oracle.set_num_threads(threads_all)
    return {"workload": w.name, "kind": "oracle", **out}


def cpu_baseline(w, A, B, target_s):
    """The host oracle on the first R rows of the workload (R chosen so the
    timed run takes about target_s seconds), scaled to TFLOP/s."""
    import oracle
    An = A.numpy()
    Bn = B.numpy()
    rows = max(1, min(w.M, 8))
    t0 = time.perf_counter()
    oracle.sgemm(An[:rows], Bn)
    t = time.perf_counter() - t0
    rows = max(1, min(w.M, int(rows * target_s / max(t, 1e-3))))
    t0 = time.perf_counter()
    oracle.sgemm(An[:rows], Bn)
    t = time.perf_counter() - t0
    flops = 2 * rows * w.N * w.K
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"first {rows} of {w.M} rows of C ({rows}x{w.N}x{w.K}), fp64 accumulation, {t:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(the library is a single-GPU SGEMM)", file=sys.stderr)
        sys.exit(2)

    import torch
    import dense_fp32_matrix_amd as lib
    import workloads

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    lib.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    w = workloads.CONFIGS[args.workload]
    A_host = w.a()
    B_host = w.b()
    A = A_host.to(dev)
    B = B_host.to(dev)
    C = torch.empty((w.M, w.N), dtype=torch.float32, device=dev)
    opts = {}
    if (args.path != "auto" or args.tile >= 0 or args.split_k or args.decomposition != "auto" or args.pack != "auto"
            or args.tile_order != "xcd" or args.row_tail != "auto"):
        opts = {"path": args.path, "tile": args.tile, "split_k": args.split_k,
                "decomposition": args.decomposition, "pack": args.pack, "tile_order": args.tile_order,
                "row_tail": args.row_tail}
    plan = lib.sgemm_plan_query(w.M, w.N, w.K, A.data_ptr(), w.lda, B.data_ptr(), w.ldb, C.data_ptr(), w.N,
                                **opts)

    def step():
        if opts:
            lib.sgemm_ex(A, B, C, **opts)
        else:
            lib.sgemm(A, B, C)

    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Clock and power while the workload runs: an untimed probe phase of
    # --probe-seconds after the warmup steps, which also brings the clocks to
    # their steady state before the timed region.
    samples = {"sclk_mhz": [], "power_w": []}
    if args.probe_seconds > 0:
        stop = threading.Event()
        th = threading.Thread(target=sample_clocks, args=(stop, samples))
        th.start()
        t_end = time.perf_counter() + args.probe_seconds
        while time.perf_counter() < t_end:
            for _ in range(8):
                step()
            torch.cuda.synchronize()
        stop.set()
        # keep the GPU busy until the last rocm-smi reading has returned: an
        # idle gap here lets the clocks drop, and the first timed steps would
        # then run while they ramp back up
        while th.is_alive():
            for _ in range(4):
                step()
            torch.cuda.synchronize()
        th.join()
    clocks = None
    if samples["sclk_mhz"]:
        tail = samples["sclk_mhz"][len(samples["sclk_mhz"]) // 2:]
        clocks = {"sclk_mhz_median_2nd_half": statistics.median(tail), "sclk_mhz_min": min(samples["sclk_mhz"]),
                  "sclk_mhz_max": max(samples["sclk_mhz"]), "samples": len(samples["sclk_mhz"]),
                  "power_w_median": statistics.median(samples["power_w"]) if samples["power_w"] else None,
                  "source": f"rocm-smi during {args.probe_seconds:g} s of untimed steps before the timed region"}

    # timed region: K back-to-back steps on the launch stream between two
    # events (no markers between the steps, which would add gaps of their own)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    event_ms_per_step = ev0.elapsed_time(ev1) / args.steps
    ms_per_step = wall * 1e3 / args.steps

    flops, alg_bytes = algorithmic(w)
    value = flops * args.steps / wall / 1e12

    # Launches from cold caches: before each, read (or write) a buffer larger
    # than the L2s and the 256 MB MALL together, so the operands come from HBM.
    # Reading leaves the caches holding clean lines; writing (the pages'
    # flush) leaves up to 256 MB of dirty lines whose write-back competes
    # with the launch's reads, so that figure is reported beside the other.
    def cold_launches(mode, fn=step):
        ts = []
        for _ in range(args.flush_launches):
            if mode == "read":
                flush.sum()
            else:
                flush.fill_(1.0)
            s = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            s.record(stream)
            fn()
            e.record(stream)
            torch.cuda.synchronize()
            ts.append(s.elapsed_time(e))
        return ts

    # Where the product is bound by reading B once (M <= 16), the library's
    # read-rate probe reads the same B -- the same bytes, from the same cache
    # state -- warm (back-to-back) and after the same flush: the attainable
    # rate the call is compared with, beside the data-sheet peak.
    hbm_bound = w.M <= 16
    b_flat = B.reshape(-1) if hbm_bound and B.is_contiguous() and B.numel() % 4 == 0 else None
    probe = None
    if b_flat is not None:
        part = torch.empty(lib.READ_PROBE_PARTIALS, dtype=torch.float32, device=dev)

        def read_b():
            lib.read_probe(b_flat, part)

        for _ in range(args.warmup):
            read_b()
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(args.steps):
            read_b()
        ev1.record(stream)
        torch.cuda.synchronize()
        read_ms = ev0.elapsed_time(ev1) / args.steps
        b_bytes = 4 * b_flat.numel()
        probe = {"what": f"sgemm_read_probe over B ({w.K} x {w.N} fp32, {b_bytes} bytes), read once",
                 "warm_ms": read_ms, "warm_gbs": b_bytes / (read_ms * 1e-3) / 1e9}

    flushed = None
    if args.flush_launches > 0:
        flush = torch.ones(args.flush_mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
        fr = cold_launches("read")
        fw = cold_launches("write")
        if probe is not None:
            pr = cold_launches("read", read_b)
            probe["flushed_ms_median"] = statistics.median(pr)
            probe["flushed_gbs"] = 4 * b_flat.numel() / (probe["flushed_ms_median"] * 1e-3) / 1e9
        del flush
        flushed = {"flush": f"{args.flush_mib} MiB read before each launch", "launches": len(fr),
                   "ms_median": statistics.median(fr), "ms_min": min(fr),
                   "write_flush_ms_median": statistics.median(fw), "write_flush_ms_min": min(fw)}

    kernel_ms = event_ms_per_step
    main_kernel = {1: "naive_gemm_kernel", 2: "valu_gemm_kernel", 3: "mfma_gemm_kernel",
                   4: "skinny_gemm_kernel"}.get(plan["path"], "?")
    src = {1: "simple.hip", 2: "valu.hip", 3: "mfma.hip", 4: "skinny.hip"}.get(plan["path"], "mfma.hip")
    digest = source_digest([f"dense_fp32_matrix_amd/csrc/{src}", "dense_fp32_matrix_amd/csrc/kernels.hpp",
                            "dense_fp32_matrix_amd/csrc/lds_layout.hpp", "dense_fp32_matrix_amd/csrc/tile_order.hpp"])
    key = (f"{main_kernel}:{w.name}:tile{plan['tile']}:{plan['decomposition_name']}:split{plan['split_k']}"
           f":vec{plan['vector']}:pack{plan['packed']}")
    if hbm_bound:
        achieved = alg_bytes / (kernel_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS}
    else:
        achieved = flops / (kernel_ms * 1e-3) / 1e12
        roof = {"bound": "mfma" if plan["path"] in (3, 4) else "alu", "achieved": achieved,
                "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_FP32_TFLOPS}
    roof["traffic"] = load_traffic(key, digest)
    roof["kernel"] = main_kernel
    roof["launch_ms"] = kernel_ms
    roof["launches_per_step"] = plan["launches"]
    if not hbm_bound and clocks is not None:
        # the same peak at the shader clock the GPU held while the workload ran
        # (power management lowers it under some loads; HBM's peak does not move with it)
        sclk = clocks["sclk_mhz_median_2nd_half"]
        peak_clk = PEAK_FP32_TFLOPS * sclk / 2400.0
        roof["clock_adjusted"] = {"sclk_mhz": sclk, "peak": peak_clk, "frac": achieved / peak_clk}
    if probe is not None:
        probe["call_vs_read_warm"] = probe["warm_ms"] / kernel_ms
        roof["read_probe"] = probe
    if roof["bound"] == "alu":
        # the VALU path's ceiling measured, beside the data-sheet figure: the
        # library's FMA-rate probe (scalar v_fmac_f32, 16 chains per lane,
        # 32 workgroups per CU)
        fma_wgs, fma_iters = 8192, 1000
        fma_out = torch.empty(fma_wgs * 256, dtype=torch.float32, device=dev)
        lib.fma_probe(fma_iters, fma_wgs, fma_out)
        fts = []
        for _ in range(5):
            s0 = torch.cuda.Event(enable_timing=True)
            s1 = torch.cuda.Event(enable_timing=True)
            s0.record(stream)
            lib.fma_probe(fma_iters, fma_wgs, fma_out)
            s1.record(stream)
            torch.cuda.synchronize()
            fts.append(s0.elapsed_time(s1))
        fma_flops = 2.0 * fma_wgs * 256 * fma_iters * lib.FMA_PROBE_FMAS_PER_ITER
        ceiling = fma_flops / (statistics.median(fts) * 1e-3) / 1e12
        roof["fma_probe"] = {"what": "sgemm_fma_probe: scalar FP32 FMA rate, 8192 x 256 lanes x 128000 FMAs",
                             "tflops": ceiling, "frac_of_probe": achieved / ceiling}

    cpu = None
    cpu_small = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(w, A_host, B_host, args.cpu_seconds)
        cpu_small = cpu_oracle_small(cpu["cores"])
    if flushed is not None:
        # the same roofline as the warm figure, on the flushed launch median (the whole call)
        fm = flushed["ms_median"] * 1e-3
        if hbm_bound:
            flushed["achieved"] = alg_bytes / fm / 1e9
            flushed["unit"] = "GB/s"
            flushed["frac"] = flushed["achieved"] / PEAK_HBM_GBS
            if probe is not None and "flushed_ms_median" in probe:
                # the probe's time for B over the call's time for A, B and C
                flushed["vs_read_probe"] = probe["flushed_ms_median"] / flushed["ms_median"]
        else:
            flushed["achieved"] = flops / fm / 1e12
            flushed["unit"] = "TFLOP/s"
            flushed["frac"] = flushed["achieved"] / PEAK_FP32_TFLOPS

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "pct_of_fp32_peak": 100.0 * value / PEAK_FP32_TFLOPS,
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "lda": w.lda, "ldb": w.ldb, "ldc": w.N,
                   "inputs": f"A~{w.a_kind}, B~{w.b_kind}", "path": plan["path_name"], "tile": plan["tile"],
                   "bm": plan["bm"], "bn": plan["bn"], "bk": plan["bk"], "split_k": plan["split_k"],
                   "decomposition": plan["decomposition_name"],
                   "vector_loads": bool(plan["vector"]), "packed": plan["packed"], "workgroups": plan["workgroups"],
                   "tail_rows": plan["tail_rows"],
                   "tile_order": args.tile_order},
        "roofline": roof,
        "cpu_baseline": cpu,
        "cpu_oracle_256": cpu_small,
        "clocks": clocks,
        "flushed": flushed,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
