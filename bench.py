"""Benchmark of the cross-tier KV transfer on one MI355X.

One step = one pass of the hot path over a 32K-token prefix of an MLA-latent KV
pool (78 layers x 576 bf16 = 1152-byte rows, page size 64): a D2H write-back of
the prefix from contiguous device pages into the pinned host pool, then an H2D
load of it (per-layer kernels and per-layer events) into another 512 device
pages. Inputs are resident (device pool in HBM, host pool pinned) before the
timed region. Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--layout layer_first]
                    [--path auto|kernel|kernel_lds|dma] [--no-matrix] [--no-cpu-baseline]
                    [--no-extra]

Besides the headline step it reports the measured link peak (1 GiB copies on
the copy engines and on the zero-copy kernel), the layout x path matrix, the
bidirectional mixed batch, the per-layer streamed load and a write-back beside
compute, the write filter and the oracle as CPU baseline. Studies that print their own JSON line and exit:

    python bench.py --host-memory-study 3 24    # pinned pool size and NUMA placement
    python bench.py --free-list-study           # FIFO vs LIFO host free list under churn
    python bench.py --tp-shared-study 8         # tensor-parallel group sharing one host pool
    python bench.py --profile-counters          # the kernels a rocprofv3 --pmc pass needs
    python bench.py --interference-loader DIR & # a load beside the consumer below, which
    rocprofv3 --pmc ... -- python bench.py --interference-consumer DIR   # runs under the profiler
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KV transfer GB/s H2D & D2H (32K-token prefix) as % of host-link peak"
PCIE_GEN5_X16_GBPS = 64.0   # PCIe 5.0 x16, per direction, 32 GT/s x 16 lanes (raw)
HBM_PEAK_GBPS = 8000.0
# the paced write-back grid's rate as a fraction of the measured D2H link peak
PACE_OF_LINK = 0.98
LAYOUTS = {"layer_first": 0, "page_first": 1, "page_first_direct": 2}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--layout", default="layer_first", choices=sorted(LAYOUTS))
    p.add_argument("--path", default="auto", choices=["auto", "kernel", "kernel_lds", "dma"])
    p.add_argument("--no-matrix", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true",
                   help="skip the bidirectional mixed-batch and per-layer streamed legs")
    p.add_argument("--cell-seconds", type=float, default=0.4,
                   help="timed repetitions per matrix cell: about this many seconds, 3..20 reps")
    p.add_argument("--host-memory-study", type=float, nargs="+", metavar="GB",
                   help="only measure the headline request against pinned host pools of "
                        "these sizes (GB), then exit")
    p.add_argument("--tp-shared-study", type=int, default=0, metavar="TP",
                   help="only run the tensor-parallel shared host pool study for a group of "
                        "TP pools on this GPU, then exit")
    p.add_argument("--free-list-study", action="store_true",
                   help="only run the FIFO-vs-LIFO host free-list churn study, then exit")
    p.add_argument("--size-sweep", action="store_true",
                   help="only time write-backs and loads of 64..32768 tokens on every path "
                        "and layout (one JSON line per size on stderr), then exit")
    p.add_argument("--overlap-study", nargs="?", const="all", choices=["all", "write-back"],
                   help="only sweep the kernel path's grid for loads beside compute "
                        "(KV_F_LOAD_OVERLAP) and for write-backs beside compute (plain and "
                        "paced grids), on the streamed workload, then exit; 'write-back': "
                        "the write-backs only")
    p.add_argument("--profile-counters", action="store_true",
                   help="only run the kernels a rocprofv3 --pmc pass needs, then exit")
    p.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="turn two rocprofv3 --pmc output directories (FETCH_SIZE, WRITE_SIZE) "
                        "into profiles/counters.json and exit")
    p.add_argument("--summarize-trace", metavar="TRACE_DIR",
                   help="print the per-kernel, per-grid launch durations of a rocprofv3 "
                        "--kernel-trace output directory as a markdown table and exit")
    p.add_argument("--summarize-link-counters", nargs=2, metavar=("WRREQ_DIR", "RDREQ_DIR"),
                   help="add the host-link bytes of two rocprofv3 --pmc output directories "
                        "(TCC_EA0_WRREQ*_sum, TCC_EA0_RDREQ*_sum) to profiles/counters.json "
                        "and exit")
    p.add_argument("--interference-loader", metavar="DIR",
                   help="one half of the interference counter study: in this process, keep "
                        "per-layer loads running on each transfer path in turn while the "
                        "consumer process (--interference-consumer DIR, the one under "
                        "rocprofv3 --pmc) asks for it through files in DIR, then exit")
    p.add_argument("--interference-consumer", metavar="DIR",
                   help="the other half: run an HBM-bound consumer alone, then beside each of "
                        "the loader's paths, then alone again, writing its phases to "
                        "DIR/consumer.json, then exit")
    p.add_argument("--summarize-interference", nargs="+", metavar="DIR",
                   help="per-phase medians of the consumer's counters and launch durations "
                        "from --interference-consumer runs under rocprofv3 (one DIR per "
                        "counter pass), as a markdown table, and exit")
    return p.parse_args()


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.summarize_link_counters:
        summarize_link_counters(*args.summarize_link_counters)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_interference:
        summarize_interference(args.summarize_interference)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this transfer path has no multi-GPU part "
              "(each GPU moves its own KV over its own host link); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import hierarchical_kv_cache_backup_amd as kvt
    from hierarchical_kv_cache_backup_amd import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.host_memory_study:
        print(json.dumps(host_memory_study(torch, kvt, workloads, args.host_memory_study)))
        return
    if args.free_list_study:
        print(json.dumps(free_list_study(torch, kvt, workloads)))
        return
    if args.size_sweep:
        print(json.dumps(size_sweep(torch, kvt, workloads)))
        return
    if args.overlap_study:
        print(json.dumps(overlap_study(torch, kvt, workloads,
                                       with_loads=args.overlap_study == "all")))
        return
    if args.tp_shared_study:
        print(json.dumps(tp_shared_study(torch, kvt, workloads, args.tp_shared_study)))
        return
    if args.interference_loader:
        interference_loader(torch, kvt, workloads, args.interference_loader)
        return
    if args.interference_consumer:
        print(json.dumps(interference_consumer(torch, args.interference_consumer)))
        return
    dev = torch.device("cuda:0")
    shape = workloads.mla32k()
    L, C, R, ps = shape.layers, shape.components, shape.row_bytes, shape.page_size
    S_dev, S_host = shape.device_slots, shape.host_slots
    n = shape.extra["tokens"]
    layout = LAYOUTS[args.layout]
    path = {"auto": kvt.PATH_AUTO, "kernel": kvt.PATH_KERNEL, "kernel_lds": kvt.PATH_KERNEL_LDS,
            "dma": kvt.PATH_DMA}[args.path]

    # concurrent H2D + D2H capacity of the link, taken before the large device
    # allocations below (copy-engine D2H beside H2D has measured slower after them)
    duplex_fresh = (None if args.no_extra or args.profile_counters
                    else _duplex_peak(torch, kvt))

    # ---- resident inputs: device pool (seeded bf16 N(0,1)), host pool, index sets
    t_setup = time.perf_counter()
    bufs = []
    for l in range(L):
        for c in range(C):
            b = torch.empty(S_dev * R, dtype=torch.uint8, device=dev)
            workloads.fill_device_buffer(b, shape, 3, l, c, torch)
            bufs.append(b)
    pages_total = S_dev // ps
    npages = n // ps
    first = workloads.contiguous_pages_at_offset(3, pages_total, npages)
    dev_b = workloads.page_indices(first, ps)
    second = (first + npages) % pages_total                  # the other 512 pages
    dev_l = workloads.page_indices(second, ps)
    host_idx = np.arange(n, dtype=np.int64)
    geom = kvt.geometry(L, C, R, S_dev, S_host, ps, layout)
    t0 = time.perf_counter()
    pool = kvt.KvPool(geom, bufs, device=0)
    t_pool = time.perf_counter() - t0
    torch.cuda.synchronize()
    log("setup %.1fs (pool create %.2fs, host pool %.2f GB)" %
        (time.perf_counter() - t_setup, t_pool, pool.host_array().nbytes / 1e9))
    s = torch.cuda.Stream()
    bytes_dir = n * L * C * R
    if args.profile_counters:
        profile_counters(torch, kvt, pool, s, dev_b, dev_l, host_idx, L)
        pool.close()
        return

    def timed(fn, reps, warm=2):
        """Median device time (s) of fn() on stream s, by events recorded on s."""
        for _ in range(warm):
            fn()
        s.synchronize()
        ts = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(s)
            fn()
            e1.record(s)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) / 1e3)
        return statistics.median(ts), ts

    # ---- measured host-link peak: the best of two contiguous 1 GiB copies per
    # direction, median of 20 each: the copy engines (hipMemcpyAsync between a
    # device buffer and pinned host memory) and the zero-copy kernel (one
    # launch over 262,144 contiguous 4 KiB rows of a one-buffer pool)
    GiB = 1 << 30
    dbuf = torch.empty(GiB, dtype=torch.uint8, device=dev)
    hbuf = torch.empty(GiB, dtype=torch.uint8, pin_memory=True)
    with torch.cuda.stream(s):
        t_h2d, _ = timed(lambda: dbuf.copy_(hbuf, non_blocking=True), 20)
        t_d2h, _ = timed(lambda: hbuf.copy_(dbuf, non_blocking=True), 20)
    memcpy_peak = {"h2d": GiB / t_h2d / 1e9, "d2h": GiB / t_d2h / 1e9}
    del hbuf
    rows = GiB // 4096
    peak_pool = kvt.KvPool(kvt.geometry(1, 1, 4096, rows, rows, 64, 0), [dbuf])
    peak_pool.set_path(kvt.PATH_KERNEL)
    pc = peak_pool.calibration()
    pc.load_split_min_bytes = 2.0 * GiB             # one launch
    pc.kernel_max_workgroups[:] = [0, 0]            # full grid both ways
    peak_pool.set_calibration(pc)
    all_rows = np.arange(rows, dtype=np.int64)
    k_d2h, _ = timed(lambda: peak_pool.backup(all_rows, all_rows, 0, 1, s), 20)
    k_h2d, _ = timed(lambda: peak_pool.load(all_rows, all_rows, 0, 1, s), 20)
    kernel_peak = {"h2d": GiB / k_h2d / 1e9, "d2h": GiB / k_d2h / 1e9}
    peak_pool.close()
    del dbuf, peak_pool
    settle(torch, 3 * GiB)      # 1 GiB device and 2 GiB pinned memory were freed
    log("1 GiB contiguous: copy engines H2D %.2f / D2H %.2f GB/s, kernel H2D %.2f / D2H %.2f"
        % (memcpy_peak["h2d"], memcpy_peak["d2h"], kernel_peak["h2d"], kernel_peak["d2h"]))

    # ---- per-path measurements on the workload (calibrates the selector)
    def run(direction, p, lay_pool):
        lay_pool.set_path(p)
        if direction == kvt.BACKUP:
            return timed(lambda: lay_pool.backup(dev_b, host_idx, 0, L, s), 5)[0]
        return timed(lambda: lay_pool.load(dev_l, host_idx, 0, L, s), 5)[0]

    # The selector models a call as fixed costs (per kernel launch, per copy-engine
    # call) plus bytes / rate. The measured call time already holds the fixed
    # costs, so each rate is fitted to the time left after the modelled fixed
    # costs of the launches and copies that call made (counted by kv_get_stats).
    # The kernel rate is the link-bound rate of a full grid; what a capped grid
    # moves is modelled per workgroup (kernel_wg_gbps / kernel_wg_row_ns).
    calib = pool.calibration()
    meas, ops = {}, {}
    full = pool.calibration()
    full.kernel_max_workgroups[:] = [0, 0]
    for d in (kvt.BACKUP, kvt.LOAD):
        for p in (kvt.PATH_KERNEL, kvt.PATH_DMA, kvt.PATH_STAGED):
            pool.set_calibration(full if p == kvt.PATH_KERNEL else calib)
            meas[(d, p)] = run(d, p, pool)
            s0 = pool.stats()
            (pool.backup(dev_b, host_idx, 0, L, s) if d == kvt.BACKUP
             else pool.load(dev_l, host_idx, 0, L, s))
            s.synchronize()
            s1 = pool.stats()
            ops[(d, p)] = (s1.kernel_launches[d] - s0.kernel_launches[d],
                           s1.dma_copies[d] - s0.dma_copies[d])
            log("%s %s: %.2f GB/s (%d launches, %d copies per call)" %
                ("D2H" if d == 0 else "H2D", kvt.PATH_NAMES[p],
                 bytes_dir / meas[(d, p)] / 1e9, *ops[(d, p)]))

        def fixed_s(p):
            k, c = ops[(d, p)]
            # the kernel path's further launches also leave the link idle; the
            # staged path's overlap its copies
            gap = calib.kernel_group_us[d] + (calib.kernel_link_gap_us[d]
                                              if p == kvt.PATH_KERNEL else 0.0)
            kern = calib.kernel_launch_us[d] + (k - 1) * gap if k else 0.0
            return (kern + c * calib.dma_copy_us[d]) * 1e-6

        def fit(p):
            return bytes_dir / max(meas[(d, p)] - fixed_s(p), 0.5 * meas[(d, p)]) / 1e9

        calib.kernel_gbps[d] = fit(kvt.PATH_KERNEL)
        calib.dma_gbps[d] = fit(kvt.PATH_DMA)
    # The staged path is modelled as its fixed costs + the copy-engine stream +
    # one small ramp chunk's device-side pass (the others overlap the copies);
    # that pass rate (staged_gather_gbps) keeps the library's value, as a few
    # microseconds of a 50 ms call cannot be fitted from it.
    # the measured peak is the better of the two contiguous 1 GiB copies per
    # direction; the workload's own best path rate is reported beside it, never
    # inside it
    link_peak = {"h2d": max(memcpy_peak["h2d"], kernel_peak["h2d"]),
                 "d2h": max(memcpy_peak["d2h"], kernel_peak["d2h"])}
    # a paced write-back grid must not issue more than this link drains
    calib.kernel_pace_gbps[0] = round(PACE_OF_LINK * link_peak["d2h"], 2)
    pool.set_calibration(calib)
    pool.set_path(path)
    best_rate = {dd: max(bytes_dir / meas[(dd, p)] / 1e9 for p in
                         (kvt.PATH_KERNEL, kvt.PATH_DMA, kvt.PATH_STAGED))
                 for dd in (kvt.BACKUP, kvt.LOAD)}
    workload_best = {"h2d": best_rate[kvt.LOAD], "d2h": best_rate[kvt.BACKUP]}

    # ---- the timed steps
    def step(ev=None):
        if ev is not None:
            ev[0].record(s)
        pool.backup(dev_b, host_idx, 0, L, s)
        if ev is not None:
            ev[1].record(s)
        pool.load(dev_l, host_idx, 0, L, s)
        if ev is not None:
            ev[2].record(s)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    stats0 = pool.stats()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    d2h_t = [e[0].elapsed_time(e[1]) / 1e3 for e in evs]
    h2d_t = [e[1].elapsed_time(e[2]) / 1e3 for e in evs]
    d2h_gbps = bytes_dir / statistics.median(d2h_t) / 1e9
    h2d_gbps = bytes_dir / statistics.median(h2d_t) / 1e9
    value = 2 * bytes_dir * args.steps / wall / 1e9
    chosen = {"d2h": kvt.PATH_NAMES[pool.last_path(kvt.BACKUP)],
              "h2d": kvt.PATH_NAMES[pool.last_path(kvt.LOAD)]}
    stats = pool.stats()
    log("steps: %.2f GB/s aggregate; D2H %.2f GB/s (%s), H2D %.2f GB/s (%s)" %
        (value, d2h_gbps, chosen["d2h"], h2d_gbps, chosen["h2d"]))

    # ---- host time per call in isolation (no back-pressure): validation,
    # planning, index staging and launch/enqueue
    submit = {}
    for dname, fn in (("d2h", lambda: pool.backup(dev_b, host_idx, 0, L, s)),
                      ("h2d", lambda: pool.load(dev_l, host_idx, 0, L, s))):
        ts = []
        for _ in range(7):
            s.synchronize()
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        submit[dname] = round(statistics.median(ts) * 1e6, 1)
    s.synchronize()

    # ---- roofline of the dominant kernel (host link bound), measured live
    step_launches = {"d2h": (stats.kernel_launches[0] - stats0.kernel_launches[0]) // args.steps,
                     "h2d": (stats.kernel_launches[1] - stats0.kernel_launches[1]) // args.steps}
    timed_calls = {"d2h": (statistics.median(d2h_t), step_launches["d2h"]),
                   "h2d": (statistics.median(h2d_t), step_launches["h2d"])}
    roof = kernel_roofline(torch, kvt, pool, s, dev_b, dev_l, host_idx, L, C, R, n, args,
                           timed_calls)

    # ---- layout x path matrix at the same geometry
    matrix = []
    if not args.no_matrix:
        settle(torch, SETTLE_BYTES)       # the roofline's staging tensors were freed
        for spec in matrix_specs(torch, kvt, workloads, shape, bufs, dev_b, dev_l, host_idx):
            matrix += transfer_matrix(torch, kvt, spec, s, link_peak, calib, args)
            del spec

    pool.close()
    del bufs
    torch.cuda.empty_cache()
    extra = {}
    if not args.no_extra:
        extra["bidirectional_mixed"] = leg_bidirectional(torch, kvt, workloads, args,
                                                         link_peak, duplex_fresh)
        torch.cuda.empty_cache()
        extra["streamed_per_layer"] = leg_streamed(torch, kvt, workloads, args,
                                                   d2h_pace=calib.kernel_pace_gbps[0])
        torch.cuda.empty_cache()
        extra["ghost_list"] = leg_ghost_list(kvt, workloads)
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline: the oracle on the timed index set")
        cpu = cpu_baseline(shape, dev_b, dev_l, host_idx)
        log("cpu baseline %.3f GB/s on %d threads" % (cpu["value"], cpu["cores"]))

    pct = {d: round(100 * v / link_peak[d], 1)
           for d, v in (("h2d", h2d_gbps), ("d2h", d2h_gbps))}
    details = {
        "link_peak_measured_gbps": link_peak,
        "copy_engine_1GiB_gbps": memcpy_peak,
        "kernel_1GiB_gbps": kernel_peak,
        "workload_best_path_gbps": workload_best,
        "submit_us_per_call": submit,
        "pool_create_s": t_pool,
        "selector_calibration": {
            "kernel_gbps": list(calib.kernel_gbps), "dma_gbps": list(calib.dma_gbps),
            "staged_gather_gbps": calib.staged_gather_gbps,
            "kernel_max_workgroups": list(calib.kernel_max_workgroups),
            "kernel_pace_gbps": list(calib.kernel_pace_gbps),
            "launches_copies_per_call": {"%s/%s" % ("d2h" if d == 0 else "h2d",
                                                    kvt.PATH_NAMES[p]): list(v)
                                         for (d, p), v in ops.items()}},
        "roofline": roof,
        "cpu_baseline": cpu,
        "matrix": matrix,
        "extra": extra,
    }
    details_path = write_details(details)
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic (seeded bf16 N(0,1) KV bytes, contiguous pages at a seeded offset)",
        "config": {"workload": "mla-latent KV, 78 layers x 576 bf16 (1152 B rows), page 64, "
                               "32768-token prefix: D2H write-back then per-layer H2D load",
                   "layers": L, "components": C, "row_bytes": R, "tokens": n, "page_size": ps,
                   "host_layout": args.layout, "path": args.path,
                   "bytes_per_direction": bytes_dir},
        "h2d_gbps": round(h2d_gbps, 3),
        "d2h_gbps": round(d2h_gbps, 3),
        "path_chosen": chosen,
        "link_peak_measured_gbps": {k: round(v, 3) for k, v in link_peak.items()},
        "link_peak_definition": "best of two contiguous 1 GiB copies per direction "
                                "(copy engines, zero-copy kernel), median of 20 each",
        "pct_of_measured_peak": pct,
        "workload_best_path_gbps": {k: round(v, 3) for k, v in workload_best.items()},
        "pct_of_pcie_gen5_x16": {"h2d": round(100 * h2d_gbps / PCIE_GEN5_X16_GBPS, 1),
                                 "d2h": round(100 * d2h_gbps / PCIE_GEN5_X16_GBPS, 1)},
        "submit_us_per_call": submit,
        "roofline": compact_roofline(roof),
        "cpu_baseline": cpu,
        "details": details_path,
    }
    line = json.dumps(out)
    if len(line) > 6000:        # the driver keeps the last 8 KB of stdout
        out["roofline"].pop("other_kernel", None)
        line = json.dumps(out)
    print(line, flush=True)


def write_details(details):
    """Writes the full record (matrix, legs, calibration) next to the run's
    other outputs; returns the path, or None if it cannot be written."""
    path = os.environ.get("KV_BENCH_DETAILS",
                          os.path.join(ROOT, "gpurun_out", "bench_details.json"))
    try:
        os.makedirs(os.path.dirname(path), exist_ok=True)
        with open(path, "w") as f:
            json.dump(details, f, indent=1, default=float)
        return os.path.relpath(path, ROOT)
    except OSError as e:
        log("details not written: %s" % e)
        return None


ROOF_KEYS = ("kernel", "bound", "achieved", "peak", "unit", "frac", "traffic",
             "algorithmic_bytes_per_launch", "mean_launch_us", "launches_timed", "workgroups",
             "host_link_bytes_per_launch")


def compact_roofline(roof):
    """The roofline entries of the one-line record: the dominant kernel, the
    other direction's kernel and the staged path's device-side pass, with the
    figures that define them (the full entries are in the details file)."""
    out = {k: roof[k] for k in ROOF_KEYS if k in roof}
    out["kernel_source_hash"] = roof.get("kernel_source_hash")
    for sub in ("other_kernel", "staged_pass"):
        if roof.get(sub):
            out[sub] = {k: roof[sub][k] for k in ROOF_KEYS if k in roof[sub]}
    if roof.get("staged_pass", {}).get("scatter"):
        sc = roof["staged_pass"]["scatter"]
        out["staged_pass"]["scatter"] = {k: sc[k] for k in ("achieved", "frac", "traffic",
                                                           "mean_launch_us") if k in sc}
    return out


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("kernels.hip", "xfer_walk.hpp"):
        with open(os.path.join(ROOT, "hierarchical_kv_cache_backup_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _counter_record(kernel_name):
    path = os.path.join(ROOT, "profiles", "counters.json")
    try:
        with open(path) as f:
            return json.load(f).get(kernel_name) or {}
    except (OSError, ValueError):
        return {}


def counter_traffic(kernel_name, src_hash):
    """HBM traffic per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    rec = _counter_record(kernel_name)
    if rec.get("kernel_source_hash") != src_hash:
        return None
    return rec.get("hbm_bytes_per_launch")


def counter_link_bytes(kernel_name, src_hash):
    """Host-link bytes per launch (remote L2-to-fabric requests) from the
    committed counter summary, if taken on the current kernel source; else None."""
    link = _counter_record(kernel_name).get("link") or {}
    if link.get("kernel_source_hash") != src_hash:
        return None
    return link.get("host_link_bytes_per_launch")


KERNEL_NAMES = {"d2h": "kvt::xfer_rows<true, true, 2> (D2H gather, whole prefix in one launch, "
                       "on the default write-back grid, paced under the measured D2H link rate)",
                "h2d": "kvt::xfer_rows<false, false, 8> (H2D scatter, one launch per layer: each "
                       "layer holds more than the 16 MiB load group threshold)"}


def _roof_entry(direction, bytes_per_launch, launch_s, launches, src_hash, source):
    key = "xfer_rows_" + direction
    achieved = bytes_per_launch / launch_s / 1e9
    return {"kernel": KERNEL_NAMES[direction],
            "bound": "host_link",
            "achieved": round(achieved, 3),
            "peak": PCIE_GEN5_X16_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PCIE_GEN5_X16_GBPS, 4),
            "traffic": counter_traffic(key, src_hash),
            "host_link_bytes_per_launch": counter_link_bytes(key, src_hash),
            "algorithmic_bytes_per_launch": bytes_per_launch,
            "mean_launch_us": round(launch_s * 1e6, 2),
            "launches_timed": launches,
            "source": source,
            "hbm_secondary": {"peak": HBM_PEAK_GBPS, "frac": round(achieved / HBM_PEAK_GBPS, 5)}}


def kernel_roofline(torch, kvt, pool, s, dev_b, dev_l, host_idx, L, C, R, n, args, timed):
    """Achieved host-link GB/s of the transfer kernels: algorithmic bytes per
    launch / mean launch time, from events recorded on the stream the kernels
    are launched on.

    `timed` holds, per direction, the median call time of the timed steps and the
    kernel launches each call made there (0 when the step ran that direction on
    the copy engines). The dominant kernel is the one with the most time in the
    timed steps, its launch time taken from them (a load's launch time includes
    the gap between its per-layer launches). Each direction's kernel is also
    timed in a loop of its own with the kernel path forced, so that both are
    reported whatever path the steps took; that loop gives the dominant entry
    only when no kernel ran in the timed steps."""
    src_hash = kernel_source_hash()
    per_launch_bytes = {"d2h": n * L * C * R, "h2d": n * C * R}
    pool.set_path(kvt.PATH_KERNEL)

    def measure(fn, launches_per_call):
        for _ in range(2):
            fn()
        s.synchronize()
        durs = []
        for _ in range(max(3, args.steps)):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(s)
            fn()
            e1.record(s)
            e1.synchronize()
            durs.append(e0.elapsed_time(e1) / 1e3 / launches_per_call)
        return statistics.mean(durs), len(durs) * launches_per_call

    loop = {"d2h": measure(lambda: pool.backup(dev_b, host_idx, 0, L, s), 1),
            "h2d": measure(lambda: pool.load(dev_l, host_idx, 0, L, s), L)}
    grids = pool.stats().last_workgroups      # the kernels' grids in that loop
    entries = {}
    for dname in ("d2h", "h2d"):
        t_call, launches = timed[dname]
        if launches:
            entries[dname] = _roof_entry(dname, per_launch_bytes[dname], t_call / launches,
                                         launches * args.steps, src_hash,
                                         "timed steps (events around each call / its launches)")
        else:
            entries[dname] = _roof_entry(dname, per_launch_bytes[dname], loop[dname][0],
                                         loop[dname][1], src_hash,
                                         "loop of its own, kernel path forced (the timed steps "
                                         "ran this direction on the copy engines)")
        entries[dname]["workgroups"] = int(grids[0 if dname == "d2h" else 1])
        entries[dname]["own_loop"] = {"mean_launch_us": round(loop[dname][0] * 1e6, 2),
                                      "achieved": round(per_launch_bytes[dname] / loop[dname][0]
                                                        / 1e9, 3)}
    in_steps = [d for d in ("d2h", "h2d") if timed[d][1]]
    dominant = (max(in_steps, key=lambda d: timed[d][0]) if in_steps else "d2h")
    other = "h2d" if dominant == "d2h" else "d2h"
    roof = dict(entries[dominant])
    roof["other_kernel"] = entries[other]
    roof["staged_pass"] = staged_pass_roofline(torch, kvt, pool, s, dev_b, dev_l, L, C, R, n,
                                               args, src_hash)
    roof["kernel_source_hash"] = src_hash
    return roof


def staged_pass_roofline(torch, kvt, pool, s, dev_b, dev_l, L, C, R, n, args, src_hash):
    """The staged path's device-side pass (HBM to HBM) on the headline prefix:
    kv_stage packs the 32768 tokens x 78 layers (2.94 GB) from the device pool
    into one staging buffer, then unpacks them into the other 512 pages, one
    launch each, timed with events on the stream the pass is launched on. The
    pass reads and writes every byte once: algorithmic HBM traffic is twice
    the payload, against the 8 TB/s HBM peak."""
    payload = n * L * C * R
    stage = torch.empty(payload, dtype=torch.uint8, device="cuda:0")

    def measure(direction, idx):
        # calls back to back, an event after each: once the GPU runs behind the
        # host, the interval between two events is one call's GPU time (its
        # index copy and its launch); the first interval, which also holds the
        # host's submission of the first call, is dropped
        for _ in range(2):
            pool.stage(direction, idx, stage, 0, L, s)
        s.synchronize()
        calls = max(5, args.steps) + 1
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(calls + 1)]
        evs[0].record(s)
        for k in range(calls):
            pool.stage(direction, idx, stage, 0, L, s)
            evs[k + 1].record(s)
        evs[-1].synchronize()
        durs = [evs[k].elapsed_time(evs[k + 1]) / 1e3 for k in range(1, calls)]
        return statistics.mean(durs), len(durs)

    (tg, ng), (ts, ns) = measure(0, dev_b), measure(1, dev_l)
    del stage
    out = {}
    for key, t, cnt, what in (("stage_gather", tg, ng, "pack (gather)"),
                              ("stage_scatter", ts, ns, "unpack (scatter)")):
        achieved = 2 * payload / t / 1e9
        out[key] = {"kernel": "kvt::stage_windows<%s, true> (staged pass, %s of the whole prefix "
                              "in one launch; one 1 KiB window of the staging buffer per wave)"
                              % ("true" if key == "stage_gather" else "false", what),
                    "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                    "traffic": counter_traffic(key, src_hash),
                    "algorithmic_bytes_per_launch": 2 * payload,
                    "mean_launch_us": round(t * 1e6, 2), "launches_timed": cnt}
    entry = dict(out["stage_gather"])
    entry["scatter"] = out["stage_scatter"]
    log("staged pass: pack %.0f GB/s (%.3f of HBM peak), unpack %.0f GB/s" %
        (out["stage_gather"]["achieved"], out["stage_gather"]["frac"],
         out["stage_scatter"]["achieved"]))
    return entry


def profile_counters(torch, kvt, pool, s, dev_b, dev_l, host_idx, L):
    """Kernels for the rocprofv3 --pmc passes: a plain copy kernel of known size
    (int32 -> float32 conversion, 256 MiB read + 256 MiB written) to scale the
    counters, then two D2H and two H2D transfers on the kernel path."""
    n_el = 64 << 20
    a = torch.ones(n_el, dtype=torch.int32, device="cuda:0")
    b = torch.empty(n_el, dtype=torch.float32, device="cuda:0")
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()
    pool.set_path(kvt.PATH_KERNEL)
    for _ in range(2):
        pool.backup(dev_b, host_idx, 0, L, s)
        s.synchronize()
    for _ in range(2):
        pool.load(dev_l, host_idx, 0, L, s)
        s.synchronize()
    stage = torch.empty(dev_b.size * L * pool.geom.num_components * pool.geom.row_bytes,
                        dtype=torch.uint8, device="cuda:0")
    for direction, idx in ((0, dev_b), (1, dev_l)):
        for _ in range(2):
            pool.stage(direction, idx, stage, 0, L, s)
            s.synchronize()
    log("profile-counters: copy kernel %d bytes read + written; 2 D2H + 2 H2D transfers; "
        "2 staged packs + 2 unpacks of the prefix" % (4 * n_el))


def _counter_rows(d):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _kernel_key(name):
    return ("copy" if "elementwise_kernel" in name and "copy" in name else
            "xfer_rows_d2h" if "xfer_rows<true, true" in name else
            "xfer_rows_h2d" if "xfer_rows<false, false" in name else
            "stage_gather" if "stage_windows<true" in name else
            "stage_scatter" if "stage_windows<false" in name else None)


def summarize_link_counters(wr_dir, rd_dir):
    """Host-link bytes per launch of the transfer kernels from the L2-to-fabric
    request counters: all requests minus those bound for local DRAM are remote,
    i.e. cross the host link. Writes are 64 or 32 bytes (TCC_EA0_WRREQ_64B
    counts the 64-byte ones); reads are 128, 64 or 32 bytes (TCC_EA0_RDREQ_64B
    and _32B count the smaller ones). Remote writes are sized 64 bytes when the
    kernel's 64-byte writes cover them, else 32; remote reads 128 bytes up to the
    kernel's count of 128-byte reads, the rest 64. The plain copy kernel of known
    size (all DRAM) checks the sizes."""
    per = {}
    for d in (wr_dir, rd_dir):
        for r in _counter_rows(d):
            key = _kernel_key(r["Kernel_Name"])
            if key is None:
                continue
            per.setdefault((key, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    med = {k: statistics.median(v) for k, v in per.items()}

    def get(key, c):
        return med.get((key, c), 0.0)

    path = os.path.join(ROOT, "profiles", "counters.json")
    with open(path) as fh:
        out = json.load(fh)
    src_hash = kernel_source_hash()
    known = 4 * (64 << 20)
    copy_w = get("copy", "TCC_EA0_WRREQ_64B_sum") * 64 + (
        get("copy", "TCC_EA0_WRREQ_sum") - get("copy", "TCC_EA0_WRREQ_64B_sum")) * 32
    copy_r = (get("copy", "TCC_EA0_RDREQ_32B_sum") * 32 + get("copy", "TCC_EA0_RDREQ_64B_sum") * 64
              + (get("copy", "TCC_EA0_RDREQ_sum") - get("copy", "TCC_EA0_RDREQ_32B_sum")
                 - get("copy", "TCC_EA0_RDREQ_64B_sum")) * 128)
    for key in ("xfer_rows_d2h", "xfer_rows_h2d"):
        wr, wr_dram = get(key, "TCC_EA0_WRREQ_sum"), get(key, "TCC_EA0_WRREQ_DRAM_sum")
        wr64 = get(key, "TCC_EA0_WRREQ_64B_sum")
        rd, rd_dram = get(key, "TCC_EA0_RDREQ_sum"), get(key, "TCC_EA0_RDREQ_DRAM_sum")
        rd32, rd64 = get(key, "TCC_EA0_RDREQ_32B_sum"), get(key, "TCC_EA0_RDREQ_64B_sum")
        rd128 = rd - rd32 - rd64
        # remote writes: sized 64 B unless the kernel issued 32 B writes
        wr_remote = wr - wr_dram
        wr_remote_bytes = wr_remote * (64 if wr64 >= wr_remote else 32)
        # remote reads: the 128 B requests beyond the DRAM ones (the kernels' host
        # reads are full lines; the DRAM side holds the small index reads)
        rd_remote = rd - rd_dram
        rd_remote_128 = min(rd_remote, rd128)
        rd_remote_bytes = rd_remote_128 * 128 + (rd_remote - rd_remote_128) * 64
        rec = out.setdefault(key, {})
        rec["link"] = {"remote_write_requests": wr_remote, "remote_write_bytes": wr_remote_bytes,
                       "dram_write_requests": wr_dram,
                       "remote_read_requests": rd_remote, "remote_read_bytes": rd_remote_bytes,
                       "dram_read_requests": rd_dram,
                       "host_link_bytes_per_launch": wr_remote_bytes + rd_remote_bytes,
                       "kernel_source_hash": src_hash}
    out["link_check_copy_kernel"] = {"known_bytes_each_way": known, "write_bytes": copy_w,
                                     "read_bytes": copy_r}
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def summarize_trace(trace_dir):
    """Launch durations (End - Start) of the library's kernels in a rocprofv3
    kernel trace, grouped by kernel and grid size: dispatches, mean, min, max."""
    import csv
    import glob
    groups = {}
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                name = r["Kernel_Name"]
                if "kvt::" not in name:
                    continue
                grid = int(r.get("Grid_Size_X") or r.get("Grid_Size") or 0)
                dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                groups.setdefault((name.split("(")[0].replace("void ", ""), grid), []).append(dur)
    print("| kernel | grid (threads) | dispatches | mean ns | min ns | max ns |")
    print("|---|---|---|---|---|---|")
    for (name, grid), d in sorted(groups.items()):
        print("| %s | %d | %d | %.1f | %d | %d |" % (name, grid, len(d), statistics.mean(d),
                                                    min(d), max(d)))


def summarize_counters(fetch_dir, write_dir):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the transfer kernels, scaled by
    what the same counters read for the plain copy kernel of known size."""
    known = 4 * (64 << 20)
    out = {}
    per = {}
    for cname, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        for r in _counter_rows(d):
            if r.get("Counter_Name") != cname:
                continue
            key = _kernel_key(r["Kernel_Name"])
            if key is None:
                continue
            per.setdefault((key, cname), []).append(float(r["Counter_Value"]) * 1024.0)
    fetch_scale = known / statistics.median(per[("copy", "FETCH_SIZE")])
    write_scale = known / statistics.median(per[("copy", "WRITE_SIZE")])
    src_hash = kernel_source_hash()
    path = os.path.join(ROOT, "profiles", "counters.json")
    try:            # keep the host-link section of an earlier summary
        with open(path) as fh:
            out = json.load(fh)
    except (OSError, ValueError):
        out = {}
    for key in ("xfer_rows_d2h", "xfer_rows_h2d", "stage_gather", "stage_scatter"):
        if (key, "FETCH_SIZE") not in per:
            continue
        f = statistics.median(per[(key, "FETCH_SIZE")]) * fetch_scale
        w = statistics.median(per[(key, "WRITE_SIZE")]) * write_scale
        out.setdefault(key, {}).update(
            {"fetch_bytes_per_launch": round(f), "write_bytes_per_launch": round(w),
             "hbm_bytes_per_launch": round(f + w), "kernel_source_hash": src_hash})
    out["scale"] = {"fetch": fetch_scale, "write": write_scale,
                    "copy_kernel_bytes_each_way": known}
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


MATRIX_PATHS = (("kernel", "PATH_KERNEL"), ("kernel_lds", "PATH_KERNEL_LDS"),
                ("dma", "PATH_DMA"), ("staged", "PATH_STAGED"), ("auto", "PATH_AUTO"))


def transfer_matrix(torch, kvt, spec, s, link_peak, calib, args):
    """Layout x direction x path cells for one geometry and request. Each cell:
    GB/s from HIP events around the call on its stream (median), and GB/s from
    the host wall clock taken from entering the call to the end of a
    synchronize on an event recorded right after it (median, p10, p90), so
    that planning and submission are inside. The auto column uses the fitted
    calibration and names the path it chose."""
    L, C, R = spec["L"], spec["C"], spec["R"]
    dev_b, dev_l, host_idx = spec["dev_b"], spec["dev_l"], spec["host_idx"]
    n = host_idx.size
    bytes_dir = n * L * C * R
    rows = []
    for lname, lay in LAYOUTS.items():
        geom = kvt.geometry(L, C, R, spec["S_dev"], spec["S_host"], spec["ps"], lay)
        with kvt.KvPool(geom, spec["bufs"]) as pool:
            pool.set_calibration(calib)
            for dname, d in (("d2h", kvt.BACKUP), ("h2d", kvt.LOAD)):
                _, copies = kvt.kv_count_dma_copies(geom, dev_b, host_idx, 0, L)
                _, segs = kvt.kv_count_segments(geom, dev_b, host_idx, 0, L)
                cell = {"geometry": spec["label"], "layout": lname, "dir": dname,
                        "segments": segs, "dma_copies": copies}
                for pname, pattr in MATRIX_PATHS:
                    if pname not in spec["paths"]:
                        continue
                    pool.set_path(getattr(kvt, pattr))
                    fn = ((lambda: pool.backup(dev_b, host_idx, 0, L, s)) if d == kvt.BACKUP
                          else (lambda: pool.load(dev_l, host_idx, 0, L, s)))
                    s.synchronize()
                    t0 = time.perf_counter()
                    fn()
                    s.synchronize()
                    first = time.perf_counter() - t0
                    reps = max(3, min(20, int(args.cell_seconds / max(first, 1e-4))))
                    ts, walls = [], []
                    for _ in range(reps):
                        e0 = torch.cuda.Event(enable_timing=True)
                        e1 = torch.cuda.Event(enable_timing=True)
                        s.synchronize()
                        t0 = time.perf_counter()
                        e0.record(s)
                        fn()
                        e1.record(s)
                        e1.synchronize()
                        walls.append(time.perf_counter() - t0)
                        ts.append(e0.elapsed_time(e1) / 1e3)
                    g = bytes_dir / statistics.median(ts) / 1e9
                    q = np.percentile(np.asarray(walls), [10, 50, 90])
                    c = {"gbps": round(g, 3),
                         "pct_of_measured_peak": round(100 * g / link_peak[dname], 1),
                         "wall_gbps": round(bytes_dir / q[1] / 1e9, 3),
                         "wall_ms_p10_p50_p90": [round(x * 1e3, 3) for x in q],
                         "reps": reps}
                    if pname == "auto":
                        c["chose"] = kvt.PATH_NAMES[pool.last_path(d)]
                    cell[pname] = c
                log("matrix %s %s %s: %s" % (
                    cell["geometry"][:24], lname, dname,
                    " ".join("%s %.1f" % (k, cell[k]["gbps"]) for k, _ in MATRIX_PATHS
                             if k in cell)))
                rows.append(cell)
        settle(torch, L * C * spec["S_host"] * R)     # the pool's host memory was freed
    return rows


# After the process frees gigabytes of device or pinned host memory, the
# runtime's copies between device and host run slower for about a second
# (driver-side work after the free): write-back copies of the next cell then
# measured up to ~45% below their rate, while the library's kernels ran at
# theirs. A matrix cell measures a path, not the previous cell's teardown, so
# after such a free the matrix waits before it times anything.
SETTLE_BYTES = 1 << 30
SETTLE_S = 1.5


def settle(torch, freed_bytes):
    if freed_bytes >= SETTLE_BYTES:
        torch.cuda.synchronize()
        time.sleep(SETTLE_S)


def matrix_specs(torch, kvt, workloads, shape, bufs, dev_b, dev_l, host_idx):
    """The geometries of the layout x path matrix, one at a time (each yields its
    device buffers, which are dropped before the next):
      - the headline geometry (78 x 1152 B), 32768 tokens, contiguous pages;
      - the same, 32768 tokens from 512 random pages of the 1024;
      - a 32-layer K/V pool of 8 x 128 bf16 (2048 B rows) at 32768 tokens from
        512 random pages of 2048 (4 GiB per direction);
      - one tensor-parallel rank's share at TP 8: the K/V pool with one head
        (256 B rows), 8192 tokens from random pages; and the headline geometry
        with 4096 tokens (n/8)."""
    L, C, R, ps = shape.layers, shape.components, shape.row_bytes, shape.page_size
    base = {"L": L, "C": C, "R": R, "S_dev": shape.device_slots, "S_host": shape.host_slots,
            "ps": ps, "bufs": bufs}
    all_paths = tuple(p for p, _ in MATRIX_PATHS)
    no_lds = ("kernel", "dma", "staged", "auto")
    yield dict(base, label="mla 78x1152, 32768 tok, contiguous", dev_b=dev_b, dev_l=dev_l,
               host_idx=host_idx, paths=all_paths)
    pages_total = shape.device_slots // ps
    np_ = host_idx.size // ps
    fb = workloads.fragmented_pages(3, pages_total, np_, workloads.P_DEV)
    rest = np.setdiff1d(np.arange(pages_total), fb)
    fl = workloads.rng(3, workloads.P_RELOAD).permutation(rest)[:np_]
    yield dict(base, label="mla 78x1152, 32768 tok, random pages",
               dev_b=workloads.page_indices(fb, ps), dev_l=workloads.page_indices(fl, ps),
               host_idx=host_idx, paths=no_lds)
    k = 4096
    yield dict(base, label="mla 78x1152, 4096 tok (TP8 share of 32768)", dev_b=dev_b[:k],
               dev_l=dev_l[:k], host_idx=host_idx[:k], paths=no_lds)
    g2 = workloads.llama8b()
    for heads, tokens, label in ((8, 32768, "gqa 32x2x2048, 32768 tok, random pages"),
                                 (1, 8192, "gqa 32x2x256 (TP8 share), 8192 tok, random pages")):
        sh = g2.scaled(heads=heads, host_slots=tokens)
        b2 = []
        for l in range(sh.layers):
            for c in range(sh.components):
                t = torch.empty(sh.device_slots * sh.row_bytes, dtype=torch.uint8,
                                device="cuda:0")
                workloads.fill_device_buffer(t, sh, 2, l, c, torch)
                b2.append(t)
        tot = sh.device_slots // sh.page_size
        npg = tokens // sh.page_size
        pb = workloads.fragmented_pages(2, tot, npg, workloads.P_DEV)
        rest = np.setdiff1d(np.arange(tot), pb)
        pl = workloads.rng(2, workloads.P_RELOAD).permutation(rest)[:npg]
        yield {"L": sh.layers, "C": sh.components, "R": sh.row_bytes, "S_dev": sh.device_slots,
               "S_host": tokens, "ps": sh.page_size, "bufs": b2, "label": label,
               "dev_b": workloads.page_indices(pb, sh.page_size),
               "dev_l": workloads.page_indices(pl, sh.page_size),
               "host_idx": np.arange(tokens, dtype=np.int64), "paths": no_lds}
        freed = sum(b.numel() for b in b2)
        del b2
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        settle(torch, freed)


def _ev(torch):
    return torch.cuda.Event(enable_timing=True)


def _duplex_peak(torch, kvt):
    """Concurrent contiguous H2D and D2H of 1 GiB each, issued through the library
    (layer_first, 2 layers x 512 MiB per direction, one pool per direction, two
    streams), for every pairing of copy engines and kernels. Returns the best
    aggregate GB/s (2 GiB / span of both) and the per-pairing figures. Both calls
    only enqueue, so one thread issues them."""
    R, S = 4096, 131072                       # 512 MiB per layer buffer
    bufs = [torch.empty(S * R, dtype=torch.uint8, device="cuda:0") for _ in range(4)]
    geom = kvt.geometry(2, 1, R, S, S, 64, 0)
    pa, pb = kvt.KvPool(geom, bufs[:2]), kvt.KvPool(geom, bufs[2:])
    idx = np.arange(S, dtype=np.int64)
    sa, sb = kvt.Stream(), kvt.Stream()                # a hardware queue each
    nb = 2 * S * R
    pairs = {}
    for h_name, h_path in (("dma", kvt.PATH_DMA), ("kernel", kvt.PATH_KERNEL)):
        for d_name, d_path in (("dma", kvt.PATH_DMA), ("kernel", kvt.PATH_KERNEL)):
            pa.set_path(h_path)
            pb.set_path(d_path)
            best = None
            for _ in range(3):
                torch.cuda.synchronize()
                e = [_ev(torch) for _ in range(4)]
                e[0].record(sa.torch)
                pa.load(idx, idx, 0, 2, sa)
                e[1].record(sa.torch)
                e[2].record(sb.torch)
                pb.backup(idx, idx, 0, 2, sb)
                e[3].record(sb.torch)
                torch.cuda.synchronize()
                start = min(0.0, e[0].elapsed_time(e[2]))
                end = max(e[0].elapsed_time(e[1]), e[0].elapsed_time(e[3]))
                r = {"h2d_gbps": round(nb / (e[0].elapsed_time(e[1]) / 1e3) / 1e9, 2),
                     "d2h_gbps": round(nb / (e[2].elapsed_time(e[3]) / 1e3) / 1e9, 2),
                     "aggregate_gbps": round(2 * nb / ((end - start) / 1e3) / 1e9, 2)}
                if best is None or r["aggregate_gbps"] > best["aggregate_gbps"]:
                    best = r
            pairs["h2d_%s+d2h_%s" % (h_name, d_name)] = best
    pa.close()
    pb.close()
    sa.close()
    sb.close()
    del bufs
    torch.cuda.empty_cache()
    log("duplex pairings %s" % json.dumps(pairs)[:160])
    return max(v["aggregate_gbps"] for v in pairs.values()), pairs


def leg_bidirectional(torch, kvt, workloads, args, link_peak, duplex_fresh):
    """Mixed batch: 64 requests, lognormal lengths (median 4096, sigma 1.0, max
    32768), 32 layers x K/V x 2048 B rows, page 64. The L2 hits (82% of each
    request, whole pages) load H2D on one stream from one caller thread while
    the new pages write back D2H on another stream from a second thread.

    Bound: the two volumes are unequal (H2D ~4.4x D2H), so no schedule beats
    wall_min = max(h2d_bytes / h2d_peak, d2h_bytes / d2h_peak,
    (h2d_bytes + d2h_bytes) / duplex_peak), with the one-direction peaks of the
    1 GiB copy-engine copies and the duplex peak of the fresh process."""
    import threading
    shape = workloads.mixed()
    plan = workloads.mixed_plan(shape, 4)
    L, C, R, ps = shape.layers, shape.components, shape.row_bytes, shape.page_size
    S = plan["device_slots"]
    h_dev, h_host = plan["h2d"]
    w_dev, w_host = plan["d2h"]
    t0 = time.perf_counter()
    bufs = []
    for l in range(L):
        for c in range(C):
            b = torch.empty(S * R, dtype=torch.uint8, device="cuda:0")
            workloads.fill_device_buffer(b, shape, 4, l, c, torch)
            bufs.append(b)
    # the two directions on streams with a hardware queue each: on one queue
    # they would run one after the other
    s_load, s_back = kvt.Stream(), kvt.Stream()
    log("bidirectional: setup %.1fs, %d requests, %.1f GB H2D, %.1f GB D2H" %
        (time.perf_counter() - t0, plan["lens"].size, h_dev.size * L * C * R / 1e9,
         w_dev.size * L * C * R / 1e9))
    hb = h_dev.size * L * C * R
    wb = w_dev.size * L * C * R
    peak_here, pairs_here = _duplex_peak(torch, kvt)
    peak, pairs = duplex_fresh
    peak = max(peak, peak_here)
    wall_min = max(hb / link_peak["h2d"], wb / link_peak["d2h"], (hb + wb) / peak) / 1e9
    bound = (hb + wb) / wall_min / 1e9
    results = {}
    # "no_duplex_caps": the duplex grid caps switched off (the load then runs
    # on a full grid; the write-back keeps its own default cap), to show what
    # the caps buy
    variants = (("layer_first", 0, "kernel", kvt.PATH_KERNEL, True),
                ("layer_first", 0, "kernel_no_duplex_caps", kvt.PATH_KERNEL, False),
                ("layer_first", 0, "auto", kvt.PATH_AUTO, True),
                ("page_first_direct", 2, "kernel", kvt.PATH_KERNEL, True),
                ("page_first_direct", 2, "staged", kvt.PATH_STAGED, True),
                ("page_first_direct", 2, "auto", kvt.PATH_AUTO, True),
                ("page_first_direct", 2, "auto_no_duplex_caps", kvt.PATH_AUTO, False))
    for lname, lay, pname, p, caps in variants:
        pool = kvt.KvPool(kvt.geometry(L, C, R, S, plan["host_slots"], ps, lay), bufs,
                          flags=kvt.F_CHECK_UNIQUE | kvt.F_DUPLEX)
        pool.set_path(kvt.PATH_KERNEL)
        pool.backup(h_dev, h_host, 0, L, s_back)      # L2 holds the hits
        s_back.synchronize()
        if not caps:
            cal = pool.calibration()
            cal.duplex_kernel_max_workgroups[:] = [0, 0]
            pool.set_calibration(cal)
        pool.set_path(p)
        load = lambda: pool.load(h_dev, h_host, 0, L, s_load)
        back = lambda: pool.backup(w_dev, w_host, 0, L, s_back)

        def alone(fn, st):
            fn()
            st.synchronize()
            e0, e1 = _ev(torch), _ev(torch)
            e0.record(st.torch)
            fn()
            e1.record(st.torch)
            e1.synchronize()
            return e0.elapsed_time(e1) / 1e3

        t_load = alone(load, s_load)
        t_back = alone(back, s_back)
        walls, h_rates, d_rates = [], [], []
        for rep in range(1 + 3):
            go = threading.Barrier(3)
            ev = [_ev(torch) for _ in range(4)]

            def run_load():
                go.wait()
                ev[0].record(s_load.torch)
                load()
                ev[1].record(s_load.torch)

            def run_back():
                go.wait()
                ev[2].record(s_back.torch)
                back()
                ev[3].record(s_back.torch)

            th = [threading.Thread(target=run_load), threading.Thread(target=run_back)]
            for x in th:
                x.start()
            torch.cuda.synchronize()
            go.wait()
            t1 = time.perf_counter()
            for x in th:
                x.join()
            s_load.synchronize()
            s_back.synchronize()
            wall = time.perf_counter() - t1
            if rep == 0:
                continue
            walls.append(wall)
            h_rates.append(hb / (ev[0].elapsed_time(ev[1]) / 1e3) / 1e9)
            d_rates.append(wb / (ev[2].elapsed_time(ev[3]) / 1e3) / 1e9)
        wall = statistics.median(walls)
        agg = (hb + wb) / wall / 1e9
        key = "%s/%s" % (lname, pname)
        st = pool.stats()
        kpaths = (kvt.PATH_KERNEL, kvt.PATH_KERNEL_LDS)
        grid = lambda d: int(st.last_workgroups[d]) if pool.last_path(d) in kpaths else None
        results[key] = {"paths_used": {"h2d": kvt.PATH_NAMES[pool.last_path(kvt.LOAD)],
                                       "d2h": kvt.PATH_NAMES[pool.last_path(kvt.BACKUP)]},
                        "kernel_workgroups": {"h2d": grid(kvt.LOAD), "d2h": grid(kvt.BACKUP)},
                        "h2d_alone_gbps": round(hb / t_load / 1e9, 3),
                        "d2h_alone_gbps": round(wb / t_back / 1e9, 3),
                        "h2d_concurrent_gbps": round(statistics.median(h_rates), 3),
                        "d2h_concurrent_gbps": round(statistics.median(d_rates), 3),
                        "aggregate_gbps": round(agg, 3),
                        "pct_of_bound": round(100 * agg / bound, 1)}
        log("bidirectional %s %s" % (key, json.dumps(results[key])[:140]))
        pool.close()
    s_load.close()
    s_back.close()
    del bufs
    torch.cuda.empty_cache()
    best = max(results, key=lambda k: results[k]["aggregate_gbps"])
    return {"workload": "64 requests, lognormal lengths (median 4096, sigma 1.0), 32 layers x "
                        "K/V x 2048 B, page 64, hits 0.82 H2D || new D2H, two threads, pool "
                        "flagged KV_F_DUPLEX",
            "tokens": int(S), "h2d_bytes": int(hb), "d2h_bytes": int(wb),
            "duplex_peak_gbps": round(peak, 3),
            "duplex_pairings_1GiB_fresh": pairs,
            "duplex_pairings_1GiB_beside_pools": pairs_here,
            "bound_gbps": round(bound, 3),
            "bound": "max(h2d/h2d_peak, d2h/d2h_peak, (h2d+d2h)/duplex_peak) as wall time",
            "best": best, "aggregate_gbps": results[best]["aggregate_gbps"],
            "variants": results}


def leg_streamed(torch, kvt, workloads, args, d2h_pace=0.0):
    """Per-layer streamed load: 61 layers x K/V x 1024 B fp8 rows, 131072-token
    prefix (256 MiB per layer). Layer l+1 loads on a side stream while a
    synthetic HBM-bound consumer reads layer l's whole K and V buffers on the
    compute stream, after kv_load_layer(l). The consumer repeats its pass k times
    so that its time per layer matches the transfer's. Then write-backs beside
    the consumer, the kernel's on the library's default grid paced to d2h_pace
    GB/s (the run's measured pace; 0 keeps the library's)."""
    shape = workloads.streamed()
    L, C, R, ps = shape.layers, shape.components, shape.row_bytes, shape.page_size
    S, n = shape.device_slots, shape.extra["tokens"]
    dev_idx, host_idx = workloads.prefix_indices(shape, 5, n, fragmented=False)
    bufs = []
    for l in range(L):
        for c in range(C):
            b = torch.empty(S * R, dtype=torch.uint8, device="cuda:0")
            workloads.fill_device_buffer(b, shape, 5, l, c, torch)
            bufs.append(b)
    s_load, s_comp = kvt.Stream(), torch.cuda.Stream()   # loads on a queue of their own
    layer_bytes = n * C * R
    acc = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    torch.cuda.synchronize()   # the fill above ran on the default stream; acc is used on s_comp

    def consume(l, k):
        for _ in range(k):
            for c in range(C):
                acc.add_(bufs[l * C + c].view(torch.int64).sum())

    # one consumer pass over a layer (both buffers), alone
    with torch.cuda.stream(s_comp):
        consume(0, 2)
        s_comp.synchronize()
        e0, e1 = _ev(torch), _ev(torch)
        e0.record(s_comp)
        consume(0, 10)
        e1.record(s_comp)
        e1.synchronize()
    t_pass = e0.elapsed_time(e1) / 1e3 / 10
    results = {}
    pfd = kvt.PAGE_FIRST_DIRECT
    variants = (("kernel", kvt.PATH_KERNEL, 0, 0),
                ("kernel_overlap_flag", kvt.PATH_KERNEL, kvt.F_LOAD_OVERLAP, 0),
                ("dma", kvt.PATH_DMA, 0, 0), ("staged", kvt.PATH_STAGED, 0, 0),
                ("auto_overlap_flag", kvt.PATH_AUTO, kvt.F_LOAD_OVERLAP, 0),
                ("page_first_direct/kernel_overlap_flag", kvt.PATH_KERNEL, kvt.F_LOAD_OVERLAP, pfd),
                ("page_first_direct/auto_overlap_flag", kvt.PATH_AUTO, kvt.F_LOAD_OVERLAP, pfd))
    for pname, p, extra_flags, lay in variants:
        geom = kvt.geometry(L, C, R, S, shape.host_slots, ps, lay)
        pool = kvt.KvPool(geom, bufs, flags=kvt.F_CHECK_UNIQUE | extra_flags)
        pool.backup(dev_idx, host_idx, 0, L, s_load)       # L2 holds the prefix
        s_load.synchronize()
        pool.set_path(p)
        pool.load(dev_idx, host_idx, 0, L, s_load)
        s_load.synchronize()
        e0, e1 = _ev(torch), _ev(torch)
        e0.record(s_load.torch)
        pool.load(dev_idx, host_idx, 0, L, s_load)
        e1.record(s_load.torch)
        e1.synchronize()
        t_h2d = e0.elapsed_time(e1) / 1e3
        k = max(1, round(t_h2d / L / t_pass))
        with torch.cuda.stream(s_comp):
            e0, e1 = _ev(torch), _ev(torch)
            e0.record(s_comp)
            for l in range(L):
                consume(l, k)
            e1.record(s_comp)
            e1.synchronize()
        t_comp = e0.elapsed_time(e1) / 1e3
        walls, h2d_ov, comp_ov = [], [], []
        for rep in range(3):
            torch.cuda.synchronize()
            ev = [_ev(torch) for _ in range(3)]
            lev = [(_ev(torch), _ev(torch)) for _ in range(L)]
            ev[0].record(s_load.torch)
            s_comp.wait_event(ev[0])
            pool.load(dev_idx, host_idx, 0, L, s_load)
            ev[1].record(s_load.torch)
            with torch.cuda.stream(s_comp):
                for l in range(L):
                    pool.load_layer(l, s_comp)
                    lev[l][0].record(s_comp)          # layer l has landed
                    consume(l, k)
                    lev[l][1].record(s_comp)
                ev[2].record(s_comp)
            ev[2].synchronize()
            s_load.synchronize()
            walls.append(ev[0].elapsed_time(ev[2]) / 1e3)
            h2d_ov.append(L * layer_bytes / (ev[0].elapsed_time(ev[1]) / 1e3) / 1e9)
            comp_ov.append(sum(a.elapsed_time(b) for a, b in lev) / 1e3)
        wall = statistics.median(walls)
        eta = (t_h2d + t_comp - wall) / min(t_h2d, t_comp)
        results[pname] = {"path_used": kvt.PATH_NAMES[pool.last_path(kvt.LOAD)],
                          "h2d_alone_gbps": round(L * layer_bytes / t_h2d / 1e9, 3),
                          "h2d_overlapped_gbps": round(statistics.median(h2d_ov), 3),
                          "compute_reps_per_layer": k,
                          "sum_h2d_ms": round(t_h2d * 1e3, 2),
                          "sum_compute_ms": round(t_comp * 1e3, 2),
                          "sum_compute_overlapped_ms": round(statistics.median(comp_ov) * 1e3, 2),
                          "compute_slowdown": round(statistics.median(comp_ov) / t_comp, 3),
                          "wall_ms": round(wall * 1e3, 2),
                          "overlap_efficiency": round(eta, 3)}
        log("streamed %s %s" % (pname, json.dumps(results[pname])[:140]))
        pool.close()

    # Write-back beside compute: layers 1..60 written back while the consumer
    # repeats its pass over layer 0 (60 passes); the consumer's time against its
    # time alone, per path and write-back grid.
    writeback = {}
    geom = kvt.geometry(L, C, R, S, shape.host_slots, ps, 0)
    pool = kvt.KvPool(geom, bufs)

    def consume_timed(reps):
        with torch.cuda.stream(s_comp):
            e0, e1 = _ev(torch), _ev(torch)
            e0.record(s_comp)
            consume(0, reps)
            e1.record(s_comp)
            e1.synchronize()
        return e0.elapsed_time(e1) / 1e3

    t_alone = statistics.median([consume_timed(60) for _ in range(3)])
    wb_bytes = n * (L - 1) * C * R
    for wname, p, cap in (("kernel_default_grid", kvt.PATH_KERNEL, None),
                          ("kernel_full_grid", kvt.PATH_KERNEL, 0),
                          ("dma", kvt.PATH_DMA, None), ("staged", kvt.PATH_STAGED, None)):
        pool.set_path(p)
        cal = pool.calibration()
        if cap is not None:
            cal.kernel_max_workgroups[0] = cap
        if d2h_pace:
            cal.kernel_pace_gbps[0] = d2h_pace
        pool.set_calibration(cal)
        slow, rates = [], []
        for rep in range(3):
            torch.cuda.synchronize()
            e0, e1 = _ev(torch), _ev(torch)
            e0.record(s_load.torch)
            pool.backup(dev_idx, host_idx, 1, L, s_load)
            e1.record(s_load.torch)
            slow.append(consume_timed(60) / t_alone)
            e1.synchronize()
            rates.append(wb_bytes / (e0.elapsed_time(e1) / 1e3) / 1e9)
        st = pool.stats()
        writeback[wname] = {"path_used": kvt.PATH_NAMES[pool.last_path(kvt.BACKUP)],
                            "workgroups": (int(st.last_workgroups[0]) if p == kvt.PATH_KERNEL
                                           else None),
                            "d2h_gbps_beside_compute": round(statistics.median(rates), 3),
                            "compute_slowdown": round(statistics.median(slow), 3)}
        log("streamed write-back %s %s" % (wname, json.dumps(writeback[wname])[:140]))
    pool.close()
    s_load.close()
    del bufs
    torch.cuda.empty_cache()
    return {"workload": "61 layers x K/V x 1024 B (fp8 random bytes), 131072-token prefix, "
                        "per-layer H2D overlapped with an HBM-bound consumer; host layout "
                        "layer_first unless the variant names page_first_direct",
            "layer_bytes": layer_bytes, "consumer_pass_ms": round(t_pass * 1e3, 3),
            "paths": results,
            "write_back_beside_compute": {
                "workload": "layers 1..60 written back (15.8 GB) while the consumer repeats "
                            "its pass over layer 0 60 times; slowdown against the consumer "
                            "alone", "consumer_alone_ms": round(t_alone * 1e3, 3),
                "paths": writeback}}


def overlap_study(torch, kvt, workloads, layers=24, with_loads=True):
    """The kernel path's grid beside an HBM-bound consumer, on the streamed
    workload's first `layers` layers (256 MiB each, K and V): (1) a per-layer
    load flagged KV_F_LOAD_OVERLAP, overlapped layer by layer with the consumer
    (as in the streamed leg), for overlap grid caps of 32 to 256 workgroups and
    the full grid; (2) a write-back of layers 1.. beside the consumer's repeated
    pass over layer 0, for write-back caps of 8 to 64 and the full grid, and
    for capped grids paced to a set rate (kernel_pace_gbps); and the copy path
    for both, as reference. with_loads=False skips (1)."""
    shape = workloads.streamed()
    L, C, R, ps = layers, shape.components, shape.row_bytes, shape.page_size
    S, n = shape.device_slots, shape.extra["tokens"]
    dev_idx, host_idx = workloads.prefix_indices(shape, 5, n, fragmented=False)
    bufs = []
    for l in range(L):
        for c in range(C):
            b = torch.empty(S * R, dtype=torch.uint8, device="cuda:0")
            workloads.fill_device_buffer(b, shape, 5, l, c, torch)
            bufs.append(b)
    s_load, s_comp = kvt.Stream(), torch.cuda.Stream()
    acc = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    torch.cuda.synchronize()
    layer_bytes = n * C * R

    def consume(l, k):
        for _ in range(k):
            for c in range(C):
                acc.add_(bufs[l * C + c].view(torch.int64).sum())

    def timed_consume(l, k):
        with torch.cuda.stream(s_comp):
            e0, e1 = _ev(torch), _ev(torch)
            e0.record(s_comp)
            consume(l, k)
            e1.record(s_comp)
            e1.synchronize()
        return e0.elapsed_time(e1) / 1e3

    timed_consume(0, 2)
    t_pass = timed_consume(0, 10) / 10
    geom = kvt.geometry(L, C, R, S, shape.host_slots, ps, 0)
    loads, backs = {}, {}
    with kvt.KvPool(geom, bufs, flags=kvt.F_CHECK_UNIQUE | kvt.F_LOAD_OVERLAP) as pool:
        pool.set_path(kvt.PATH_KERNEL)
        pool.backup(dev_idx, host_idx, 0, L, s_load)
        s_load.synchronize()
        load_cells = [(cap, ex) for ex in (1, 0) for cap in (8, 16, 24, 32, 48, 96)]
        load_cells += [(0, 0), ("dma", 0)]
        for cap, ex in load_cells if with_loads else ():
            cal = pool.calibration()
            if cap == "dma":
                pool.set_path(kvt.PATH_DMA)
            else:
                cal.overlap_kernel_max_workgroups = cap
                cal.kernel_cu_exclusive[1] = ex
                pool.set_calibration(cal)
            pool.load(dev_idx, host_idx, 0, L, s_load)
            s_load.synchronize()
            e0, e1 = _ev(torch), _ev(torch)
            e0.record(s_load.torch)
            pool.load(dev_idx, host_idx, 0, L, s_load)
            e1.record(s_load.torch)
            e1.synchronize()
            t_h2d = e0.elapsed_time(e1) / 1e3
            k = max(1, round(t_h2d / L / t_pass))
            t_comp = sum(timed_consume(l, k) for l in range(L))
            walls, rates, comp = [], [], []
            for rep in range(3):
                torch.cuda.synchronize()
                ev = [_ev(torch) for _ in range(3)]
                lev = [(_ev(torch), _ev(torch)) for _ in range(L)]
                ev[0].record(s_load.torch)
                s_comp.wait_event(ev[0])
                pool.load(dev_idx, host_idx, 0, L, s_load)
                ev[1].record(s_load.torch)
                with torch.cuda.stream(s_comp):
                    for l in range(L):
                        pool.load_layer(l, s_comp)
                        lev[l][0].record(s_comp)
                        consume(l, k)
                        lev[l][1].record(s_comp)
                    ev[2].record(s_comp)
                ev[2].synchronize()
                s_load.synchronize()
                walls.append(ev[0].elapsed_time(ev[2]) / 1e3)
                rates.append(L * layer_bytes / (ev[0].elapsed_time(ev[1]) / 1e3) / 1e9)
                comp.append(sum(a.elapsed_time(b) for a, b in lev) / 1e3)
            wall = statistics.median(walls)
            key = "dma" if cap == "dma" else ("full" if cap == 0 else
                                               str(cap) + (" cu-exclusive" if ex else ""))
            loads[key] = {"h2d_alone_gbps": round(L * layer_bytes / t_h2d / 1e9, 2),
                          "h2d_overlapped_gbps": round(statistics.median(rates), 2),
                          "compute_slowdown": round(statistics.median(comp) / t_comp, 3),
                          "overlap_efficiency": round((t_h2d + t_comp - wall) / min(t_h2d, t_comp), 3)}
            log("overlap study load %s %s" % (key, json.dumps(loads[key])))
        pool.set_path(kvt.PATH_KERNEL)
        t_alone = statistics.median([timed_consume(0, 40) for _ in range(3)])
        wb_bytes = n * (L - 1) * C * R
        # (grid cap, pace, burst blocks, a compute unit per workgroup, lane depth)
        plain = [(cap, 0.0, 0, 0, 2) for cap in (8, 12, 16, 18, 20, 24, 32)]
        plain += [(cap, 0.0, 0, 0, 8) for cap in (4, 6, 8, 10, 12)]
        plain += [(cap, 0.0, 0, 0, 1) for cap in (16, 32)]
        plain += [(0, 0.0, 0, 0, 2)]
        paced = [(cap, gbps, 32, 0, 2) for cap in (14, 16, 18, 20, 24, 28)
                 for gbps in (54.0, 56.0)]
        paced += [(cap, gbps, 32, 0, 8) for cap in (8, 9, 10, 12) for gbps in (54.0, 56.0)]
        paced += [(cap, gbps, 32, 0, 1) for cap in (32, 36, 40, 48) for gbps in (54.0, 56.0)]
        paced += [(cap, 56.0, 32, 0, 4) for cap in (10, 12, 14)]
        paced += [(18, 54.0, 32, 1, 2), (9, 54.0, 32, 1, 8)]
        for cap, pace, burst, ex, depth in plain + paced + [("dma", 0.0, 0, 0, 2)]:
            cal = pool.calibration()
            if cap == "dma":
                pool.set_path(kvt.PATH_DMA)
            else:
                cal.kernel_max_workgroups[0] = cap
                cal.kernel_pace_gbps[0] = pace
                cal.kernel_pace_burst_blocks[0] = burst
                cal.kernel_cu_exclusive[0] = ex
                cal.kernel_lane_depth[0] = depth
                pool.set_calibration(cal)
            slow, rates = [], []
            for rep in range(3):
                torch.cuda.synchronize()
                e0, e1 = _ev(torch), _ev(torch)
                e0.record(s_load.torch)
                pool.backup(dev_idx, host_idx, 1, L, s_load)
                e1.record(s_load.torch)
                slow.append(timed_consume(0, 40) / t_alone)
                e1.synchronize()
                rates.append(wb_bytes / (e0.elapsed_time(e1) / 1e3) / 1e9)
            key = "dma" if cap == "dma" else ("full" if cap == 0 else str(cap))
            if cap != "dma":
                key += " depth %d" % depth
            if pace:
                key += " paced %g burst %d" % (pace, burst)
            if cap not in ("dma", 0) and ex:
                key += " cu-exclusive"
            backs[key] = {"d2h_gbps_beside_compute": round(statistics.median(rates), 2),
                          "compute_slowdown": round(statistics.median(slow), 3)}
            log("overlap study write-back %s %s" % (key, json.dumps(backs[key])))
    s_load.close()
    return {"study": "kernel-path grid beside an HBM-bound consumer (torch int64 sums of "
                     "each layer's K and V)",
            "workload": "%d layers x K/V x 1024 B fp8, 131072-token prefix, layer_first" % L,
            "consumer_pass_ms": round(t_pass * 1e3, 3),
            "load_overlap_caps": loads, "write_back_caps": backs}


# ---- interference counters: a transfer in one process, the consumer in another

# The loader's variants, in the order the consumer asks for them: a label, the
# load path, the grid cap of a load flagged KV_F_LOAD_OVERLAP (None: the pool's
# default overlap grid; 0: full grid) and whether a capped load's workgroups
# take compute units of their own (kernel_cu_exclusive[1]; None: the default).
INTERFERENCE_VARIANTS = (("kernel_overlap_grid", "PATH_KERNEL", None, None),
                         ("kernel_overlap_grid_shared_cus", "PATH_KERNEL", None, 0),
                         ("kernel_full_grid", "PATH_KERNEL", 0, None),
                         ("dma", "PATH_DMA", None, None))
INTERFERENCE_WAIT_S = 120.0
INTERFERENCE_LAYERS = 8


def _await_file(path, deadline_s=INTERFERENCE_WAIT_S):
    t0 = time.monotonic()
    while not os.path.exists(path):
        if time.monotonic() - t0 > deadline_s:
            raise TimeoutError("no %s after %.0f s" % (path, deadline_s))
        time.sleep(0.002)
    with open(path) as f:
        return f.read()


def _put_file(path, text=""):
    tmp = path + ".tmp"
    with open(tmp, "w") as f:
        f.write(text)
    os.replace(tmp, path)


def interference_loader(torch, kvt, workloads, d):
    """The transfer side of the interference counter study, in a process of its
    own so that the profiler's per-dispatch counter collection in the consumer's
    process does not serialize it. On the streamed workload's first
    INTERFERENCE_LAYERS layers (256 MiB each, K and V, 1024 B rows, 131072-token
    prefix, layer_first): for each variant, wait for DIR/go.<name>, then issue
    per-layer loads of the whole range back to back on a queue of its own until
    DIR/stop.<name> appears; write DIR/running.<name> once the first load has
    landed and DIR/stopped.<name> (the loads' GB/s) at the end. Every wait ends
    after INTERFERENCE_WAIT_S seconds."""
    shape = workloads.streamed()
    L, C, R, ps = INTERFERENCE_LAYERS, shape.components, shape.row_bytes, shape.page_size
    S, n = shape.device_slots, shape.extra["tokens"]
    dev_idx, host_idx = workloads.prefix_indices(shape, 5, n, fragmented=False)
    bufs = []
    for l in range(L):
        for c in range(C):
            b = torch.empty(S * R, dtype=torch.uint8, device="cuda:0")
            workloads.fill_device_buffer(b, shape, 5, l, c, torch)
            bufs.append(b)
    torch.cuda.synchronize()
    s = kvt.Stream()
    geom = kvt.geometry(L, C, R, S, shape.host_slots, ps, 0)
    load_bytes = n * L * C * R
    with kvt.KvPool(geom, bufs, flags=kvt.F_CHECK_UNIQUE | kvt.F_LOAD_OVERLAP) as pool:
        pool.set_path(kvt.PATH_KERNEL)
        pool.backup(dev_idx, host_idx, 0, L, s)
        s.synchronize()
        default_cal = pool.calibration()
        _put_file(os.path.join(d, "loader_ready"))
        for name, path, cap, exclusive in INTERFERENCE_VARIANTS:
            _await_file(os.path.join(d, "go." + name))
            cal = pool.calibration()
            cal.overlap_kernel_max_workgroups = (default_cal.overlap_kernel_max_workgroups
                                                 if cap is None else cap)
            cal.kernel_cu_exclusive[1] = (default_cal.kernel_cu_exclusive[1]
                                          if exclusive is None else exclusive)
            pool.set_calibration(cal)
            pool.set_path(getattr(kvt, path))
            pool.load(dev_idx, host_idx, 0, L, s)
            s.synchronize()
            _put_file(os.path.join(d, "running." + name))
            stop = os.path.join(d, "stop." + name)
            t0, loads = time.perf_counter(), 0
            while not os.path.exists(stop):
                pool.load(dev_idx, host_idx, 0, L, s)
                s.synchronize()
                loads += 1
                if time.perf_counter() - t0 > INTERFERENCE_WAIT_S:
                    raise TimeoutError("no %s" % stop)
            dt = time.perf_counter() - t0
            st = pool.stats()
            rec = {"variant": name, "path_used": kvt.PATH_NAMES[pool.last_path(kvt.LOAD)],
                   "workgroups": int(st.last_workgroups[1]) if path == "PATH_KERNEL" else None,
                   "cu_exclusive": (bool(cal.kernel_cu_exclusive[1])
                                    if path == "PATH_KERNEL" and cal.overlap_kernel_max_workgroups > 0
                                    else None),
                   "loads": loads, "h2d_gbps": round(loads * load_bytes / dt / 1e9, 3)}
            log("interference loader %s" % json.dumps(rec))
            _put_file(os.path.join(d, "stopped." + name), json.dumps(rec))
    s.close()


def interference_consumer(torch, d, reps=40):
    """The compute side, run under rocprofv3 --pmc: an HBM-bound consumer (torch
    int64 sums over two 256 MiB buffers, one reduction kernel each) runs `reps`
    passes alone, then beside each of the loader's variants (asked for and
    released through files in DIR), then alone again. DIR/consumer.json lists
    the phases in order with their reduction dispatches, so that the counter
    rows can be split by phase (the profiler serializes this process's
    dispatches, not the loader's)."""
    bufs = [torch.randint(0, 1 << 30, (32 << 20,), dtype=torch.int64, device="cuda:0")
            for _ in range(2)]
    acc = torch.zeros(1, dtype=torch.int64, device="cuda:0")

    def passes(k):
        for _ in range(k):
            for b in bufs:
                acc.add_(b.sum())
        torch.cuda.synchronize()

    phases = []

    def phase(name, k):
        t0 = time.perf_counter()
        passes(k)
        phases.append({"phase": name, "reduce_dispatches": k * len(bufs),
                       "wall_s": round(time.perf_counter() - t0, 4)})

    phase("warmup", 4)
    _await_file(os.path.join(d, "loader_ready"))
    phase("alone_before", reps)
    loader = {}
    for name, _, _, _ in INTERFERENCE_VARIANTS:
        _put_file(os.path.join(d, "go." + name))
        _await_file(os.path.join(d, "running." + name))
        phase(name, reps)
        _put_file(os.path.join(d, "stop." + name))
        loader[name] = json.loads(_await_file(os.path.join(d, "stopped." + name)))
    phase("alone_after", reps)
    out = {"consumer": "torch int64 sum over 2 x 256 MiB, %d passes per phase" % reps,
           "phases": phases, "loader": loader}
    _put_file(os.path.join(d, "consumer.json"), json.dumps(out, indent=1))
    return out


# per-dispatch ratios the summary derives: name -> (numerator, denominator)
INTERFERENCE_RATIOS = {
    "ea_read_latency_cycles": ("TCC_EA0_RDREQ_LEVEL_sum", "TCC_EA0_RDREQ_sum"),
    "tcp_tcc_read_latency_cycles": ("TCP_TCC_READ_REQ_LATENCY_sum", "TCP_TCC_READ_REQ_sum"),
}


def summarize_interference(dirs):
    """Per-phase medians of the consumer's reduction dispatches over one or
    more --interference-consumer directories (one rocprofv3 --pmc pass each,
    with --kernel-trace): every counter, the launch duration, and the derived
    ratios (EA read latency = TCC_EA0_RDREQ_LEVEL / TCC_EA0_RDREQ; L1-to-L2 read
    latency = TCP_TCC_READ_REQ_LATENCY / TCP_TCC_READ_REQ), each taken per
    dispatch. The reduction kernel is torch's reduce_kernel (the most frequent
    one, if several); its dispatches, in dispatch order, are cut into the phases
    DIR/consumer.json lists, and a count that differs from the list's is
    refused."""
    import csv
    import glob
    table = {}
    order = []
    loader = {}
    for d in dirs:
        with open(os.path.join(d, "consumer.json")) as f:
            meta = json.load(f)
        loader.update(meta["loader"])
        per_dispatch = {}
        names = {}
        for r in _counter_rows(d):
            did = int(r.get("Dispatch_Id") or r["Correlation_Id"])
            per_dispatch.setdefault(did, {})[r["Counter_Name"]] = float(r["Counter_Value"])
            names[did] = r["Kernel_Name"]
        durations = {}
        for f in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    did = int(r.get("Dispatch_Id") or r["Correlation_Id"])
                    durations[did] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        counts = {}
        for did, name in names.items():
            counts[name] = counts.get(name, 0) + 1
        reduce_name = max(counts, key=lambda k: ("reduce_kernel" in k, counts[k]))
        ids = sorted(did for did, name in names.items() if name == reduce_name)
        want = sum(p["reduce_dispatches"] for p in meta["phases"])
        if len(ids) != want:
            raise SystemExit("%s: %d dispatches of %s, consumer.json lists %d"
                             % (d, len(ids), reduce_name[:60], want))
        pos = 0
        for p in meta["phases"]:
            chunk = ids[pos:pos + p["reduce_dispatches"]]
            pos += p["reduce_dispatches"]
            if p["phase"] not in order:
                order.append(p["phase"])
            row = table.setdefault(p["phase"], {})
            for did in chunk:
                vals = dict(per_dispatch[did])
                for ratio, (num, den) in INTERFERENCE_RATIOS.items():
                    if vals.get(den):
                        vals[ratio] = vals[num] / vals[den]
                for c, v in vals.items():
                    row.setdefault(c, []).append(v)
                if did in durations:
                    row.setdefault("duration_us", []).append(durations[did] / 1e3)
    med = {ph: {c: statistics.median(v) for c, v in row.items()} for ph, row in table.items()}
    cols = sorted({c for row in med.values() for c in row})
    cols.remove("duration_us") if "duration_us" in cols else None
    cols = ["duration_us"] + cols
    print("| phase | " + " | ".join(cols) + " |")
    print("|---|" + "---|" * len(cols))
    for ph in order:
        print("| %s | " % ph + " | ".join(
            ("%.6g" % med[ph][c]) if c in med[ph] else "" for c in cols) + " |")
    print()
    print("loader: " + json.dumps(loader))


def leg_ghost_list(kvt, workloads):
    """The write-through-selective filter (host only): page-boundary hashing of
    the mixed batch's token sequences (seeded random ids, page 64), inserting
    evicted page hashes into a Ghost List of 1,048,576 entries (64 per call, as
    a request's pages leave the GPU pool, and all in one call), and proven-reuse
    scans of 64-page prefixes (half of them with a hit). The oracle is timed
    beside it on a sample of the same operations."""
    from oracle import ghost
    rng = np.random.default_rng([4, 6])
    ps = 64
    lens, _, _ = workloads.mixed_requests(workloads.mixed(), 4)
    seqs = [rng.integers(0, 150000, size=int(n), dtype=np.int64).astype(np.int32) for n in lens]
    ntok = int(sum(x.size for x in seqs))
    t0 = time.perf_counter()
    hashes = [kvt.kv_page_hashes(x, ps) for x in seqs]
    t_hash = time.perf_counter() - t0
    cap = 1 << 20
    g = kvt.GhostList(cap)
    stream = rng.integers(0, 2**63, size=2 * cap, dtype=np.int64).astype(np.uint64)
    batches = np.array_split(stream, stream.size // 64)
    t0 = time.perf_counter()
    for b in batches:
        g.insert(b)
    t_ins = time.perf_counter() - t0
    g2 = kvt.GhostList(cap)                    # the same inserts in one call
    t0 = time.perf_counter()
    g2.insert(stream)
    t_ins1 = time.perf_counter() - t0
    g2.close()
    held = np.asarray(g.order()[-cap // 2:], dtype=np.uint64)
    queries = []
    for k in range(10000):
        q = rng.integers(0, 2**63, size=64, dtype=np.int64).astype(np.uint64)
        if k % 2 == 0:
            q[int(rng.integers(0, 64))] = held[int(rng.integers(0, held.size))]
        queries.append(q)
    t0 = time.perf_counter()
    hits = sum(1 for q in queries if g.reuse_prefix(q) > 0)
    t_scan = time.perf_counter() - t0
    g.close()
    # oracle on samples
    og = ghost.GhostList(cap)
    sample = stream[:200_000].tolist()
    t0 = time.perf_counter()
    for j in range(0, len(sample), 64):
        og.insert(sample[j:j + 64])
    t_oins = time.perf_counter() - t0
    oq = [q.tolist() for q in queries[:2000]]
    t0 = time.perf_counter()
    for q in oq:
        og.reuse_prefix(q)
    t_oscan = time.perf_counter() - t0
    tok_sample = seqs[0][:64 * ps].tolist()
    t0 = time.perf_counter()
    ghost.page_hashes(tok_sample, ps)
    t_ohash = time.perf_counter() - t0
    out = {"workload": "page 64; hashing: the mixed batch's %d tokens in %d requests; "
                       "Ghost List of %d entries: %d inserts in batches of 64, 10000 "
                       "proven-reuse scans of 64 pages (%d with a hit)"
                       % (ntok, len(seqs), cap, stream.size, hits),
           "hash_tokens_per_s": round(ntok / t_hash),
           "insert_per_s_one_call": round(stream.size / t_ins1),
           "insert_per_s": round(stream.size / t_ins),
           "scan_pages_per_s": round(10000 * 64 / t_scan),
           "oracle": {"hash_tokens_per_s": round(len(tok_sample) / t_ohash),
                      "insert_per_s": round(len(sample) / t_oins),
                      "scan_pages_per_s": round(len(oq) * 64 / t_oscan),
                      "sample": "hashing: one 4096-token sequence (every page hash recomputed "
                                "from the root, as the oracle defines it); 200,000 inserts; "
                                "2,000 scans"}}
    log("ghost list %s" % json.dumps(out)[:160])
    return out


def host_memory_study(torch, kvt, workloads, sizes_gb):
    """Pinned-size sweep: the headline request (32768 tokens x 78 layers x 1152 B,
    contiguous device pages) against layer_first host pools of the given sizes,
    each placed three ways: the default policy, bound to NUMA node 0, and
    interleaved over the online nodes (KV_F_HOST_INTERLEAVE).
    The request's host rows are 512 random pages of the whole pool, so that the
    pages it touches spread over all of it (a layer_first pool also puts each
    layer in its own region). Per size: pool creation time, and device-event
    GB/s of kernel and copy-engine backups and loads (median of 5)."""
    shape = workloads.mla32k()
    L, C, R, ps = shape.layers, shape.components, shape.row_bytes, shape.page_size
    S_dev, n = shape.device_slots, shape.extra["tokens"]
    bufs = []
    for l in range(L):
        b = torch.empty(S_dev * R, dtype=torch.uint8, device="cuda:0")
        workloads.fill_device_buffer(b, shape, 3, l, 0, torch)
        bufs.append(b)
    first = workloads.contiguous_pages_at_offset(3, S_dev // ps, n // ps)
    dev_idx = workloads.page_indices(first, ps)
    s = torch.cuda.Stream()
    nb = n * L * C * R
    out = []
    placements = (("default", -1, 0), ("bind_node0", 0, 0),
                  ("interleave", -1, kvt.F_HOST_INTERLEAVE))
    for gb, (pl_name, numa, pl_flag) in [(g, pl) for g in sizes_gb for pl in placements]:
        S_host = max(n, int(gb * 1e9 / (L * C * R)) // ps * ps)
        host_pages = workloads.fragmented_pages(3, S_host // ps, n // ps, workloads.P_HOST)
        host_idx = workloads.page_indices(host_pages, ps)
        t0 = time.perf_counter()
        try:
            pool = kvt.KvPool(kvt.geometry(L, C, R, S_dev, S_host, ps, 0), bufs, numa_node=numa,
                              flags=kvt.F_CHECK_UNIQUE | pl_flag)
        except kvt.KvError as e:        # the driver's pinned-memory limit
            log("host pool of %.1f GB (%s) refused: %s" % (gb, pl_name, e))
            out.append({"host_pool_gb": round(S_host * L * C * R / 1e9, 2),
                        "placement": pl_name, "refused": str(e)})
            continue
        t_create = time.perf_counter() - t0
        log("host pool %.1f GB (%s) created in %.1f s" %
            (pool.host_array().nbytes / 1e9, pl_name, t_create))
        cell = {"host_pool_gb": round(pool.host_array().nbytes / 1e9, 2), "placement": pl_name,
                "create_s": round(t_create, 2)}
        for pname, p in (("kernel", kvt.PATH_KERNEL), ("dma", kvt.PATH_DMA)):
            pool.set_path(p)
            for dname, fn in (("d2h", lambda: pool.backup(dev_idx, host_idx, 0, L, s)),
                              ("h2d", lambda: pool.load(dev_idx, host_idx, 0, L, s))):
                fn()
                s.synchronize()
                ts = []
                for _ in range(5):
                    e0, e1 = _ev(torch), _ev(torch)
                    e0.record(s)
                    fn()
                    e1.record(s)
                    e1.synchronize()
                    ts.append(e0.elapsed_time(e1) / 1e3)
                cell["%s_%s_gbps" % (pname, dname)] = round(nb / statistics.median(ts) / 1e9, 3)
        log("host memory %s" % json.dumps(cell))
        out.append(cell)
        t0 = time.perf_counter()
        pool.close()
        cell["destroy_s"] = round(time.perf_counter() - t0, 2)
    nodes = sorted(os.listdir("/sys/devices/system/node")) if os.path.isdir(
        "/sys/devices/system/node") else []
    return {"study": "pinned host pool size and placement",
            "request": "32768 tokens x 78 x 1152 B, 512 random host pages, layer_first",
            "numa_nodes": [d for d in nodes if d.startswith("node")], "rows": out}


def tp_shared_study(torch, kvt, workloads, tp, reps=5):
    """A tensor-parallel group of `tp` ranks holding the same MLA latent (78 x 1152 B
    rows, 32768-token prefix), each rank a pool over its own device buffers, all
    on this one GPU. Shared: one host pool (kv_pool_create_shared); the writer
    backs up, the other ranks' backups move nothing and wait for it. Private:
    every rank has its own host pool and backs up. Per mode: pinned host bytes,
    bytes written over the host link, the group write-back's time (all ranks'
    calls, device events; ranks share one link here, where a real group has
    one per GPU), the sharing ranks' submit time, and every rank's load rate.
    Before timing, each sharing rank's loaded rows are checked against the
    writer's source rows on the device."""
    shape = workloads.mla32k()
    L, C, R, ps = shape.layers, shape.components, shape.row_bytes, shape.page_size
    S_dev, S_host, n = shape.device_slots, shape.host_slots, shape.extra["tokens"]
    geom = kvt.geometry(L, C, R, S_dev, S_host, ps, kvt.LAYER_FIRST)
    ranks = []
    for r in range(tp):
        bufs = []
        for l in range(L):
            b = torch.empty(S_dev * R, dtype=torch.uint8, device="cuda:0")
            if r == 0:
                workloads.fill_device_buffer(b, shape, 3, l, 0, torch)
            bufs.append(b)
        ranks.append(bufs)
    first = workloads.contiguous_pages_at_offset(3, S_dev // ps, n // ps)
    dev_idx = workloads.page_indices(first, ps)
    host_idx = np.arange(n, dtype=np.int64)
    nbytes = n * L * C * R
    s = torch.cuda.Stream()
    out = {"tp": tp, "workload": "mla latent 78 x 1152 B, 32768-token prefix, layer_first",
           "bytes_per_rank": nbytes}
    for mode in ("shared", "private"):
        pools = []
        for r in range(tp):
            share = pools[0] if (mode == "shared" and r > 0) else None
            pools.append(kvt.KvPool(geom, ranks[r], share_with=share))
        pinned = sum(p.host_array().nbytes for p in pools[:1 if mode == "shared" else tp])
        if mode == "private":   # every rank's L1 holds the same latent
            for r in range(1, tp):
                for a, b in zip(ranks[r], ranks[0]):
                    a.copy_(b)
        torch.cuda.synchronize()

        def group_backup():
            for p in pools:
                p.backup(dev_idx, host_idx, 0, L, s)

        def group_load():
            for p in pools:
                p.load(dev_idx, host_idx, 0, L, s)

        group_backup()
        group_load()
        s.synchronize()
        if mode == "shared":   # the loaded rows (a contiguous run of slots) match the writer's
            lo, hi = int(dev_idx[0]), int(dev_idx[0]) + n
            assert np.array_equal(dev_idx, np.arange(lo, hi))
            for r in range(1, tp):
                for l in range(L):
                    assert torch.equal(ranks[r][l].view(S_dev, R)[lo:hi],
                                       ranks[0][l].view(S_dev, R)[lo:hi]), (r, l)
        t_b, t_l, sub = [], [], []
        for _ in range(reps):
            e0, e1, e2 = _ev(torch), _ev(torch), _ev(torch)
            e0.record(s)
            pools[0].backup(dev_idx, host_idx, 0, L, s)
            t0 = time.perf_counter()
            for p in pools[1:]:
                p.backup(dev_idx, host_idx, 0, L, s)
            sub.append((time.perf_counter() - t0) / max(1, tp - 1))
            e1.record(s)
            group_load()
            e2.record(s)
            e2.synchronize()
            t_b.append(e0.elapsed_time(e1) / 1e3)
            t_l.append(e1.elapsed_time(e2) / 1e3)
        tb, tl = statistics.median(t_b), statistics.median(t_l)
        link_d2h = nbytes * (1 if mode == "shared" else tp)
        cell = {"pinned_host_bytes": pinned, "d2h_link_bytes": link_d2h,
                "group_backup_ms": round(tb * 1e3, 3),
                "group_backup_link_gbps": round(link_d2h / tb / 1e9, 3),
                "other_ranks_backup_submit_us": round(statistics.median(sub) * 1e6, 1),
                "paths": {"writer": kvt.PATH_NAMES[pools[0].last_path(kvt.BACKUP)],
                          "others": kvt.PATH_NAMES[pools[-1].last_path(kvt.BACKUP)]},
                "load_per_rank_gbps": round(nbytes * tp / tl / 1e9, 3)}
        log("tp shared %s %s" % (mode, json.dumps(cell)))
        out[mode] = cell
        for p in pools:
            p.close()
    return out


def size_sweep(torch, kvt, workloads):
    """Request size against path: write-backs and loads of 64 to 32768 tokens of
    the 78 x 1152 B MLA latent (contiguous device and host slots), in each host
    layout, on the kernel path (write-backs on the default capped grid and on
    a full grid), the copy engines, the staged path and AUTO (with the path it
    chose). Per call: the median over 6-12 calls of HIP events around the call
    on its stream, in microseconds; one JSON line per layout and size on
    stderr, and the rows in the return value."""
    shape = workloads.mla32k()
    L, C, R, ps = shape.layers, shape.components, shape.row_bytes, shape.page_size
    S_dev, S_host = shape.device_slots, shape.host_slots
    bufs = []
    for l in range(L):
        for c in range(C):
            b = torch.empty(S_dev * R, dtype=torch.uint8, device="cuda:0")
            workloads.fill_device_buffer(b, shape, 3, l, c, torch)
            bufs.append(b)
    s = torch.cuda.Stream()

    def call_us(fn, reps):
        for _ in range(2):
            fn()
        s.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = _ev(torch), _ev(torch)
            e0.record(s)
            fn()
            e1.record(s)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        return statistics.median(ts)

    rows = []
    for lname, lay in LAYOUTS.items():
        with kvt.KvPool(kvt.geometry(L, C, R, S_dev, S_host, ps, lay), bufs) as pool:
            base = pool.calibration()
            full = pool.calibration()
            full.kernel_max_workgroups[:] = [0, 0]
            for n in (64, 128, 256, 512, 1024, 2048, 4096, 8192, 16384, 32768):
                d = np.arange(n, dtype=np.int64) + 128
                h = np.arange(n, dtype=np.int64)
                reps = 12 if n <= 4096 else 6
                row = {"layout": lname, "tokens": n, "bytes": n * L * C * R}
                for dname, dd in (("d2h", kvt.BACKUP), ("h2d", kvt.LOAD)):
                    fn = ((lambda: pool.backup(d, h, 0, L, s)) if dd == kvt.BACKUP
                          else (lambda: pool.load(d, h, 0, L, s)))
                    legs = [("kernel", kvt.PATH_KERNEL, base), ("dma", kvt.PATH_DMA, base),
                            ("staged", kvt.PATH_STAGED, base), ("auto", kvt.PATH_AUTO, base)]
                    if dd == kvt.BACKUP:
                        legs.insert(1, ("kernel_full_grid", kvt.PATH_KERNEL, full))
                    for pname, p, cal in legs:
                        pool.set_path(p)
                        pool.set_calibration(cal)
                        row["%s_%s_us" % (dname, pname)] = round(call_us(fn, reps), 1)
                        if p == kvt.PATH_AUTO:
                            row[dname + "_auto_chose"] = kvt.PATH_NAMES[pool.last_path(dd)]
                    pool.set_calibration(base)
                log("size sweep", json.dumps(row))
                rows.append(row)
        settle(torch, L * C * S_host * R)            # the pool's host memory was freed
    del bufs
    torch.cuda.synchronize()
    return {"size_sweep": rows}


def free_list_study(torch, kvt, workloads, count=160):
    """FIFO vs LIFO host free list under churn. A stream of write-back requests
    (lengths like the mixed batch's, at most 512 pages) goes into a host pool of
    2048 pages (131072 tokens of the 78 x 1152 B MLA latent, 11.8 GB) while at
    most 512 pages stay cached: before each request the oldest cached requests
    are evicted (their pages freed) until it fits, then its pages are allocated
    and its KV is backed up. The allocation sequence depends only on the policy,
    so it is planned once per policy and replayed on each path. Reported per
    layout and policy: distinct host pages written, runs of consecutive host
    pages per request, copy-engine copies per request, allocator time per
    request (median, binding included), and D2H GB/s (device events summed
    over the requests) on the
    kernel, copy-engine and AUTO paths."""
    import collections
    shape = workloads.mla32k()
    L, C, R, ps = shape.layers, shape.components, shape.row_bytes, shape.page_size
    S_dev = shape.device_slots
    pool_pages, cap_pages = 2048, 512
    S_host = pool_pages * ps
    reqs = workloads.churn_requests(shape, 6, count, S_dev // ps, cap_pages)
    bufs = []
    for l in range(L):
        b = torch.empty(S_dev * R, dtype=torch.uint8, device="cuda:0")
        workloads.fill_device_buffer(b, shape, 6, l, 0, torch)
        bufs.append(b)
    s = torch.cuda.Stream()
    rows = []
    for layout in (kvt.LAYER_FIRST, kvt.PAGE_FIRST_DIRECT):
        geom = kvt.geometry(L, C, R, S_dev, S_host, ps, layout)
        pool = kvt.KvPool(geom, bufs)
        for pname, policy in (("fifo", kvt.FREE_FIFO), ("lifo", kvt.FREE_LIFO)):
            alloc = kvt.HostPages(pool_pages, policy)
            live, live_pages, plan = collections.deque(), 0, []
            t_alloc = []
            for npg, first in reqs:
                t0 = time.perf_counter()
                while live_pages + npg > cap_pages:
                    old = live.popleft()
                    alloc.free(old)
                    live_pages -= len(old)
                pages = alloc.alloc(npg)
                t_alloc.append(time.perf_counter() - t0)
                live.append(pages)
                live_pages += npg
                plan.append((workloads.page_indices(np.arange(first, first + npg), ps),
                             workloads.page_indices(pages, ps), pages))
            alloc.close()
            touched = len(set(int(p) for _, _, pg in plan for p in pg))
            runs = [1 + int(np.count_nonzero(np.diff(pg) != 1)) for _, _, pg in plan]
            copies = [kvt.kv_count_dma_copies(geom, d, h, 0, L)[1] for d, h, _ in plan]
            total = sum(len(d) for d, _, _ in plan) * L * C * R
            cell = {"layout": workloads.LAYOUT_NAMES[layout], "policy": pname,
                    "requests": len(plan), "pool_pages": pool_pages, "cached_pages_max": cap_pages,
                    "distinct_host_pages_written": touched,
                    "host_page_runs_per_request": round(statistics.mean(runs), 2),
                    "dma_copies_per_request": round(statistics.mean(copies), 1),
                    "alloc_free_us_per_request_median": round(statistics.median(t_alloc) * 1e6, 2),
                    "bytes": total}
            for path_name, path in (("kernel", kvt.PATH_KERNEL), ("dma", kvt.PATH_DMA),
                                    ("auto", kvt.PATH_AUTO)):
                pool.set_path(path)
                d0, h0, _ = plan[0]
                pool.backup(d0, h0, 0, L, s)
                s.synchronize()
                evs = []
                for d, h, _ in plan:
                    e0, e1 = _ev(torch), _ev(torch)
                    e0.record(s)
                    pool.backup(d, h, 0, L, s)
                    e1.record(s)
                    evs.append((e0, e1))
                s.synchronize()
                t = sum(a.elapsed_time(b) for a, b in evs) / 1e3
                cell["%s_gbps" % path_name] = round(total / t / 1e9, 3)
            log("free list %s" % json.dumps(cell))
            rows.append(cell)
        pool.close()
    # the oracle's free list on the same churn (CPU baseline of the allocator)
    from oracle import slots as oracle_slots
    base = {}
    for pname, policy in (("fifo", oracle_slots.FIFO), ("lifo", oracle_slots.LIFO)):
        fl = oracle_slots.FreeList(pool_pages, policy)
        live, live_pages, ts = collections.deque(), 0, []
        for npg, _ in reqs:
            t0 = time.perf_counter()
            while live_pages + npg > cap_pages:
                old = live.popleft()
                fl.release(old)
                live_pages -= len(old)
            live.append(fl.alloc(npg)[1])
            live_pages += npg
            ts.append(time.perf_counter() - t0)
        base[pname + "_alloc_free_us_per_request_median"] = round(statistics.median(ts) * 1e6, 2)
    return {"study": "FIFO vs LIFO host free list under churn",
            "request": "%d write-backs, 78 x 1152 B rows, page 64, lengths lognormal(median 4096 "
                       "tokens, sigma 1) capped at 512 pages" % len(reqs),
            "rows": rows, "cpu_baseline": dict(base, kind="oracle", cores=1)}


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(shape, dev_b, dev_l, host_idx):
    """The oracle as it stands, on this host, on the timed steps' index set: a
    write-back of the 32768-token prefix from device slots dev_b, then a load of
    it into slots dev_l, all 78 layers, on layer_first host mirrors of the same
    geometry (65536 device slots, 32768 host slots). T threads (the cores this
    process may run on, at most 16) each run the oracle on their own slice of
    the layers (its C calls release the GIL); one pass is the T slices of one
    write-back + load. 3 untimed passes (the first also touches the mirrors),
    then the median of 20 timed passes gives `value`; one thread's median of 3
    passes is reported beside it."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    L, C, R, ps = shape.layers, shape.components, shape.row_bytes, shape.page_size
    n = host_idx.size
    g = oracle.Geometry(L, C, R, shape.device_slots, shape.host_slots, ps, 0)
    # written through once, so no read lands on never-written (shared zero) pages
    dev = [np.full(g.S_dev * R, 0x5A, np.uint8) for _ in range(L * C)]
    host = np.full(g.host_bytes(), 0xA5, np.uint8)
    T = max(1, min(16, len(os.sched_getaffinity(0)), L))
    cuts = np.linspace(0, L, T + 1).astype(int)

    def piece(l0, l1):
        assert oracle.backup(g, dev, host, dev_b, host_idx, l0, l1) == 0
        assert oracle.load(g, dev, host, dev_l, host_idx, l0, l1) == 0

    def passes(pool, k, count):
        ts = []
        for _ in range(count):
            t0 = time.perf_counter()
            list(pool.map(lambda j: piece(int(cuts[j]), int(cuts[j + 1])), range(k)))
            ts.append(time.perf_counter() - t0)
        return ts

    bytes_pass = 2 * n * L * C * R
    with ThreadPoolExecutor(T) as pool:
        passes(pool, T, 3)
        tT = statistics.median(passes(pool, T, 20))
    t1 = statistics.median([passes_one(piece, L) for _ in range(3)])
    return {"value": round(bytes_pass / tT / 1e9, 3), "unit": "GB/s", "cores": T,
            "kind": "oracle",
            "single_thread_gbps": round(bytes_pass / t1 / 1e9, 3),
            "nproc": os.cpu_count(), "cpu_model": cpu_model(),
            "sample": "the timed steps' index set: write-back then load of the 32768-token "
                      "prefix, 78 layers x 1152 B, layer_first host mirrors; %d threads over "
                      "layer slices, median of 20 passes after 3 (%.2f s per pass)"
                      % (T, tT)}


def passes_one(piece, L):
    t0 = time.perf_counter()
    piece(0, L)
    return time.perf_counter() - t0


if __name__ == "__main__":
    main()
