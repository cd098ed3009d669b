#!/usr/bin/env python3
"""Throughput of the paged Q4 KV-cache quantize + dequantize path on one GPU.

Step = one pass of the hot path over one batch: fp16 K and V rows of 32
sequences x 256 new tokens, resolved through block_table / cache_seqlens
(4096 physical pages x 256 tokens, 8 heads x 128), quantized to 4-bit codes
+ fp16 scales (one launch for K and V), then dequantized back to fp16 (one
launch).  The ExLlamaV2 cache page describes these operations
(fp16_to_q_kv / q_to_fp16_kv, paged mode with page_size 256 in its usage
example).

Cold data: 32 seeded (cache_seqlens, block_table) draws are rotated, so each
launch touches rows the previous 31 did not (about 1.4 GB between reuses,
beyond the 256 MB last-level cache).  The timed job is K quantize launches
over the rotated draws, then K dequantize launches (quantized data is not
cache-resident when it is read back), each replayed as HIP graphs between
device synchronisations and timed with HIP events.

Output: one JSON line: value = algorithmic bytes of the K steps / (quantize
+ dequantize kernel time), the roofline of the slower kernel, cpu_baseline
= the CPU oracle on a bounded sample timed on the host cores, and secondary
figures (the whole job on concurrent step chains, a plain-copy floor at the
same launch size, the other formats and layouts).

(The "ExLlamaV2 cache page" in this file is the page "Implementation: Turboderp org
Exllamav2 Ext Cache".)
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KV quant+dequant GB/s (read+write) and % of HBM peak, paged Q4, 1 MI355X"
HBM_PEAK_GBS = 8000.0
DRAWS = 32
HEADS, HEAD_DIM, PAGE = 8, 128, 256
ROW = HEADS * HEAD_DIM


def q_row_bytes(wbits):
    """Algorithmic bytes per token row, either direction: fp16 row + codes + scales."""
    return ROW * 2 + ROW * wbits // 8 + (ROW // 32) * 2


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=6400)
    p.add_argument("--warmup", type=int, default=64)
    p.add_argument("--graph-steps", type=int, default=4 * DRAWS,
                   help="launches per captured graph of the timed regions")
    p.add_argument("--chain-graph-steps", type=int, default=20 * DRAWS,
                   help="steps per captured graph of the whole-job figure")
    p.add_argument("--streams", type=int, default=3,
                   help="concurrent step chains of the whole-job figure (secondary.whole_job)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-secondary", action="store_true", help="skip the other workloads' kernel timings")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run a plain device copy of known size (counter calibration)")
    p.add_argument("--cpu-draws", type=int, default=16, help="draws in the CPU-oracle sample")
    return p.parse_args()


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


class PagedKV:
    """Device state of the paged workload (4096 pages x 256 tokens, 8 heads x
    128, 32 sequences x 256 new tokens, 32 rotated paging draws) at one code
    width, and its two launches.  `share` reuses another instance's fp16
    caches and paging tables."""

    def __init__(self, torch, kvq, synth, wbits=4, share=None):
        self.torch, self.kvq, self.wbits = torch, kvq, wbits
        w = synth.q4_paged(draws=DRAWS)
        self.w = w
        shape = w.shape
        t = torch
        if share is None:
            log("allocating paged caches %s x 2 (fp16) + codes/scales/outputs" % (shape,))
            self.k = synth.device_normal_f16(t, shape, w.extra["device_seed"])
            self.v = synth.device_normal_f16(t, shape, w.extra["device_seed"] + 1)
            self.ko = t.zeros(shape, dtype=t.float16, device="cuda")
            self.vo = t.zeros(shape, dtype=t.float16, device="cuda")
            self.tables = [(t.from_numpy(sl).cuda(), t.from_numpy(bt).cuda()) for sl, bt in w.extra["tables"]]
        else:
            self.k, self.v, self.ko, self.vo, self.tables = share.k, share.v, share.ko, share.vo, share.tables
        cs, ss = kvq.code_shape(shape, wbits), kvq.scale_shape(shape)
        self.kq = t.zeros(cs, dtype=t.uint8, device="cuda")
        self.vq = t.zeros(cs, dtype=t.uint8, device="cuda")
        self.ks = t.zeros(ss, dtype=t.float16, device="cuda")
        self.vs = t.zeros(ss, dtype=t.float16, device="cuda")
        self.rows_per_launch = 2 * w.batch_size * w.width            # K and V rows
        self.bytes_per_launch = self.rows_per_launch * q_row_bytes(wbits)
        self.bytes_per_step = 2 * self.bytes_per_launch
        self.elems_per_launch = self.rows_per_launch * ROW
        self.elems_per_step = 2 * self.elems_per_launch

    def quant(self, d):
        sl, bt = self.tables[d]
        w = self.w
        self.kvq.kvq_fp16_to_q_kv(self.k, self.kq, self.ks, self.v, self.vq, self.vs, w.batch_size,
                                  w.offset, w.width, w.page_size, sl, bt, self.wbits)

    def dequant(self, d):
        sl, bt = self.tables[d]
        w = self.w
        self.kvq.kvq_q_to_fp16_kv(self.kq, self.ko, self.ks, self.vq, self.vo, self.vs, w.batch_size,
                                  w.offset, w.width, w.page_size, sl, bt, self.wbits)

    def step(self, d):
        self.quant(d)
        self.dequant(d)


def time_kernels(torch, launches, reps, replays=9):
    """Device duration per launch of each named launch: `reps` launches of
    that kernel alone (rotating over its argument list) are captured in one
    HIP graph; after two untimed replays (the first inputs touched, clocks
    up after any host-side setup) the graph is replayed `replays` times,
    each between two events on the current stream, and the median replay
    time over `reps` is taken.  Consecutive launches in a graph run back to
    back, so this is the kernel's own duration plus the (near-zero)
    dispatch gap; returns {name: seconds}."""
    out = {}
    for name, fn, args in launches:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(len(args)):
                fn(args[i])
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(reps):
                fn(args[i % len(args)])
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        times = []
        for _ in range(replays):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) * 1e-3 / reps)
        out[name] = float(np.median(times))
        del g
    return out


def cpu_baseline(wl, oracle, rows_fn, draws):
    """The CPU oracle (plain scalar C) quantizing then dequantizing the same
    rows as `draws` GPU steps, rows split over host threads.  Returns the
    timing and, per (draw, tensor), the oracle's codes / scales / fp16 rows."""
    from concurrent.futures import ThreadPoolExecutor
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    groups = []                                  # (draw, name, rows, host fp16 rows)
    for d in range(draws):
        sl, bt = wl.w.extra["tables"][d]
        rows = oracle.call_rows(wl.w.shape[0], wl.w.shape[1], wl.w.batch_size, wl.w.offset,
                                wl.w.width, wl.w.page_size, sl, bt)
        rows = rows[rows >= 0]
        groups.append((d, "K", rows, rows_fn(wl.k, rows)))
        groups.append((d, "V", rows, rows_fn(wl.v, rows)))
    jobs = [(g, chunk) for g in range(len(groups))
            for chunk in np.array_split(np.arange(groups[g][3].shape[0]), threads)]

    def work(job):
        g, chunk = job
        c, s = oracle.quant_rows(groups[g][3][chunk], 4)
        return c, s, oracle.dequant_rows(c, s, 4)

    with ThreadPoolExecutor(max_workers=threads) as pool:
        t0 = time.perf_counter()
        results = list(pool.map(work, jobs))
        dt = time.perf_counter() - t0
    per_group = []
    for g, (d, name, rows, _) in enumerate(groups):
        mine = [r for (gg, _), r in zip(jobs, results) if gg == g]
        per_group.append((d, name, rows, *(np.concatenate([m[k] for m in mine]) for k in range(3))))
    n_rows = sum(g[2].size for g in groups)
    return {"seconds": dt, "threads": threads, "rows": n_rows,
            "bytes": n_rows * q_row_bytes(4) * 2, "groups": per_group}


def oracle_detail(wl, oracle, rows_fn, kvq):
    """Single-thread oracle rate on one draw's rows, and the naive oracle
    count_match beside the library's 64-bit-chunk scan (same ids)."""
    sl, bt = wl.w.extra["tables"][0]
    rows = oracle.call_rows(wl.w.shape[0], wl.w.shape[1], wl.w.batch_size, wl.w.offset,
                            wl.w.width, wl.w.page_size, sl, bt)
    rows = rows[rows >= 0]
    x = rows_fn(wl.k, rows)
    t0 = time.perf_counter()
    c, s = oracle.quant_rows(x, 4)
    oracle.dequant_rows(c, s, 4)
    dt = time.perf_counter() - t0
    # the other formats on the same rows, one thread
    per_format = {}
    for wb in (6, 8):
        t1 = time.perf_counter()
        c6, s6 = oracle.quant_rows(x, wb)
        oracle.dequant_rows(c6, s6, wb)
        d6 = time.perf_counter() - t1
        per_format["Q%d" % wb] = round(rows.size * q_row_bytes(wb) * 2 / d6 / 1e9, 4)
    x4 = x.reshape(1, rows.size, HEADS, HEAD_DIM)
    b8 = np.empty(x4.shape, np.uint8)
    back = np.empty(x4.shape, np.float16)
    t1 = time.perf_counter()
    oracle.fp16_to_fp8(x4, b8, 1, 0, rows.size)
    oracle.fp8_to_fp16(b8, back, 1, 0, rows.size)
    d8 = time.perf_counter() - t1
    per_format["8-bit"] = round(rows.size * ROW * 3 * 2 / d8 / 1e9, 4)
    from kv_cache_quantization_kvq_amd import synth
    mw = synth.mix_paged()
    a, b = mw.extra["ids_a"], mw.extra["ids_b"]
    reps = 20
    t1 = time.perf_counter()
    for _ in range(reps):
        m_oracle = oracle.count_match(a, b, a.size)
    t_or = (time.perf_counter() - t1) / reps
    t1 = time.perf_counter()
    for _ in range(reps):
        m_lib = kvq.kvq_count_match(a, b, a.size)
    t_lib = (time.perf_counter() - t1) / reps
    if m_oracle != m_lib:
        log("count_match mismatch: oracle %d, library %d" % (m_oracle, m_lib))
        sys.exit(4)
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": cpu_model, "host_threads_available": len(os.sched_getaffinity(0)),
            "single_thread_other_formats_GBps": per_format,
            "single_thread": {"GB/s": round(rows.size * q_row_bytes(4) * 2 / dt / 1e9, 4),
                              "elements_per_s": round(rows.size * ROW * 2 / dt, 1),
                              "sample": "%d K rows of one paged-Q4 step quantized then dequantized, 1 thread"
                                        % rows.size},
            "count_match": {"n": int(a.size), "match": m_lib, "oracle_us": round(t_or * 1e6, 2),
                            "library_us": round(t_lib * 1e6, 2)}}


def capture_graph(torch, fn, n):
    """A HIP graph of fn(0) .. fn(n - 1) launched back to back on one stream."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    return g


def time_region(torch, fn, steps, per):
    """`steps` launches fn(i % DRAWS), i < steps, replayed as graphs of `per`
    back-to-back launches on the current stream, each replay between two
    events; the region is bracketed by device synchronisation.  Returns
    (median per-launch seconds over the replays, total seconds of the
    region).  Inside a replay consecutive dispatches follow each other with
    no measurable gap, so the per-launch time of a replay is the kernel's
    own duration; the median discards the occasional replay that waits on
    host-side submission."""
    full, rem = steps // per, steps % per
    distinct = DRAWS // math.gcd(per, DRAWS)              # replays r and r + distinct launch the same draws
    graphs = [(capture_graph(torch, lambda i, r=r: fn((r * per + i) % DRAWS), per), per)
              for r in range(min(full, distinct))]
    g_rem = capture_graph(torch, lambda i: fn((full * per + i) % DRAWS), rem) if rem else None
    for g, _ in graphs:
        g.replay()                                        # untimed: graph upload
    if g_rem is not None:
        g_rem.replay()
    torch.cuda.synchronize()
    order = [graphs[r % len(graphs)] for r in range(full)] + ([(g_rem, rem)] if g_rem is not None else [])
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(order) + 1)]
    t0 = time.perf_counter()
    ev[0].record()
    for i, (g, _) in enumerate(order):
        g.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_launch = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e-3 / n for i, (_, n) in enumerate(order))
    total = ev[0].elapsed_time(ev[-1]) * 1e-3
    return per_launch[len(per_launch) // 2], total, wall


def whole_job(torch, wl, steps, per, streams):
    """Independent steps (quantize then dequantize of one draw) spread
    round-robin over `streams` concurrent chains, graphs of `per` steps.
    Steps of different draws touch different rows; two steps of one draw
    write identical bytes to the same rows, so no result depends on how the
    chains interleave.  Returns seconds for `steps` steps."""
    chains = [torch.cuda.Stream() for _ in range(streams)]
    for c in chains:
        c.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()

    def capture(n, first):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cap = torch.cuda.current_stream()
            for c in chains:
                c.wait_stream(cap)                        # fork
            for d in range(n):
                with torch.cuda.stream(chains[d % streams]):
                    wl.step((first + d) % DRAWS)
            for c in chains:
                cap.wait_stream(c)                        # join
        return g

    per = max(1, min(per, steps))
    full, rem = steps // per, steps % per
    graphs = [capture(per, 0)] if full else []
    g_rem = capture(rem, full * per) if rem else None
    for g in graphs + ([g_rem] if g_rem else []):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(full):
        graphs[0].replay()
    if g_rem is not None:
        g_rem.replay()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (each token row "
              "converts independently; sharding by heads or sequences needs no exchange). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0 or args.streams < 1 or args.graph_steps < 1 or args.chain_graph_steps < 1:
        print("bench.py: --steps, --streams and the graph sizes must be at least 1, --warmup at least 0",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import kv_cache_quantization_kvq_amd as kvq
    from kv_cache_quantization_kvq_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(3)
    kvq.load_library()                                   # fail loudly without the HIP library
    dev_name = torch.cuda.get_device_name(0)
    wl = PagedKV(torch, kvq, synth, wbits=4)

    # warmup: eager steps over the draws (every draw's codes exist before the
    # dequantize region)
    for i in range(max(args.warmup, DRAWS)):
        wl.step(i % DRAWS)
    torch.cuda.synchronize()

    # the timed job: K quantize launches over the rotated draws, then K
    # dequantize launches (the cold-data protocol: quantized data is not
    # cache-resident when it is read back)
    per = max(1, min(args.graph_steps, args.steps))
    log("timing %d quantize then %d dequantize launches (graphs of %d) on %s"
        % (args.steps, args.steps, per, dev_name))
    tq, tq_total, wq = time_region(torch, wl.quant, args.steps, per)
    td, td_total, wd = time_region(torch, wl.dequant, args.steps, per)
    # value: the algorithmic bytes of a step over the sum of the two kernels'
    # per-launch times (the kernel-time definition of the metric)
    value = wl.bytes_per_step / (tq + td) / 1e9
    ms_per_step = (tq + td) * 1e3

    kt = {"quant": tq, "dequant": td}
    dom = max(kt, key=kt.get)                             # the slower kernel
    achieved = wl.bytes_per_launch / kt[dom] / 1e9
    traffic, traffic_src = traffic_for(dom, wl.bytes_per_launch)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "traffic_source": traffic_src,
                "kernel": KERNEL_NAMES[dom], "bytes_per_launch": wl.bytes_per_launch,
                "avg_us": {k: round(v * 1e6, 3) for k, v in kt.items()},
                "timing": "median over %d graph replays of %d back-to-back launches (rotated draws) "
                          "of event time / launches" % (-(-args.steps // per), per),
                "region_us_per_launch": {"quant": round(tq_total / args.steps * 1e6, 3),
                                         "dequant": round(td_total / args.steps * 1e6, 3)}}
    # counter cross-check: HBM bytes the counters saw per launch over the same duration
    roofline["counter_GBps"] = round(traffic / kt[dom] / 1e9, 1) if traffic is not None else None
    roofline["rocprof"] = rocprof_check(roofline["avg_us"])

    def rows_fn(t, rows):
        idx = torch.from_numpy(np.asarray(rows, np.int64)).cuda()
        x = t.view(t.shape[0] * t.shape[1], -1).index_select(0, idx)
        a = x.cpu().numpy()
        return a.view(np.uint16) if a.dtype == np.float16 else a

    # the CPU-baseline leg: the oracle timed on the host, and its outputs
    # checked against the device outputs of the timed draws
    cpu = cpu_detail = None
    if not args.no_cpu_baseline:
        import oracle
        log("timing the CPU oracle on %d draws" % args.cpu_draws)
        cb = cpu_baseline(wl, oracle, rows_fn, args.cpu_draws)
        for d, name, rows, c, sc, y in cb["groups"]:
            q, s_, o = (wl.kq, wl.ks, wl.ko) if name == "K" else (wl.vq, wl.vs, wl.vo)
            if not (np.array_equal(rows_fn(q, rows), c) and np.array_equal(rows_fn(s_, rows), sc)
                    and np.array_equal(rows_fn(o, rows), y)):
                log("PARITY FAILURE on the timed data (draw %d, %s)" % (d, name))
                sys.exit(4)
        log("timed data matches the oracle on %d rows" % cb["rows"])
        cpu_detail = oracle_detail(wl, oracle, rows_fn, kvq)
        cpu = {"value": round(cb["bytes"] / cb["seconds"] / 1e9, 4), "unit": "GB/s", "cores": cb["threads"],
               "kind": "oracle",
               "sample": "%d rows (K and V of %d paged-Q4 steps) quantized then dequantized by the "
                         "scalar C oracle, rows split over %d threads, %.2f s wall"
                         % (cb["rows"], args.cpu_draws, cb["threads"], cb["seconds"])}

    secondary = {}
    t_wj = whole_job(torch, wl, args.steps, args.chain_graph_steps, args.streams)
    secondary["whole_job"] = {"GB/s": round(wl.bytes_per_step * args.steps / t_wj / 1e9, 1),
                              "us_per_step": round(t_wj / args.steps * 1e6, 3),
                              "what": "%d steps (quantize then dequantize of one draw) on %d concurrent "
                                      "chains, graphs of %d steps, host wall clock"
                                      % (args.steps, args.streams, min(args.chain_graph_steps, args.steps))}
    secondary["copy_floor"] = copy_floor(torch, kvq, wl.bytes_per_launch)
    if not args.no_secondary:
        secondary.update(secondary_workloads(torch, kvq, synth, wl))

    def add_frac(d):
        if isinstance(d, dict):
            if "GB/s" in d:
                d["frac"] = round(d["GB/s"] / HBM_PEAK_GBS, 4)
            for v in d.values():
                add_frac(v)
    add_frac(secondary)
    if args.calibrate_copy:
        calibrate_copy(torch)

    kernel_pair = {"us": round((tq + td) * 1e6, 3), "GB/s": round(value, 1), "frac": round(value / HBM_PEAK_GBS, 4),
                   "elements_per_s": round(wl.elems_per_step / (tq + td), 1)}
    rec = {"metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
           "arith": "fp16 data; fp32 quotients and scales (quantize), fp16 products (dequantize); "
                    "4-bit codes",
           "data": "synthetic", "hbm_frac": round(value / HBM_PEAK_GBS, 4),
           "elements_per_s": round(wl.elems_per_step / (tq + td), 1),
           "config": {"workload": "paged_q4", "pages": wl.w.shape[0], "page_size": PAGE,
                      "heads": HEADS, "head_dim": HEAD_DIM, "batch": wl.w.batch_size,
                      "width": wl.w.width, "wbits": 4, "draws_rotated": DRAWS,
                      "bytes_per_step": wl.bytes_per_step,
                      "timed": "%d quantize launches then %d dequantize launches, graphs of %d launches, "
                               "HIP events per replay; value = bytes per step / (quantize + dequantize "
                               "per-launch kernel time)" % (args.steps, args.steps, per),
                      "region_wall_s": round(wq + wd, 4),
                      "device": dev_name},
           "roofline": roofline, "kernel_pair": kernel_pair, "cpu_baseline": cpu}
    if cpu_detail is not None:
        rec["cpu_detail"] = cpu_detail
    rec["secondary"] = secondary
    print(json.dumps(rec), flush=True)


# kernel names of the paged-Q4 launches (rocprofv3 spelling)
KERNEL_NAMES = {"quant": "kvq::narrow_run_kernel<4, 1, 2>",
                "dequant": "kvq::widen_run_kernel<4, 1, 2, false, 4, 2>"}


def copy_floor(torch, kvq, launch_bytes):
    """A plain non-temporal copy moving the bytes of one paged-Q4 launch
    (half read, half written), 32 rotated buffer pairs (cold), over bytes per
    lane, waves per workgroup and one tile per wave against waves striding
    inside one resident generation: the bandwidth one launch of this size
    reaches without any conversion work."""
    nbytes = launch_bytes // 2 // 16 * 16
    src = torch.empty((DRAWS, nbytes), dtype=torch.uint8, device="cuda")
    dst = torch.empty((DRAWS, nbytes), dtype=torch.uint8, device="cuda")
    src.fill_(1)
    out = {"bytes_moved": 2 * nbytes, "configs": []}
    best = None
    for lane_bytes in (16, 32, 64, 128):
        for group_waves in (1, 2, 4):
            for max_waves in (0, 4096):
                fn = (lambda d, lb=lane_bytes, gw=group_waves, mw=max_waves:
                      kvq.kvq_selftest_copy(src[d], dst[d], lb, gw, mw))
                t = time_kernels(torch, [("copy", fn, list(range(DRAWS)))], 4 * DRAWS)["copy"]
                tiles = -(-nbytes // (lane_bytes * 64))
                row = {"lane_bytes": lane_bytes, "group_waves": group_waves,
                       "waves": tiles if max_waves == 0 else min(tiles, max_waves),
                       "us": round(t * 1e6, 3), "GB/s": round(2 * nbytes / t / 1e9, 1)}
                out["configs"].append(row)
                if best is None or t < best[0]:
                    best = (t, row)
    out["best"] = dict(best[1])
    assert torch.equal(dst[DRAWS - 1], src[DRAWS - 1]), "copy floor: copy mismatch"
    del src, dst
    # the same bytes per launch in the conversions' uneven shapes: each lane
    # reads lane_elems 16-byte elements per element it writes (gather, like
    # quantize: 3.6 bytes read per byte written) or the reverse (scatter,
    # like dequantize)
    out["uneven"] = []
    for gather in (True, False):
        for lane_elems in (2, 4, 8):
            light = 2 * nbytes // (lane_elems + 1) // 1024 * 1024
            heavy = light * lane_elems
            src = torch.empty((DRAWS, heavy if gather else light), dtype=torch.uint8, device="cuda")
            dst = torch.empty((DRAWS, light if gather else heavy), dtype=torch.uint8, device="cuda")
            src.fill_(1)
            for group_waves in (1, 4):
                fn = (lambda d, le=lane_elems, gw=group_waves: kvq.kvq_selftest_stream(src[d], dst[d], le, gw))
                t = time_kernels(torch, [("stream", fn, list(range(DRAWS)))], 4 * DRAWS)["stream"]
                out["uneven"].append({"shape": "%s %d:1" % ("read:write" if gather else "write:read", lane_elems),
                                      "lane_elems": lane_elems, "group_waves": group_waves,
                                      "bytes_moved": heavy + light, "us": round(t * 1e6, 3),
                                      "GB/s": round((heavy + light) / t / 1e9, 1)})
            del src, dst
    return out


def read_profile_keys(name):
    """key = value lines of a committed profile summary, or None if absent."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    return kv


def rocprof_check(avg_us):
    """This run's per-launch event times against the per-dispatch means of
    the committed rocprofv3 trace of the same command, when that trace was
    taken on the same kernel sources."""
    name = "paged_q4_kernel_trace.txt"
    kv = read_profile_keys(name)
    if kv is None:
        return {"source": None, "reason": "no trace summary"}
    if kv.get("sources_sha256") != sources_digest():
        return {"source": "profiles/" + name, "reason": "taken on other kernel sources"}
    out = {"source": "profiles/" + name, "trace_mean_us": {}, "event_vs_trace": {}}
    for k in ("quant", "dequant"):
        tr = float(kv["%s_trace_mean_ns" % k]) / 1000.0
        out["trace_mean_us"][k] = round(tr, 3)
        out["event_vs_trace"][k] = "%+.1f%%" % ((avg_us[k] / tr - 1.0) * 100.0)
    return out


def traffic_for(kernel, algo_bytes):
    """HBM bytes per launch from the committed counter summary and a label of
    where they come from, or (None, reason) when the summary was taken on
    other kernel sources."""
    kv = read_profile_keys("traffic_paged_q4.txt")
    if kv is None:
        return None, "no counter summary"
    if kv.get("sources_sha256") != sources_digest():
        return None, "profiles/traffic_paged_q4.txt was taken on other kernel sources"
    key = "%s_traffic_bytes_per_launch" % kernel
    if key not in kv:
        return None, "no figure for this kernel"
    return float(kv[key]), ("profiles/traffic_paged_q4.txt: rocprofv3 FETCH_SIZE + WRITE_SIZE per dispatch, "
                            "each scaled by its reading for the library's plain copy kernel (committed, taken on "
                            "the same kernel sources)")


def sources_digest():
    """sha256 of the kernel sources with comments and whitespace removed, so
    that the recorded counters stay attached to the code they measured."""
    import re
    h = hashlib.sha256()
    for f in ("kvq_kernels.hip", "kvq_device.h", "kvq_internal.h"):
        with open(os.path.join(ROOT, "kv_cache_quantization_kvq_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def fmt_row_bytes(fmt):
    """Algorithmic bytes per token row, either direction, for a per-tensor
    format (0 = 8-bit high byte)."""
    return ROW * 2 + ROW if fmt == 0 else q_row_bytes(fmt)


def secondary_workloads(torch, kvq, synth, wl):
    """Kernel-time GB/s of the other paths, each with cold inputs (rotated
    paging draws) unless labelled hot (inputs repeated, partly
    cache-resident: context only)."""
    t = torch
    out = {}
    w = wl.w
    rows = w.batch_size * w.width
    # the same paged-Q4 launches with one draw repeated (rows and tables
    # cache-resident): context only
    kt = time_kernels(t, [("quant", wl.quant, [0]), ("dequant", wl.dequant, [0])], 4 * DRAWS)
    out["paged_q4_hot"] = {k: {"us": round(v * 1e6, 2), "GB/s": round(wl.bytes_per_launch / v / 1e9, 1)}
                           for k, v in kt.items()}
    # the paged-Q4 step called eagerly from Python (no graph), one stream:
    # host submission time per step beside the wall time per step
    n_eager = 640
    for i in range(64):
        wl.step(i % DRAWS)
    t.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n_eager):
        wl.step(i % DRAWS)
    t1 = time.perf_counter()
    t.cuda.synchronize()
    t2 = time.perf_counter()
    out["paged_q4_eager"] = {"steps": n_eager, "host_us_per_step": round((t1 - t0) / n_eager * 1e6, 2),
                             "us_per_step": round((t2 - t0) / n_eager * 1e6, 2),
                             "GB/s": round(wl.bytes_per_step * n_eager / (t2 - t0) / 1e9, 1)}
    # per-layer use: 8 layers' caches (1024 pages each) converted with one
    # shared paging draw, as a decode step does layer after layer -- the
    # tables stay hot, each layer's rows are cold (344 MB between reuses)
    lsh = (1024, w.shape[1], w.shape[2], w.shape[3])
    lrng = np.random.default_rng(9009)
    lsl = t.from_numpy(lrng.integers(0, 7937, size=w.batch_size).astype(np.int32)).cuda()
    lbt = t.from_numpy(lrng.permutation(1024).astype(np.int32).reshape(w.batch_size, -1)).cuda()
    layers = []
    for i in range(8):
        layers.append((synth.device_normal_f16(t, lsh, 9100 + 2 * i), synth.device_normal_f16(t, lsh, 9101 + 2 * i),
                       t.empty(kvq.code_shape(lsh, 4), dtype=t.uint8, device="cuda"),
                       t.empty(kvq.code_shape(lsh, 4), dtype=t.uint8, device="cuda"),
                       t.empty(kvq.scale_shape(lsh), dtype=t.float16, device="cuda"),
                       t.empty(kvq.scale_shape(lsh), dtype=t.float16, device="cuda"),
                       t.empty(lsh, dtype=t.float16, device="cuda"), t.empty(lsh, dtype=t.float16, device="cuda")))
    la = (w.batch_size, 0, w.width, w.shape[1], lsl, lbt)
    kt = time_kernels(t, [
        ("quant", lambda i: kvq.kvq_fp16_to_q_kv(layers[i][0], layers[i][2], layers[i][4], layers[i][1],
                                                 layers[i][3], layers[i][5], *la, 4), list(range(8))),
        ("dequant", lambda i: kvq.kvq_q_to_fp16_kv(layers[i][2], layers[i][6], layers[i][4], layers[i][3],
                                                   layers[i][7], layers[i][5], *la, 4), list(range(8)))], 16 * 8)
    out["paged_q4_layers_shared_table"] = {k: {"us": round(v * 1e6, 2), "GB/s": round(wl.bytes_per_launch / v / 1e9, 1)}
                                           for k, v in kt.items()}
    del layers
    # the same Q4 conversions at other batch sizes (8 to 128 sequences x 256
    # new tokens over the same 4096-page caches, 32 rotated seeded paging
    # draws each): the launch's fixed costs against its size
    sweep = {}
    for nb_seq in (8, 16, 64, 128):
        srng = np.random.default_rng(9300 + nb_seq)
        tabs = [tuple(t.from_numpy(a).cuda() for a in synth.paging(srng, nb_seq, 32, 4096, 7936))
                for _ in range(DRAWS)]
        qa = lambda d, tabs=tabs, n=nb_seq: kvq.kvq_fp16_to_q_kv(wl.k, wl.kq, wl.ks, wl.v, wl.vq, wl.vs, n, 0,
                                                                 w.width, w.page_size, *tabs[d], 4)
        da = lambda d, tabs=tabs, n=nb_seq: kvq.kvq_q_to_fp16_kv(wl.kq, wl.ko, wl.ks, wl.vq, wl.vo, wl.vs, n, 0,
                                                                 w.width, w.page_size, *tabs[d], 4)
        for d in range(DRAWS):
            qa(d)
        kt = time_kernels(t, [("quant", qa, list(range(DRAWS))), ("dequant", da, list(range(DRAWS)))], 4 * DRAWS)
        nbytes = 2 * nb_seq * w.width * q_row_bytes(4)
        sweep["batch_%d" % nb_seq] = {k: {"us": round(v * 1e6, 2), "GB/s": round(nbytes / v / 1e9, 1)}
                                      for k, v in kt.items()}
        sweep["batch_%d" % nb_seq]["MB"] = round(nbytes / 1e6, 2)
    out["paged_q4_batch_sweep"] = sweep
    # other block widths on the paged workload
    for wb in (6, 8):
        other = PagedKV(torch, kvq, synth, wbits=wb, share=wl)
        kt = time_kernels(t, [("quant", other.quant, list(range(DRAWS))),
                              ("dequant", other.dequant, list(range(DRAWS)))], 4 * DRAWS)
        out["paged_q%d_cold" % wb] = {k: {"us": round(v * 1e6, 2), "GB/s": round(other.bytes_per_launch / v / 1e9, 1)}
                                      for k, v in kt.items()}
        del other
    # paged 8-bit (high byte) through the per-tensor entry points
    kc = t.zeros(w.shape, dtype=t.uint8, device="cuda")
    vc = t.zeros(w.shape, dtype=t.uint8, device="cuda")

    def narrow(d):
        sl, bt = wl.tables[d]
        kvq.kvq_fp16_to_kv(wl.k, kc, None, 0, wl.v, vc, None, 0, w.batch_size, w.offset, w.width, w.page_size, sl, bt)

    def widen(d):
        sl, bt = wl.tables[d]
        kvq.kvq_kv_to_fp16(kc, wl.ko, None, 0, vc, wl.vo, None, 0, w.batch_size, w.offset, w.width, w.page_size, sl, bt)

    kt = time_kernels(t, [("fp16_to_8bit", narrow, list(range(DRAWS))), ("8bit_to_fp16", widen, list(range(DRAWS)))],
                      4 * DRAWS)
    nb = 2 * rows * fmt_row_bytes(0)
    out["paged_fp8_cold"] = {k: {"us": round(v * 1e6, 2), "GB/s": round(nb / v / 1e9, 1)} for k, v in kt.items()}
    del kc, vc
    # full-prefix widen of the Q4 caches: positions [0, cache_seqlens[b] + width)
    max_len = w.block_table.shape[1] * w.page_size
    pbytes = [2 * int(np.minimum(sl.astype(np.int64) + w.width, max_len).sum()) * q_row_bytes(4)
              for sl, _ in w.extra["tables"]]

    def prefix(d):
        sl, bt = wl.tables[d]
        kvq.kvq_kv_to_fp16_prefix(wl.kq, wl.ko, wl.ks, 4, wl.vq, wl.vo, wl.vs, 4, w.batch_size, w.width, max_len, sl, bt)

    # the same launch with every sequence full (no position past its end)
    full = t.full((w.batch_size,), max_len - w.width, dtype=t.int32, device="cuda")

    def prefix_full(d):
        kvq.kvq_kv_to_fp16_prefix(wl.kq, wl.ko, wl.ks, 4, wl.vq, wl.vo, wl.vs, 4, w.batch_size, w.width, max_len,
                                  full, wl.tables[d][1])

    kt = time_kernels(t, [("prefix", prefix, list(range(DRAWS))), ("full", prefix_full, list(range(DRAWS)))],
                      2 * DRAWS)
    out["prefix_widen_q4_cold"] = {"us": round(kt["prefix"] * 1e6, 2), "MB": round(np.mean(pbytes) / 1e6, 1),
                                   "GB/s": round(np.mean(pbytes) / kt["prefix"] / 1e9, 1)}
    fbytes = 2 * w.batch_size * max_len * q_row_bytes(4)
    out["prefix_widen_q4_all_live_cold"] = {"us": round(kt["full"] * 1e6, 2), "MB": round(fbytes / 1e6, 1),
                                            "GB/s": round(fbytes / kt["full"] / 1e9, 1)}
    # contiguous workloads (hot)
    x = t.from_numpy(synth.fp8_contig().k).cuda()
    o8 = t.empty(x.shape, dtype=t.uint8, device="cuda")
    ob = t.empty(x.shape, dtype=t.float16, device="cuda")
    kt = time_kernels(t, [("to_fp8", lambda _: kvq.kvq_fp16_to_fp8(x, o8, 1, 0, 256), [0]),
                          ("to_fp16", lambda _: kvq.kvq_fp8_to_fp16(o8, ob, 1, 0, 256), [0])], 64)
    nb = 256 * ROW * 3
    out["fp8_contig_hot"] = {k: {"us": round(v * 1e6, 2), "GB/s": round(nb / v / 1e9, 1)} for k, v in kt.items()}
    # the launch floor these small launches sit on: a one-element fill,
    # timed the same way (graph of back-to-back launches)
    one = t.zeros(1, dtype=t.float32, device="cuda")
    kt = time_kernels(t, [("fill", lambda _: one.fill_(1.0), [0])], 64)
    out["launch_floor"] = {"us": round(kt["fill"] * 1e6, 2), "what": "one-element fill, graph of 64 launches"}
    for name, fn, wb in (("q4_contig_hot", synth.q4_contig, 4), ("q6_contig_hot", synth.q6_contig, 6)):
        cw = fn()
        k, v = t.from_numpy(cw.k).cuda(), t.from_numpy(cw.v).cuda()
        cs, ss = kvq.code_shape(cw.shape, wb), kvq.scale_shape(cw.shape)
        kq, vq = t.empty(cs, dtype=t.uint8, device="cuda"), t.empty(cs, dtype=t.uint8, device="cuda")
        ks, vs = t.empty(ss, dtype=t.float16, device="cuda"), t.empty(ss, dtype=t.float16, device="cuda")
        ko, vo = t.empty_like(k), t.empty_like(v)
        a = (cw.batch_size, cw.offset, cw.width)
        kt = time_kernels(t, [
            ("quant", lambda _: kvq.kvq_fp16_to_q_kv(k, kq, ks, v, vq, vs, *a, wbits=wb), [0]),
            ("dequant", lambda _: kvq.kvq_q_to_fp16_kv(kq, ko, ks, vq, vo, vs, *a, wbits=wb), [0])], 32)
        nb = 2 * cw.batch_size * cw.width * q_row_bytes(wb)
        out[name] = {kk: {"us": round(vv * 1e6, 2), "GB/s": round(nb / vv / 1e9, 1)} for kk, vv in kt.items()}
        del k, v, kq, vq, ks, vs, ko, vo
    # the Q6 contiguous shape (189 MB per launch) with 4 rotated buffer sets
    # filled on the device (more than the 256 MB MALL between reuses)
    cw = synth.q6_contig()
    sets = []
    for i in range(4):
        k = synth.device_normal_f16(t, cw.shape, 7000 + 2 * i, std=0.5)
        v = synth.device_normal_f16(t, cw.shape, 7001 + 2 * i, std=0.5)
        cs, ss = kvq.code_shape(cw.shape, 6), kvq.scale_shape(cw.shape)
        sets.append((k, v, t.empty(cs, dtype=t.uint8, device="cuda"), t.empty(cs, dtype=t.uint8, device="cuda"),
                     t.empty(ss, dtype=t.float16, device="cuda"), t.empty(ss, dtype=t.float16, device="cuda"),
                     t.empty_like(k), t.empty_like(v)))
    a6 = (cw.batch_size, cw.offset, cw.width)
    kt = time_kernels(t, [
        ("quant", lambda d: kvq.kvq_fp16_to_q_kv(sets[d][0], sets[d][2], sets[d][4], sets[d][1], sets[d][3],
                                                 sets[d][5], *a6, wbits=6), [0, 1, 2, 3]),
        ("dequant", lambda d: kvq.kvq_q_to_fp16_kv(sets[d][2], sets[d][6], sets[d][4], sets[d][3], sets[d][7],
                                                   sets[d][5], *a6, wbits=6), [0, 1, 2, 3])], 16)
    nb = 2 * cw.batch_size * cw.width * q_row_bytes(6)
    out["q6_contig_cold"] = {kk: {"us": round(vv * 1e6, 2), "GB/s": round(nb / vv / 1e9, 1)} for kk, vv in kt.items()}
    # contiguous 8-bit at the same shape: each set's K cache narrowed into
    # bytes and widened back (101 MB per launch), sets rotated
    b8 = [t.empty(cw.shape, dtype=t.uint8, device="cuda") for _ in range(4)]
    kt = time_kernels(t, [
        ("to_8bit", lambda d: kvq.kvq_fp16_to_fp8(sets[d][0], b8[d], *a6), [0, 1, 2, 3]),
        ("to_fp16", lambda d: kvq.kvq_fp8_to_fp16(b8[d], sets[d][6], *a6), [0, 1, 2, 3])], 16)
    nb = cw.batch_size * cw.width * ROW * 3
    out["fp8_contig_large_cold"] = {kk: {"us": round(vv * 1e6, 2), "GB/s": round(nb / vv / 1e9, 1)}
                                    for kk, vv in kt.items()}
    del b8
    del sets
    # large paged K-Q4 + V-Q6 (8 GiB per fp16 cache), 8 rotated draws:
    # two single-width launches per direction vs one per-tensor launch
    mw = synth.mix_paged(draws=8)
    shape = mw.shape
    k = synth.device_normal_f16(t, shape, mw.extra["device_seed"])
    v = synth.device_normal_f16(t, shape, mw.extra["device_seed"] + 1)
    kq = t.zeros(kvq.code_shape(shape, 4), dtype=t.uint8, device="cuda")
    vq = t.zeros(kvq.code_shape(shape, 6), dtype=t.uint8, device="cuda")
    ks = t.zeros(kvq.scale_shape(shape), dtype=t.float16, device="cuda")
    vs = t.zeros(kvq.scale_shape(shape), dtype=t.float16, device="cuda")
    ko, vo = t.empty_like(k), t.empty_like(v)
    tabs = [(t.from_numpy(sl).cuda(), t.from_numpy(bt).cuda()) for sl, bt in mw.extra["tables"]]
    nd = len(tabs)

    def ar(d):
        return (mw.batch_size, mw.offset, mw.width, mw.page_size) + tabs[d]

    kt = time_kernels(t, [
        ("quant_k4_then_v6", lambda d: (kvq.kvq_fp16_to_q_kv(k, kq, ks, None, None, None, *ar(d), 4),
                                        kvq.kvq_fp16_to_q_kv(None, None, None, v, vq, vs, *ar(d), 6)), list(range(nd))),
        ("dequant_k4_then_v6", lambda d: (kvq.kvq_q_to_fp16_kv(kq, ko, ks, None, None, None, *ar(d), 4),
                                          kvq.kvq_q_to_fp16_kv(None, None, None, vq, vo, vs, *ar(d), 6)), list(range(nd))),
        ("quant_one_launch", lambda d: kvq.kvq_fp16_to_kv(k, kq, ks, 4, v, vq, vs, 6, *ar(d)), list(range(nd))),
        ("dequant_one_launch", lambda d: kvq.kvq_kv_to_fp16(kq, ko, ks, 4, vq, vo, vs, 6, *ar(d)), list(range(nd)))],
        4 * nd)
    nb = mw.batch_size * mw.width * (q_row_bytes(4) + q_row_bytes(6))
    out["mix_paged_cold"] = {kk: {"us": round(vv * 1e6, 2), "GB/s": round(nb / vv / 1e9, 1)} for kk, vv in kt.items()}
    del k, v, kq, vq, ks, vs, ko, vo
    # a plain device copy moving the same bytes as one paged-Q4 launch
    # (read half, write half): the practical bandwidth at this launch size
    n = 2 * 32 * 256 * q_row_bytes(4) // 2 // 2
    src = t.empty((DRAWS, n), dtype=t.float16, device="cuda")
    dst = t.empty((DRAWS, n), dtype=t.float16, device="cuda")
    kt = time_kernels(t, [("copy", lambda d: dst[d].copy_(src[d]), list(range(DRAWS)))], 4 * DRAWS)
    out["copy_same_bytes"] = {"us": round(kt["copy"] * 1e6, 2), "GB/s": round(4 * n / kt["copy"] / 1e9, 1)}
    del src, dst
    ids_a, ids_b = mw.extra["ids_a"], mw.extra["ids_b"]
    reps = 200
    t0 = time.perf_counter()
    for _ in range(reps):
        m = kvq.kvq_count_match(ids_a, ids_b, ids_a.size)
    dt = (time.perf_counter() - t0) / reps
    out["count_match"] = {"us": round(dt * 1e6, 2), "match": m, "n": int(ids_a.size)}
    torch.cuda.empty_cache()
    return out


def calibrate_copy(torch):
    """A plain device-to-device copy of 1 GiB (fp16 elementwise copy kernel)
    for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    n = (1 << 30) // 2
    a = torch.ones(n, dtype=torch.float16, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log("copy calibration: 3 x 1 GiB fp16 copies")


if __name__ == "__main__":
    main()
