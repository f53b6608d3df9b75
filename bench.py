#!/usr/bin/env python3
"""Throughput of the Ulysses all_to_all_4D exchange on one MI355X.

One step = one mode-0 exchange (scatter heads, gather sequence) followed by
one mode-1 exchange (its inverse) of the video-DiT-scale workload: w = 8
virtual ranks, B = 1, S_local = 9450 (75 600 tokens in all), H = 40 heads
(5 per rank), D = 128, bf16, N(0,1) seeded synthetic data, all ranks stacked
in one HBM allocation per tensor (FastVideo "ulysses_a2a" API page, method
run_armed, for the two modes).  Inputs are resident in HBM before the timed
region starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

prints ONE JSON line.  `value` is achieved HBM read+write GB/s over the K
timed steps (algorithmic bytes: every element read once and written once per
exchange, 2 * 774 144 000 B per exchange, two exchanges per step); the timed region holds the K steps and
nothing else.  The `roofline` object is for the slower of the two
permutation kernels, its average launch duration taken from K back-to-back
launches between HIP events recorded on the stream the kernel is launched on.
`per_config` gives every workload's rate in both modes (and the four-plane
workload chunked), each output checked against the oracle outside the timed
launches.  `cpu_baseline` times the plain CPU oracle on the host on a bounded
sample of the same workload, on one thread and with the senders split over
threads (`all_cores`, with the CPU count and model).  A device-to-device copy
of the same byte count is timed beside it (`memcpy_GBps`).

    python bench.py --traffic-from DIR

reads the counter CSVs of two rocprofv3 --pmc runs (FETCH_SIZE, then
WRITE_SIZE) under DIR and writes profiles/traffic_direct_video_dit.json, which
later runs report as roofline.traffic while the built library is unchanged.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E, AMD's published peak
WORKLOAD = "video_dit"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_direct_video_dit.json")
DIRECT_KERNEL = "ua2a_direct"        # ua2a_direct_kernel (1-D grid) and ua2a_direct3d_kernel
COPY_KERNEL_HINT = "copyBuffer"     # the runtime's device-to-device copy kernel


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def library_hash() -> str:
    """Hash of the built library (kernels and launch logic; the build is
    deterministic, so comment-only source edits keep it): traffic counters
    are valid only for the build they were taken on."""
    import ulysses_all_re_amd as ua
    h = hashlib.sha256()
    with open(ua.LIBRARY, "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic():
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("library_hash") != library_hash():
        return None          # counters were taken on another build of the kernels
    return t


def cpu_baseline(x_cpu, w, steps, moved_bytes, workload):
    """The oracle as it stands on `steps` full round trips: on one thread, and
    with each exchange's senders split over threads (one per sender, up to the
    host share of cores; each thread makes one per-rank oracle call, and the
    result must equal the single-thread one)."""
    import numpy as np

    import oracle
    from workloads import BITS_VIEW
    xb = x_cpu.view(BITS_VIEW[x_cpu.element_size()]).numpy()
    t0 = time.perf_counter()
    for _ in range(steps):
        y = oracle.exchange(xb, 0, w)
        z = oracle.exchange(y, 1, w)
    dt = time.perf_counter() - t0
    threads, dt_n = 1, 0.0
    for k in range(steps):
        yn, s0, threads = oracle_on_threads(xb, 0, w)
        zn, s1, _ = oracle_on_threads(yn, 1, w)
        dt_n += s0 + s1
        if k == 0 and not (np.array_equal(yn, y) and np.array_equal(zn, z)):
            raise SystemExit("the threaded oracle differs from the single-thread oracle")
        del yn, zn
    algorithmic = 2 * moved_bytes * steps
    return {
        "value": round(algorithmic / dt / 1e9, 3),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{steps} full {workload} round trips (mode 0 then mode 1, {algorithmic} "
                  f"algorithmic bytes) through the C nested-loop oracle, one thread, {dt:.2f} s",
        "nproc": os.cpu_count(),
        "cpu_model": cpu_model(),
        "all_cores": {
            "value": round(algorithmic / dt_n / 1e9, 3),
            "unit": "GB/s",
            "cores": threads,
            "kind": "oracle",
            "sample": f"the same {steps} round trips with each exchange's {w} senders split over "
                      f"{threads} threads (one per-rank oracle call per thread; host share "
                      f"{HOST_CPU_SHARE} of {os.cpu_count()} CPUs), {dt_n:.2f} s",
        },
    }


def rotation(tensor_bytes: int) -> int:
    """Buffer sets to rotate through so that a cycle moves about 1 GiB: small
    tensors are then timed against HBM, not the 256 MB on-package cache (at
    most 64 sets; one for tensors of 512 MiB and more)."""
    return max(1, min(64, -(-(1 << 30) // (2 * tensor_bytes))))


PER_CONFIG = (("tiny", False), ("mid", False), ("video_dit", False), ("chunked", False),
              ("chunked", True), ("awkward", False))


def per_config(dev, stream, K, main=None):
    """The five workloads, both modes (the chunked workload also chunked):
    back-to-back microseconds per exchange over K launches (bound calls,
    Plan.bind, one per buffer set) rotating through buffer sets, GB/s and fraction of 8 TB/s on the algorithmic bytes, and
    whether the output equals the oracle's byte for byte (checked outside
    the timed launches).  Mode-0 inputs come from the workload's first seed,
    mode-1 inputs are an independent tensor of the mode-1 shape from its
    second seed.  `main` = (x, y, z, avg0_ms, avg1_ms) of the bench's own
    video-DiT run, whose timings and outputs are reused (z = mode 1 of y)."""
    import numpy as np
    import torch

    import oracle
    import ulysses_all_re_amd as ua
    from workloads import BITS_VIEW, CONFIGS, DTYPES, make_tensor

    out = {}
    for name, chunked in PER_CONFIG:
        c = CONFIGS[name]
        w, B, S, H, D = c["w"], c["B"], c["S_local"], c["H"], c["D"]
        dt = DTYPES[c["dtype"]]
        e = torch.empty((), dtype=dt).element_size()
        lay = ua.ua2a_layout(w, B, S, H, D, e)
        moved = lay["moved_bytes"]
        key = f"{name}_chunked" if chunked else name
        entry = {}
        if name == "video_dit" and not chunked and main is not None:
            x, y, z, avg0, avg1 = main
            bits = BITS_VIEW[e]
            xb = x.cpu().view(bits).numpy()
            yb = y.cpu().view(bits).numpy()
            exact0 = bool(np.array_equal(yb, oracle.exchange(xb, 0, w)))
            exact1 = bool(np.array_equal(z.cpu().view(bits).numpy(), oracle.exchange(yb, 1, w)))
            for m, avg, exact in ((0, avg0, exact0), (1, avg1, exact1)):
                gb = moved / (avg * 1e-3) / 1e9
                entry[f"mode{m}"] = {"us": round(avg * 1e3, 2), "GBps": round(gb, 1),
                                     "frac": round(gb / PEAK_HBM_GBPS, 4), "bit_exact": exact,
                                     "input": "seed 0" if m == 0 else "mode 0's output"}
            entry["buffer_sets"] = 1
            out[key] = entry
            continue
        window = torch.empty(lay["window_bytes"], dtype=torch.uint8, device=dev) if chunked else None
        plan = ua.Plan(w, B, S, H, D, dt, window=window, device=dev)
        rot = rotation(lay["tensor_bytes"])
        for mode in (0, 1):
            shape = (w, B, S, H, D) if mode == 0 else (w, B, S * w, H // w, D)
            x_cpu = make_tensor(shape, c["dtype"], c["dist"], c["seed0"] if mode == 0 else c["seed1"])
            xs = [x_cpu.to(dev)]
            xs += [xs[0].clone() for _ in range(rot - 1)]
            ys = [torch.empty(plan.out_shape(mode), dtype=dt, device=dev) for _ in range(rot)]
            plan.exchange(xs[0], mode, chunked, out=ys[0], stream=stream)
            torch.cuda.synchronize(dev)
            want = oracle.exchange(x_cpu.view(BITS_VIEW[e]).numpy(), mode, w, chunked=chunked)
            exact = bool(np.array_equal(ys[0].cpu().view(BITS_VIEW[e]).numpy(), want))
            del want
            # one bound call per buffer set: checked once, so a small exchange's
            # loop is not paced by the per-call checks of exchange()
            calls = [plan.bind(xs[i], mode, chunked, out=ys[i], stream=stream) for i in range(rot)]
            for i in range(2 * rot):                       # warm-up, every set at least twice
                calls[i % rot]()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize(dev)
            a.record(stream)
            for i in range(K):
                calls[i % rot]()
            b.record(stream)
            torch.cuda.synchronize(dev)
            us = a.elapsed_time(b) * 1e3 / K
            gb = moved / (us * 1e-6) / 1e9
            info = plan.describe(xs[0], mode, chunked, out=ys[0])
            entry[f"mode{mode}"] = {"us": round(us, 2), "GBps": round(gb, 1),
                                    "frac": round(gb / PEAK_HBM_GBPS, 4), "bit_exact": exact,
                                    "launches": info["launches"],
                                    "path": {ua.UA2A_PATH_DIRECT: "direct", ua.UA2A_PATH_LDS: "lds"}[info["path"]],
                                    "input": f"seed {c['seed0'] if mode == 0 else c['seed1']}"
                                             if c["dist"] != "index" else "flat index"}
            del xs, ys, calls
        entry["buffer_sets"] = rot
        entry["bytes_per_exchange"] = moved
        out[key] = entry
        plan.close()
        del window
        torch.cuda.empty_cache()
    return out


def run(args):
    import torch

    import ulysses_all_re_amd as ua
    from workloads import CONFIGS, DTYPES, MEASURE, make_tensor

    name = args.workload
    c = {**CONFIGS, **MEASURE}[name]
    w, B, S, H, D = c["w"], c["B"], c["S_local"], c["H"], c["D"]
    dt = DTYPES[c["dtype"]]
    e = torch.empty((), dtype=dt).element_size()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    lay = ua.ua2a_layout(w, B, S, H, D, e)
    moved = lay["moved_bytes"]                     # per exchange: read + write
    chunked = bool(args.chunked)
    log(f"workload {name} w={w} B={B} S_local={S} H={H} D={D} {c['dtype']}, "
        f"{lay['tensor_bytes']} B per tensor, chunked={chunked}")
    dist = "index_bits" if c["dist"] == "index" else c["dist"]
    x_cpu = make_tensor((w, B, S, H, D), c["dtype"], dist, c["seed0"])
    x = x_cpu.to(dev)
    window = torch.empty(lay["window_bytes"], dtype=torch.uint8, device=dev) if chunked else None
    plan = ua.Plan(w, B, S, H, D, dt, blocks=args.blocks, window=window, device=dev)
    plan.set_path({"auto": ua.UA2A_PATH_AUTO, "direct": ua.UA2A_PATH_DIRECT,
                   "lds": ua.UA2A_PATH_LDS}[args.path])
    stream = torch.cuda.current_stream(dev)
    bits = {1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}[e]

    def round_trips_ok():
        if args.ranks is None:
            return all(torch.equal(zk.view(bits), xk.view(bits)) for xk, _, zk in sets)
        return torch.equal(torch.stack([t.view(bits) for t in zs]), x.view(bits))

    # Buffer sets the exchanges rotate through: enough that a cycle moves
    # about 1 GiB, so that tensors smaller than the 256 MB Infinity Cache are
    # timed against HBM too (at most 64 sets; one for the video-DiT tensors).
    rotate = args.rotate if args.rotate > 0 else rotation(lay["tensor_bytes"])
    if args.ranks is not None or args.graph:
        rotate = 1
    if args.ranks is None:
        sets = []
        for k in range(rotate):
            xk = x if k == 0 else x.clone()
            sets.append((xk, torch.empty(plan.out_shape(0), dtype=dt, device=dev),
                         torch.empty(plan.out_shape(1), dtype=dt, device=dev)))
        x, y, z = sets[0]
        info0 = plan.describe(x, 0, chunked, out=y)
        info1 = plan.describe(y, 1, chunked, out=z)
        turn = [0, 0]

        def ex0():
            xk, yk, _ = sets[turn[0]]
            turn[0] = (turn[0] + 1) % rotate
            plan.exchange(xk, 0, chunked, out=yk, stream=stream)

        def ex1():
            _, yk, zk = sets[turn[1]]
            turn[1] = (turn[1] + 1) % rotate
            plan.exchange(yk, 1, chunked, out=zk, stream=stream)
    else:
        # per-rank allocations: every rank's tensors are allocations of their own
        if chunked:
            raise SystemExit("--ranks has no chunked form")
        xs = [x[k].clone() for k in range(w)]
        ys = [torch.empty(plan.out_shape(0)[1:], dtype=dt, device=dev) for _ in range(w)]
        zs = [torch.empty(plan.out_shape(1)[1:], dtype=dt, device=dev) for _ in range(w)]
        senders = [(0, w)] if args.ranks == "all" else [(j, 1) for j in range(w)]
        calls0 = [plan.bind_ranks(xs, 0, ys, f, n, stream) for f, n in senders]
        calls1 = [plan.bind_ranks(ys, 1, zs, f, n, stream) for f, n in senders]
        info0 = plan.describe_ranks(xs, ys, 0, *senders[0])
        info1 = plan.describe_ranks(ys, zs, 1, *senders[0])
        info0["launches"] = info1["launches"] = len(senders)

        def ex0():
            for call in calls0:
                call()

        def ex1():
            for call in calls1:
                call()
    log(f"mode 0 launch {info0}")
    log(f"mode 1 launch {info1}")

    # one round trip through every buffer set, checked before anything is timed
    for _ in range(rotate):
        ex0()
        ex1()
    torch.cuda.synchronize(dev)
    if not round_trips_ok():
        raise SystemExit("round trip did not return the input; refusing to report a number")
    log(f"round trip bit-exact on {rotate} buffer set(s)")
    # the W warm-up steps come right before the timed region, with no check or
    # host wait between them (a pause there left the first timed steps slower)
    for _ in range(args.warmup):
        ex0()
        ex1()
    log(f"warmup done ({args.warmup} steps)")

    K = args.steps

    def timed(fn, n):
        """ms for n back-to-back calls of fn, HIP events on the launch stream."""
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize(dev)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize(dev)
        return a.elapsed_time(b)

    def step():
        ex0()
        ex1()

    if args.graph and args.ranks is not None:
        raise SystemExit("--graph times the rank-stacked exchange only")
    if args.graph:
        # one step captured once as a HIP graph; the timed region replays it
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize(dev)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            plan.exchange(x, 0, chunked, out=y, stream=side)
            plan.exchange(y, 1, chunked, out=z, stream=side)
        torch.cuda.synchronize(dev)
        bits_z = z.view(bits)
        bits_z.fill_(-1)
        graph.replay()
        torch.cuda.synchronize(dev)
        if not torch.equal(z.view(bits), x.view(bits)):
            raise SystemExit("graph replay did not return the input; refusing to report a number")
        step = graph.replay
        log("timing graph replays of one step")

    # the timed region: K whole steps, nothing else on the stream
    total_ms = timed(step, K)
    log(f"timed {K} steps in {total_ms:.3f} ms")
    # per-exchange averages for the roofline: each mode K times back to back
    avg0 = timed(ex0, K) / K
    avg1 = timed(ex1, K) / K
    # device-to-device copy of the same byte count, timed the same way (over
    # the same rotation of buffer sets)
    cps = [torch.empty_like(x) for _ in range(rotate)]
    cturn = [0]

    def copy_leg():
        k = cturn[0]
        cturn[0] = (k + 1) % rotate
        cps[k].copy_(sets[k][0] if args.ranks is None else x)

    timed(copy_leg, 3)
    avgc = timed(copy_leg, K) / K
    if not round_trips_ok():
        raise SystemExit("round trip no longer returns the input after the timed steps; "
                         "refusing to report a number")
    log(f"per exchange: mode 0 {avg0 * 1e3:.1f} us, mode 1 {avg1 * 1e3:.1f} us, "
        f"copy {avgc * 1e3:.1f} us")

    def gbps(ms):
        return moved / (ms * 1e-3) / 1e9

    value = 2 * moved * K / (total_ms * 1e-3) / 1e9
    traffic = load_traffic() if (name == WORKLOAD and not chunked and args.path == "auto") else None
    if args.ranks is not None:
        traffic = None
    dom_mode, dom_avg = (0, avg0) if avg0 >= avg1 else (1, avg1)
    dom_info = info0 if dom_mode == 0 else info1
    if args.ranks is not None:
        kname = "ua2a_ranks_kernel"
    elif chunked and dom_info["path"] == ua.UA2A_PATH_DIRECT:
        kname = "ua2a_chunked_kernel" if dom_info["grid_dims"] == 3 else "ua2a_chunked_flat_kernel"
    elif chunked:
        kname = "ua2a_lds_chunked_kernel"
    elif dom_info["path"] == ua.UA2A_PATH_DIRECT:
        kname = "ua2a_direct3d_kernel" if dom_info["grid_dims"] == 3 else "ua2a_direct_kernel"
    else:
        kname = "ua2a_lds_kernel"
    roofline = {
        "bound": "hbm",
        "kernel": f"{kname}<{dom_info['vector_bytes']}, mode {dom_mode}>"
                  + (f", {w} launches of one sender each" if args.ranks == "one" else ""),
        "achieved": round(gbps(dom_avg), 1),
        "peak": PEAK_HBM_GBPS,
        "unit": "GB/s",
        "frac": round(gbps(dom_avg) / PEAK_HBM_GBPS, 4),
        "traffic": traffic[f"mode{dom_mode}_bytes_per_launch"] if traffic else None,
        "algorithmic_bytes": moved,
        "avg_launch_us": round(dom_avg * 1e3, 2),
    }

    def mode_entry(avg, info, m):
        return {"GBps": round(gbps(avg), 1), "us_per_exchange": round(avg * 1e3, 2),
                "pct_peak": round(100 * gbps(avg) / PEAK_HBM_GBPS, 2),
                "traffic_bytes": traffic[f"mode{m}_bytes_per_launch"] if traffic else None,
                "launch": info}

    result = {
        "metric": "achieved HBM GB/s (read+write) and % of peak, mode0/mode1, 1 MI355X",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": c["dtype"],
        "data": "synthetic",
        "config": {"workload": name, "w": w, "B": B, "S_local": S, "S_global": S * w,
                   "H": H, "D": D, "elem": c["dtype"], "run_bytes": lay["run_bytes"],
                   "chunked": chunked, "path": args.path, "graph": bool(args.graph),
                   "ranks": args.ranks,
                   "step": "mode 0 then mode 1",
                   "bytes_per_step": 2 * moved,
                   "buffer_sets": rotate,
                   "cache_resident": rotate * lay["tensor_bytes"] * 2 <= 256 * 2 ** 20},
        "pct_peak": round(100 * value / PEAK_HBM_GBPS, 2),
        "mode0": mode_entry(avg0, info0, 0),
        "mode1": mode_entry(avg1, info1, 1),
        "memcpy_GBps": round(gbps(avgc), 1),
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if chunked:
        # what the window path actually moves: permute into the window + copy out of it
        result["window_path_bytes_per_exchange"] = 2 * moved
    if not args.no_per_config and args.ranks is None and not args.graph:
        log("per-configuration rates and oracle checks")
        main = (x, y, z, avg0, avg1) if (name == WORKLOAD and not chunked and args.path == "auto"
                                         and rotate == 1) else None
        result["per_config"] = per_config(dev, stream, max(K, 20), main)
    if not args.no_cpu_baseline:
        log(f"cpu baseline: {args.cpu_steps} oracle round trips, one thread and threaded")
        result["cpu_baseline"] = cpu_baseline(x_cpu, w, args.cpu_steps, moved, name)
    plan.close()
    print(json.dumps(result), flush=True)


def run_overlap(args):
    """Mode 0 followed by a per-receiver consumer, serial versus pipelined on
    readiness credits.  The consumer of receiving rank r is one bf16 GEMM on
    its gathered sequence, [B*S_global, H/w*D] @ [H/w*D, H/w*D] (a stand-in for
    the projection or attention that follows the exchange; torch.matmul).
    Serial: exchange, then the w GEMMs, one stream.  Pipelined: the publishing
    exchange (one part per receiving rank) on the main stream; on a second
    stream, for each r, a wait for r's credit, then r's GEMM.  Prints one JSON
    line.  `--publish-blocks` caps the grid of the publishing exchange (its
    parts then loop over their tiles): beside the GEMMs, 8192 single-wave
    workgroups measured best, ahead of the uncapped one-tile-per-workgroup
    grid (also timed, as `pipelined_uncapped`) and of smaller caps."""
    import torch

    import ulysses_all_re_amd as ua
    from workloads import CONFIGS, DTYPES, MEASURE, make_tensor

    name = args.workload
    c = {**CONFIGS, **MEASURE}[name]
    w, B, S, H, D = c["w"], c["B"], c["S_local"], c["H"], c["D"]
    dt = DTYPES[c["dtype"]]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    plan = ua.Plan(w, B, S, H, D, dt, device=dev)
    pub = ua.Plan(w, B, S, H, D, dt, blocks=args.publish_blocks, device=dev)
    x = make_tensor((w, B, S, H, D), c["dtype"], "normal", c["seed0"]).to(dev)
    y = torch.empty(plan.out_shape(0), dtype=dt, device=dev)
    k = (H // w) * D
    rows = B * S * w
    wgt = (torch.randn(k, k, generator=torch.Generator("cpu").manual_seed(3)) / k ** 0.5).to(dt).to(dev)
    z = torch.empty(w, rows, k, dtype=dt, device=dev)
    credits = torch.zeros(w, dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    main = torch.cuda.current_stream(dev)
    side = torch.cuda.Stream(dev)
    epoch = [0]

    def consume(r):
        torch.matmul(y[r].view(rows, k), wgt, out=z[r])

    def serial():
        plan.exchange(x, 0, out=y, stream=main)
        for r in range(w):
            consume(r)

    def pipelined(p=pub):
        main.wait_stream(side)               # the previous step's consumers are done with y
        p.exchange_publish(x, 0, credits, out=y, stream=main)
        epoch[0] += 1
        for r in range(w):
            ua.wait_credits(credits, r, 1, epoch[0], status, stream=side)
            with torch.cuda.stream(side):
                consume(r)
        main.wait_stream(side)

    def timed(fn, n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize(dev)
        a.record(main)
        for _ in range(n):
            fn()
        b.record(main)
        torch.cuda.synchronize(dev)
        return a.elapsed_time(b) / n

    for _ in range(args.warmup):
        serial()
        pipelined()
        pipelined(plan)
    torch.cuda.synchronize(dev)
    serial()
    ref = z.clone()
    for p in (pub, plan):
        z.zero_()
        pipelined(p)
        torch.cuda.synchronize(dev)
        if int(status.item()) != 0:
            raise SystemExit("a credit wait timed out; refusing to report a number")
        if not torch.equal(z, ref):
            raise SystemExit("pipelined consumers saw different data than serial ones")
    K = args.steps
    t_exchange = timed(lambda: plan.exchange(x, 0, out=y, stream=main), K)

    def publish_only():
        pub.exchange_publish(x, 0, credits, out=y, stream=main)
        epoch[0] += 1

    t_publish = timed(publish_only, K)

    def consume_all():
        for r in range(w):
            consume(r)

    t_consume = timed(consume_all, K)
    t_serial = timed(serial, K)
    t_pipe = timed(pipelined, K)
    t_pipe_uncapped = timed(lambda: pipelined(plan), K)
    if int(status.item()) != 0:
        raise SystemExit("a credit wait timed out; refusing to report a number")
    flops = 2.0 * rows * k * k * w
    result = {
        "metric": "mode-0 exchange + per-rank consumer, serial vs pipelined on readiness credits",
        "value": round(t_serial / t_pipe, 4), "unit": "x (serial time / pipelined time)",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "higher_is_better": True,
        "dtype": c["dtype"], "data": "synthetic",
        "config": {"workload": name, "w": w, "B": B, "S_local": S, "H": H, "D": D,
                   "consumer": f"per rank: [{rows}, {k}] @ [{k}, {k}] {c['dtype']} GEMM (torch.matmul)",
                   "parts": w, "publish_blocks": args.publish_blocks},
        "ms": {"exchange": round(t_exchange, 4), "exchange_publish": round(t_publish, 4),
               "consumers": round(t_consume, 4), "serial": round(t_serial, 4),
               "pipelined": round(t_pipe, 4), "pipelined_uncapped": round(t_pipe_uncapped, 4)},
        "publish_overhead": round(t_publish / t_exchange - 1, 4),
        "consumer_TFLOPs": round(flops / (t_consume * 1e-3) / 1e12, 1),
    }
    plan.close()
    pub.close()
    print(json.dumps(result), flush=True)


# ------------------------------------------------------------ pack / unpack

def run_pack(args):
    """The per-rank exchange in two steps through receive windows, as one
    device of a multi-device exchange runs it: ua2a_pack_ranks with one
    sender per launch (its push into every receiver's window), then
    ua2a_unpack_ranks with one receiver per launch (window -> output).  Both
    modes; next to it, the direct push of one sender per launch
    (ua2a_exchange_ranks), which writes into the receivers' outputs.  Each
    launch moves one rank's tensor in and one out (tensor / w each way); the
    line gives microseconds and GB/s per launch, averaged over K rounds of w
    launches.  The round trip (pack + unpack in mode 0, then in mode 1) is
    checked to return the input before timing.  Prints one JSON line."""
    import torch

    import ulysses_all_re_amd as ua
    from workloads import CONFIGS, DTYPES, MEASURE, make_tensor

    name = args.workload
    c = {**CONFIGS, **MEASURE}[name]
    w, B, S, H, D = c["w"], c["B"], c["S_local"], c["H"], c["D"]
    dt = DTYPES[c["dtype"]]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    plan = ua.Plan(w, B, S, H, D, dt, device=dev)
    plan.set_path({"auto": ua.UA2A_PATH_AUTO, "direct": ua.UA2A_PATH_DIRECT,
                   "lds": ua.UA2A_PATH_LDS}[args.path])
    dist = "index_bits" if c["dist"] == "index" else c["dist"]
    x = make_tensor((w, B, S, H, D), c["dtype"], dist, c["seed0"]).to(dev)
    xs = [x[k].clone() for k in range(w)]
    del x
    wins = [torch.empty(plan.window_shape(), dtype=dt, device=dev) for _ in range(w)]
    ys = [torch.empty(plan.out_shape(0)[1:], dtype=dt, device=dev) for _ in range(w)]
    zs = [torch.empty(plan.out_shape(1)[1:], dtype=dt, device=dev) for _ in range(w)]
    per_launch = 2 * plan.layout["tensor_bytes"] // w

    def pack(mode, src):
        for k in range(w):
            plan.pack_ranks(src, mode, wins, first=k, count=1, stream=stream)

    def unpack(mode, dst):
        for q in range(w):
            plan.unpack_ranks(wins, mode, dst, first=q, count=1, stream=stream)

    pushes = {m: [plan.bind_ranks(src, m, dst, k, 1, stream) for k in range(w)]
              for m, src, dst in ((0, xs, ys), (1, ys, zs))}
    pack(0, xs)
    unpack(0, ys)
    pack(1, ys)
    unpack(1, zs)
    torch.cuda.synchronize(dev)
    bits = {1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}[xs[0].element_size()]
    if not all(torch.equal(z.view(bits), x.view(bits)) for z, x in zip(zs, xs)):
        raise SystemExit("pack + unpack round trip did not return the input; refusing to report a number")
    K = args.steps

    def timed(fn):
        for _ in range(max(1, args.warmup)):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize(dev)
        a.record(stream)
        for _ in range(K):
            fn()
        b.record(stream)
        torch.cuda.synchronize(dev)
        us = a.elapsed_time(b) * 1e3 / (K * w)
        return {"us_per_launch": round(us, 2), "GBps": round(per_launch / (us * 1e-6) / 1e9, 1)}

    def push_all(m):
        for call in pushes[m]:
            call()

    result = {
        "metric": "per-launch time of one sender's pack and one receiver's unpack, 1 MI355X",
        "unit": "us per launch", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "dtype": c["dtype"], "data": "synthetic",
        "config": {"workload": name, "w": w, "B": B, "S_local": S, "H": H, "D": D,
                   "run_bytes": plan.layout["run_bytes"], "bytes_per_launch": per_launch,
                   "path": args.path},
        "mode0": {"pack": timed(lambda: pack(0, xs)), "unpack": timed(lambda: unpack(0, ys)),
                  "direct_push": timed(lambda: push_all(0))},
        "mode1": {"pack": timed(lambda: pack(1, ys)), "unpack": timed(lambda: unpack(1, zs)),
                  "direct_push": timed(lambda: push_all(1))},
    }
    plan.close()
    print(json.dumps(result), flush=True)


# ------------------------------------------------------------ size sweep

SWEEP_S_LOCAL = (50, 100, 200, 305, 400, 600, 800, 1200, 1600, 2400, 3200, 4800, 6400)


def fit_line(xs, ys):
    """Least-squares y = a + b x."""
    n = len(xs)
    mx, my = sum(xs) / n, sum(ys) / n
    b = sum((x - mx) * (y - my) for x, y in zip(xs, ys)) / sum((x - mx) ** 2 for x in xs)
    return my - b * mx, b


def run_sweep(args):
    """The exchange's launch time against its size: the video-DiT head layout
    (w = 8, H = 40, D = 128, bf16, 1280-byte runs) at S_local from 50 to 6400
    tokens per rank (4 to 524 MB per tensor), both modes, K back-to-back
    launches rotating through buffer sets (about 1 GiB per cycle).  One JSON
    line per (mode, size), then per mode the fit t = t0 + moved / BW over the
    sizes of 64 MB and up, and each size's excess over that line."""
    import torch

    import ulysses_all_re_amd as ua

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    K = args.steps
    w, B, H, D = 8, 1, 40, 128
    pts = {0: [], 1: []}
    for S in SWEEP_S_LOCAL:
        plan = ua.Plan(w, B, S, H, D, torch.bfloat16, device=dev)
        n = plan.layout["tensor_bytes"]
        sets = rotation(n)
        for mode in (0, 1):
            xs = [torch.ones(plan.in_shape(mode), dtype=torch.bfloat16, device=dev) for _ in range(sets)]
            ys = [torch.empty(plan.out_shape(mode), dtype=torch.bfloat16, device=dev) for _ in range(sets)]
            for i in range(2 * sets):
                plan.exchange(xs[i % sets], mode, out=ys[i % sets], stream=stream)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize(dev)
            a.record(stream)
            for i in range(K):
                plan.exchange(xs[i % sets], mode, out=ys[i % sets], stream=stream)
            b.record(stream)
            torch.cuda.synchronize(dev)
            us = a.elapsed_time(b) * 1e3 / K
            moved = 2 * n
            pts[mode].append((moved, us))
            print(json.dumps({"record": "sweep", "mode": mode, "S_local": S, "bytes_moved": moved,
                              "buffer_sets": sets, "us": round(us, 3),
                              "GBps": round(moved / (us * 1e-6) / 1e9, 1)}), flush=True)
            del xs, ys
        plan.close()
        torch.cuda.empty_cache()
    for mode, p in pts.items():
        big = [(m, t) for m, t in p if m >= 128 << 20]
        t0, slope = fit_line([m for m, _ in big], [t for _, t in big])
        bw = 1e-3 / slope            # bytes per us -> GB/s
        excess = {str(m): round(t - (t0 + m * slope), 2) for m, t in p}
        print(json.dumps({"record": "sweep_fit", "mode": mode, "t0_us": round(t0, 3),
                          "BW_GBps": round(bw, 1), "fit_from_bytes_moved": 128 << 20,
                          "excess_us_by_bytes_moved": excess}), flush=True)


# ------------------------------------------------- per-configuration records

RECORD_WORKLOADS = ("tiny", "mid", "video_dit", "chunked", "awkward")
HOST_CPU_SHARE = 16      # host threads a GPU job may use on the MI355X hosts


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_on_threads(xb, mode, w):
    """The oracle over every sender, the senders split into contiguous ranges
    run by as many threads as there are senders (at most the host share): each
    range is one per-rank oracle call, which writes only the runs its senders
    send, so the ranges write disjoint bytes of the same output.  Returns
    (output, seconds, threads)."""
    import concurrent.futures

    import numpy as np

    import oracle

    B, S_local, H, D = oracle.local_shape(xb.shape, mode, w)
    out = np.empty((w, B, S_local * w, H // w, D) if mode == 0 else (w, B, S_local, H, D),
                   dtype=xb.dtype)
    threads = max(1, min(w, HOST_CPU_SHARE, os.cpu_count() or 1))
    cuts = [w * t // threads for t in range(threads + 1)]
    xs, outs = [xb[k] for k in range(w)], [out[k] for k in range(w)]
    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(threads) as pool:     # the calls release the GIL
        for f in [pool.submit(oracle.exchange_ranks, xs, outs, mode, cuts[t], cuts[t + 1] - cuts[t])
                  for t in range(threads)]:
            f.result()
    return out, time.perf_counter() - t0, threads


def run_records(args):
    """One JSON line per (workload, mode, chunked) over the five workloads: the
    chunked form only where the workload asks for it.  Each record holds the
    per-launch time from HIP events recorded around every one of `--steps`
    launches on the launch stream (median, min; the launches rotate through
    buffer sets as in the main bench, so small tensors are timed against HBM),
    the average of the same number of back-to-back launches, the runtime's
    device-to-device copy of the same bytes timed per launch the same way, the
    oracle's single-thread time on the same input (and, unchunked, its time
    with the senders split over threads, one per sender up to the host share,
    checked equal to the single-thread result), whether the output equals the
    oracle's byte for byte, and the SHA-256 of the input bytes.  Mode-0
    inputs use the workload's first seed, mode-1 inputs an independent tensor
    of the mode-1 shape from its second seed."""
    import statistics

    import numpy as np
    import torch

    import oracle
    import ulysses_all_re_amd as ua
    from workloads import BITS_VIEW, CONFIGS, DTYPES, make_tensor

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    K = args.steps
    names = (args.records_workload,) if args.records_workload else RECORD_WORKLOADS
    for name in names:
        c = CONFIGS[name]
        w, B, S, H, D = c["w"], c["B"], c["S_local"], c["H"], c["D"]
        dt = DTYPES[c["dtype"]]
        e = torch.empty((), dtype=dt).element_size()
        lay = ua.ua2a_layout(w, B, S, H, D, e)
        moved = lay["moved_bytes"]
        rotate = rotation(lay["tensor_bytes"])
        window = torch.empty(lay["window_bytes"], dtype=torch.uint8, device=dev) if c["chunked"] else None
        plan = ua.Plan(w, B, S, H, D, dt, window=window, device=dev)
        for mode in (0, 1):
            shape = (w, B, S, H, D) if mode == 0 else (w, B, S * w, H // w, D)
            seed = c["seed0"] if mode == 0 else c["seed1"]
            x_cpu = make_tensor(shape, c["dtype"], c["dist"], seed)
            xb = x_cpu.view(BITS_VIEW[e]).numpy()
            sha = hashlib.sha256(xb.tobytes()).hexdigest()
            for chunked in ((False, True) if c["chunked"] else (False,)):
                log(f"records: {name} mode {mode} chunked={chunked}")
                xs = [x_cpu.to(dev)] + [None] * (rotate - 1)
                for k in range(1, rotate):
                    xs[k] = xs[0].clone()
                outs = [torch.empty(plan.out_shape(mode), dtype=dt, device=dev) for _ in range(rotate)]
                info = plan.describe(xs[0], mode, chunked, out=outs[0])
                t0 = time.perf_counter()
                want = oracle.exchange(xb, mode, w, chunked=chunked)
                oracle_s = time.perf_counter() - t0
                plan.exchange(xs[0], mode, chunked, out=outs[0], stream=stream)
                torch.cuda.synchronize(dev)
                exact = bool(np.array_equal(outs[0].cpu().view(BITS_VIEW[e]).numpy(), want))
                if not chunked:
                    got_n, oracle_n_s, n_threads = oracle_on_threads(xb, mode, w)
                    if not np.array_equal(got_n, want):
                        raise SystemExit(f"records: the threaded oracle differs on {name} mode {mode}")
                    del got_n
                del want

                def launch(i):
                    plan.exchange(xs[i % rotate], mode, chunked, out=outs[i % rotate], stream=stream)

                def copy(i):
                    outs[i % rotate].view(-1).view(torch.uint8).copy_(xs[i % rotate].view(-1).view(torch.uint8))

                def per_launch(fn):
                    for i in range(2 * rotate):          # warm-up, every buffer set once or twice
                        fn(i)
                    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                          for _ in range(K)]
                    torch.cuda.synchronize(dev)
                    for i, (a, b) in enumerate(ev):
                        a.record(stream)
                        fn(i)
                        b.record(stream)
                    torch.cuda.synchronize(dev)
                    return [a.elapsed_time(b) * 1e3 for a, b in ev]      # us

                def back_to_back(fn):
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    torch.cuda.synchronize(dev)
                    a.record(stream)
                    for i in range(K):
                        fn(i)
                    b.record(stream)
                    torch.cuda.synchronize(dev)
                    return a.elapsed_time(b) * 1e3 / K

                ts = per_launch(launch)
                t_avg = back_to_back(launch)
                tc = per_launch(copy)
                med = statistics.median(ts)
                rec = {
                    "record": "exchange", "workload": name, "w": w, "B": B, "S_local": S, "H": H,
                    "D": D, "dtype": c["dtype"], "mode": mode, "chunked": chunked,
                    "path": {ua.UA2A_PATH_DIRECT: "direct", ua.UA2A_PATH_LDS: "lds"}[info["path"]],
                    "bytes": moved,
                    "launches_timed": K, "buffer_sets": rotate,
                    "t_median_us": round(med, 3), "t_min_us": round(min(ts), 3),
                    "t_avg_back_to_back_us": round(t_avg, 3),
                    "GBps": round(moved / (med * 1e-6) / 1e9, 1),
                    "pct_peak": round(100 * moved / (med * 1e-6) / 1e9 / PEAK_HBM_GBPS, 2),
                    "memcpy_GBps": round(moved / (statistics.median(tc) * 1e-6) / 1e9, 1),
                    "oracle_1core_s": round(oracle_s, 4),
                    "oracle_ncore_s": None if chunked else round(oracle_n_s, 4),
                    "ncores": None if chunked else n_threads,
                    "oracle_ncore_form": None if chunked else "sender ranges on threads",
                    "host_cpus": os.cpu_count(), "cpu_model": cpu_model(),
                    "bit_exact": exact,
                    "input_sha256": sha,
                }
                if chunked:
                    rec["window_path_bytes"] = 2 * moved
                print(json.dumps(rec), flush=True)
                del xs, outs
                torch.cuda.empty_cache()
        plan.close()


# ----------------------------------------------------- counter post-processing

def _read_counter_rows(d):
    rows = []
    for p in glob.glob(os.path.join(d, "**", "*counter_collection*.csv"), recursive=True):
        with open(p, newline="") as f:
            rows += list(csv.DictReader(f))
    return rows


def _is_mode1(kernel_name: str) -> bool:
    """Whether a (demangled or mangled) direct-kernel name is the mode-1 instance:
    its second template argument, after the vector width."""
    m = re.search(r"_kernel<\d+, (true|false)", kernel_name)
    if m:
        return m.group(1) == "true"
    m = re.search(r"_kernelILi\d+ELb([01])", kernel_name)
    return bool(m) and m.group(1) == "1"


def traffic_from(d):
    """Turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs of this bench into bytes per launch.

    Each counter reads KiB per dispatch.  It is scaled by what the same counter
    reads for the runtime's device-to-device copy of a known size (the memcpy
    leg of this bench: tensor_bytes read and tensor_bytes written).
    """
    import ulysses_all_re_amd as ua
    from workloads import CONFIGS
    c = CONFIGS[WORKLOAD]
    lay = ua.ua2a_layout(c["w"], c["B"], c["S_local"], c["H"], c["D"], 2)
    rows = _read_counter_rows(d)
    if not rows:
        raise SystemExit(f"no counter_collection CSV under {d}")
    kcol = next(k for k in rows[0] if k.lower() in ("kernel_name", "kernel-name", "kernelname"))
    ncol = next(k for k in rows[0] if k.lower() in ("counter_name", "counter-name"))
    vcol = next(k for k in rows[0] if k.lower() in ("counter_value", "counter-value"))
    vals = {}
    for r in rows:
        name = r[kcol]
        key = ("mode1" if _is_mode1(name) else "mode0") if DIRECT_KERNEL in name else \
              ("copy" if COPY_KERNEL_HINT in name else None)
        if key is None:
            continue
        vals.setdefault((key, r[ncol]), []).append(float(r[vcol]))
    # the bench's copy leg moves tensor_bytes each way; other (small) runtime
    # copies in the same process are left out by keeping the largest dispatches
    for k in [k for k in vals if k[0] == "copy"]:
        top = max(vals[k])
        vals[k] = [v for v in vals[k] if v >= 0.95 * top]
    avg = {k: sum(v) / len(v) for k, v in vals.items()}
    known = lay["tensor_bytes"]
    fetch_f = avg[("copy", "FETCH_SIZE")] * 1024 / known
    write_f = avg[("copy", "WRITE_SIZE")] * 1024 / known
    out = {"library_hash": library_hash(), "workload": WORKLOAD, "counters_dir": d,
           "copy_scale": {"FETCH_SIZE": round(fetch_f, 4), "WRITE_SIZE": round(write_f, 4),
                          "known_bytes_each_way": known}}
    for m in ("mode0", "mode1"):
        fk = avg[(m, "FETCH_SIZE")] * 1024 / fetch_f
        wk = avg[(m, "WRITE_SIZE")] * 1024 / write_f
        out[f"{m}_fetch_bytes"] = round(fk)
        out[f"{m}_write_bytes"] = round(wk)
        out[f"{m}_bytes_per_launch"] = round(fk + wk)
        out[f"{m}_raw_kib"] = {"FETCH_SIZE": avg[(m, "FETCH_SIZE")], "WRITE_SIZE": avg[(m, "WRITE_SIZE")]}
    out["algorithmic_bytes_per_launch"] = lay["moved_bytes"]
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=2)
    print(json.dumps(out, indent=2))


def summarize_trace(d, workload, ranks=None, chunked=False):
    """Markdown table of a rocprofv3 --kernel-trace --stats --output-format csv run
    (with ranks == "one", each exchange launch moves one sender's share, 1/w;
    a chunked exchange is one launch, its rate on the algorithmic bytes)."""
    paths = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no kernel_stats.csv under {d}")
    import torch

    import ulysses_all_re_amd as ua
    from workloads import CONFIGS, DTYPES, MEASURE
    c = {**CONFIGS, **MEASURE}[workload]
    e = torch.empty((), dtype=DTYPES[c["dtype"]]).element_size()
    moved = ua.ua2a_layout(c["w"], c["B"], c["S_local"], c["H"], c["D"], e)["moved_bytes"]
    share = moved // c["w"] if ranks == "one" else moved
    print(f"| kernel | calls | avg us | min us | max us | GB/s at avg (2 x {share // 2} B"
          + (", one sender" if ranks == "one" else ", algorithmic" if chunked else "") + ") |")
    print("|---|---|---|---|---|---|")
    with open(paths[0], newline="") as f:
        for r in csv.DictReader(f):
            name = r["Name"]
            if len(name) > 70:
                name = name[:67] + "..."
            avg = float(r["AverageNs"])
            rate = ""
            if "ua2a_" in r["Name"]:
                rate = f"{share / (avg * 1e-9) / 1e9:.1f}"
            elif COPY_KERNEL_HINT in r["Name"] and ranks is None:   # per-rank runs also clone ranks
                rate = f"{moved / (avg * 1e-9) / 1e9:.1f}"
            print(f"| `{name}` | {r['Calls']} | {avg / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                  f"{float(r['MaxNs']) / 1e3:.2f} | {rate} |")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100,
                    help="timed steps (about 0.5 ms each on the default workload)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--blocks", type=int, default=0, help="grid-size cap (0 = library default)")
    ap.add_argument("--workload", default=WORKLOAD,
                    help="workload to time (default: the video-DiT exchange the metric is quoted on)")
    ap.add_argument("--chunked", action="store_true", help="time the chunked exchange (through a window of one batch plane)")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step as a HIP graph and time its replays")
    ap.add_argument("--ranks", choices=("all", "one"), default=None,
                    help="per-rank allocations (ua2a_exchange_ranks): one launch with every "
                         "sender, or one launch per sender (what each device of a multi-device "
                         "exchange runs)")
    ap.add_argument("--overlap", action="store_true",
                    help="time mode 0 + a per-rank consumer GEMM, serial vs pipelined on "
                         "readiness credits (its own JSON line)")
    ap.add_argument("--publish-blocks", type=int, default=8192,
                    help="--overlap: grid cap of the publishing exchange (0 = one tile per workgroup)")
    ap.add_argument("--rotate", type=int, default=0,
                    help="buffer sets to rotate through (0 = enough for about 1 GiB per cycle, "
                         "at most 64; 1 for the video-DiT tensors)")
    ap.add_argument("--path", choices=("auto", "direct", "lds"), default="auto",
                    help="force a kernel family (default: the library's choice)")
    ap.add_argument("--cpu-steps", type=int, default=12,
                    help="oracle round trips timed for cpu_baseline (about 1 s each on the "
                         "video-DiT workload, so about 12 s in all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-config", action="store_true",
                    help="leave out the per_config object (rates and oracle checks of all five workloads)")
    ap.add_argument("--records", action="store_true",
                    help="one JSON line per (workload, mode, chunked) over the five workloads: "
                         "median and min per-launch time, copy baseline, oracle time, "
                         "bit-exactness, input SHA-256")
    ap.add_argument("--pack", action="store_true",
                    help="time one sender's pack (ua2a_pack_ranks) and one receiver's unpack "
                         "(ua2a_unpack_ranks) per launch, next to the direct one-sender push")
    ap.add_argument("--sweep", action="store_true",
                    help="time the exchange at 13 sizes (4-524 MB per tensor) and fit t = t0 + bytes/BW")
    ap.add_argument("--records-workload", default=None, choices=RECORD_WORKLOADS,
                    help="--records for this workload only")
    ap.add_argument("--traffic-from", metavar="DIR", default=None,
                    help="turn rocprofv3 FETCH_SIZE/WRITE_SIZE CSVs under DIR into traffic bytes")
    ap.add_argument("--summarize-trace", metavar="DIR", default=None,
                    help="print a table of a rocprofv3 kernel-trace stats CSV under DIR")
    args = ap.parse_args()
    if args.traffic_from:
        traffic_from(args.traffic_from)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.workload, args.ranks, args.chunked)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        msg = ("this exchange runs all w virtual ranks on ONE GPU; there is no multi-GPU "
               f"configuration to measure (asked for --gpus {args.gpus}, WORLD_SIZE={world})")
        if int(os.environ.get("RANK", "0")) == 0:
            print(msg, file=sys.stderr, flush=True)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        raise SystemExit("--steps must be >= 1 and --warmup >= 0")
    if args.overlap:
        run_overlap(args)
        return
    if args.records:
        run_records(args)
        return
    if args.sweep:
        run_sweep(args)
        return
    if args.pack:
        run_pack(args)
        return
    run(args)


if __name__ == "__main__":
    main()
