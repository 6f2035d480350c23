#!/usr/bin/env python3
"""One-GPU benchmark of shared-prefix decode attention on MI355X.

A step is one pass of the whole path over one synthetic batch whose inputs
are resident in HBM: by default the decode kernel (partials) followed by the
merge kernel (bf16 output); with --fused one cap_decode_step launch (decode
kernel with the per-request merge done by the item that completes it).
Before every step (warm-up and timed) a 1 GiB read of another buffer evicts
L2 and the 256 MB Infinity Cache, so KV is read from HBM, not from cache; a
read leaves clean lines behind, so no write-back of the flush competes with
the step.  Step time is the HIP-event time around the step's kernels on the
stream they run on (no event between them); the decode kernel's own launch
time, for the roofline, comes from a separate timed loop of that kernel
alone under the same eviction.  The planner and the uploads run once,
before timing.

Prints one JSON line.  Default: the headline workload is the largest tree,
the 256-request random radix tree (depth 1-4, branching U[1,8], geometric
node lengths with mean 1024, 32 q / 8 KV heads, D=128), and `per_config`
carries the same figures for the shared system prompt, the two-level tree,
the long shared document and the radix tree's unshared control batch.
--config N times one shape only.
"""
import argparse
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from decode_attention_prefix_amd.prof_summary import kernel_hash  # noqa: E402

METRIC = "decode attn unique-KV HBM GB/s (% of peak) + request-heads/s per step, 1 GPU"
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_kernel_cfg{cfg}_traffic.txt")
TRACE_FILE = os.path.join(ROOT, "profiles", "decode_kernel_cfg{cfg}_kernel_trace.txt")


def load_traffic(cfg: int, kernel: str):
    """HBM bytes per decode launch from a committed rocprofv3 --pmc summary,
    if it was taken on the current kernel source and the same kernel; else
    None."""
    path = TRAFFIC_FILE.format(cfg=cfg)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_code_sha256_16") != kernel_hash() or kv.get("kernel") != kernel:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


COUNTERS_FILE = os.path.join(ROOT, "profiles", "decode_kernel_cfg{cfg}_counters.txt")


def load_counters(cfg, kernel: str):
    """The derived figures (MfmaUtil_pct, VALUBusy_pct, ...) of a committed
    rocprofv3 counter summary of the decode kernel, if it was taken on the
    current kernel source and the same kernel; else None."""
    path = COUNTERS_FILE.format(cfg=cfg)
    if not os.path.exists(path):
        return None
    kv, derived, section = {}, {}, None
    for line in open(path):
        if line.startswith("derived"):
            section = "derived"
            continue
        if ":" in line:
            k, v = line.split(":", 1)
            if section == "derived":
                try:
                    derived[k.strip()] = float(v)
                except ValueError:
                    pass
            else:
                kv[k.strip()] = v.strip()
    if kv.get("kernel_code_sha256_16") != kernel_hash() or kv.get("kernel") != kernel or not derived:
        return None
    keep = ("MfmaUtil_pct", "VALUBusy_pct", "LdsUtil_pct", "LDSBankConflict_pct",
            "wave_cycles_waiting_for_any_instruction_pct")
    return {k: derived[k] for k in keep if k in derived}


def load_trace_us(cfg: int, kernel: str):
    """Average duration (us) of the decode kernel in a committed rocprofv3
    --kernel-trace --stats summary, if it was taken on the current kernel
    source; else None."""
    path = TRACE_FILE.format(cfg=cfg)
    if not os.path.exists(path):
        return None
    h = None
    for line in open(path):
        if line.startswith("kernel_code_sha256_16:"):
            h = line.split(":", 1)[1].strip()
        elif line.startswith(kernel) and h == kernel_hash():
            try:
                return float(line[len(kernel):].split()[1])
            except (IndexError, ValueError):
                return None
    return None


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


def bench_rows(args, dev):
    """One JSON line for a wide-row workload: the chosen schedule's HBM rate
    on the evaluation's row count, with the two-pass schedule and torch's own
    kernel timed beside it and the fp64 oracle on a bounded sample."""
    import torch

    from decode_attention_prefix_amd import cap
    from decode_attention_prefix_amd import workloads as wl
    from decode_attention_prefix_amd.prof_summary import ROWS_SRC

    kind, W = args.rows, args.width
    x, g, b = wl.make_rows(kind, W, seed=args.seed)
    M = x.shape[0]
    xd = torch.from_numpy(x).to(dev)
    yd = torch.empty_like(xd)
    gd = torch.from_numpy(g).to(dev) if g is not None else None
    bd = torch.from_numpy(b).to(dev) if b is not None else None
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    flush = torch.empty(max(args.flush_mb, 1) << 20, dtype=torch.uint8, device=dev)
    sink = torch.empty(8192, dtype=torch.int32, device=dev)
    cap.cap_bench_fill(flush.data_ptr(), flush.numel(), 0, sp)

    def launch(mode):
        if kind == "softmax":
            cap.cap_rows_softmax(xd.data_ptr(), yd.data_ptr(), M, W, mode, sp)
        else:
            cap.cap_rows_layernorm(xd.data_ptr(), gd.data_ptr(), bd.data_ptr(), yd.data_ptr(), M, W, 1e-5,
                                   mode, sp)

    def torch_op():
        # torch's own kernel, for context only (its output is discarded)
        if kind == "softmax":
            torch.softmax(xd, dim=1)
        else:
            torch.nn.functional.layer_norm(xd, (W,), gd, bd, eps=1e-5)

    def timed(fn, steps):
        for _ in range(args.warmup):
            fn()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for e in ev:
            if args.flush_mb > 0:
                cap.cap_bench_read(flush.data_ptr(), flush.numel(), sink.data_ptr(), sp)
            e[0].record(stream)
            fn()
            e[1].record(stream)
        torch.cuda.synchronize(dev)
        return [a.elapsed_time(b_) * 1e3 for a, b_ in ev]

    # achievable read + write rate: a plain copy of as many bytes as x
    nb = M * W * 4
    cdst = torch.empty(nb, dtype=torch.uint8, device=dev)
    copy_us = timed(lambda: cap.cap_bench_copy(cdst.data_ptr(), xd.data_ptr(), nb, sp), args.steps)
    # the streaming floor: non-temporal loads and stores, in 256 KB runs per
    # workgroup and in one-row runs (the retained kernel's own shape)
    stream_us = {run: timed(lambda run=run: cap.cap_bench_copy_stream(cdst.data_ptr(), xd.data_ptr(), nb, run, sp),
                            args.steps)
                 for run in (0, W * 4 if (W * 4) % 16 == 0 else 0)}
    del cdst
    mode = args.row_mode
    us = timed(lambda: launch(mode), args.steps)
    reread_us = timed(lambda: launch(2), args.steps)
    torch_us = timed(torch_op, max(3, args.steps // 3))
    mean_us = statistics.fmean(us)
    alg = 2 * M * W * 4 + (2 * W * 4 if kind == "layernorm" else 0)
    value = alg / (mean_us * 1e-6) / 1e9
    src_hash = kernel_hash(ROWS_SRC)
    # the kernel the library runs (the rule of cap_rows.h's mode argument)
    retained = mode in (1, 3) or (mode == 0 and W <= 65536 and W % 4 == 0) or (mode == 0 and W <= 16384)
    pipelined = ((mode == 3 or (mode == 0 and kind == "layernorm" and W % 4 == 0 and 8192 <= W <= 16384
                                and M >= 1024))
                 and W <= (16384 if kind == "layernorm" or W % 4 else 32768))
    kname = ("rows_pipelined_kernel" if pipelined else "rows_retained_kernel") if retained else "rows_reread_kernel"
    traffic = None
    tpath = os.path.join(ROOT, "profiles", f"rows_{kind}_{W}_traffic.txt")
    if os.path.exists(tpath):
        kv = {}
        for line in open(tpath):
            if ":" in line:
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        if kv.get("kernel_code_sha256_16") == src_hash and kv.get("kernel", "").startswith(kname):
            traffic = float(kv["hbm_bytes_per_launch"])
    result = {
        "metric": f"row {kind} HBM GB/s (rows read + written once), 1 GPU",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(mean_us / 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{kind} over {M} rows x {W} FP32 (N(0,1) inputs)", "rows": M, "width": W,
                   "mode": {0: "auto", 1: "retained row", 2: "two passes", 3: "retained rows, pipelined"}[mode]},
        "roofline": {"bound": "hbm", "achieved": round(value, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(value / PEAK_HBM_GBS, 4), "traffic": traffic, "kernel": kname,
                     "algorithmic_bytes_per_launch": alg, "kernel_us_mean": round(mean_us, 3)},
        "t_us": {"mean": round(mean_us, 3), "median": round(statistics.median(us), 3), "min": round(min(us), 3)},
        "two_pass_us_mean": round(statistics.fmean(reread_us), 3),
        "torch_us_mean": round(statistics.fmean(torch_us), 3),
        "speedup_vs_two_pass": round(statistics.fmean(reread_us) / mean_us, 3),
        "speedup_vs_torch": round(statistics.fmean(torch_us) / mean_us, 3),
        "kernel_code_sha256_16": src_hash,
    }
    # read + write floor: copies of x's bytes, timed like the kernel (mean
    # over the timed launches; min for reference); the rows kernel's rate on
    # the same x + y bytes against the fastest copy's mean
    copies = {"cached_grid_stride": copy_us}
    copies.update({("stream_256KB_runs" if run == 0 else "stream_row_runs"): t for run, t in stream_us.items()})
    rates = {k: {"mean_gbs": round(2 * nb / (statistics.fmean(t) * 1e-6) / 1e9, 1),
                 "best_gbs": round(2 * nb / (min(t) * 1e-6) / 1e9, 1)} for k, t in copies.items()}
    best = max(rates, key=lambda k: rates[k]["mean_gbs"])
    result["copy_floor"] = {"rates": rates, "fastest": best,
                            "kernel_pct_of_fastest_mean": round(100 * (2 * nb / (mean_us * 1e-6) / 1e9)
                                                                / rates[best]["mean_gbs"], 2)}
    if not args.no_cpu_baseline:
        from oracle import rows_np
        # the whole workload, run again until about 10 s of CPU time has
        # passed (at least 2 runs, at most 20), median run time
        runs = []
        t_all = time.perf_counter()
        while len(runs) < 2 or (time.perf_counter() - t_all < 10.0 and len(runs) < 20):
            t1 = time.perf_counter()
            if kind == "softmax":
                rows_np.softmax_rows(x)
            else:
                rows_np.layernorm_rows(x, g, b)
            runs.append(time.perf_counter() - t1)
        t = statistics.median(runs)
        result["cpu_baseline"] = {"value": round(alg / t / 1e9, 4), "unit": "GB/s", "cores": 1,
                                  "kind": "oracle",
                                  "sample": f"whole workload ({M} rows), median of {len(runs)} runs, {t:.3f} s each"}
    print(json.dumps(result), flush=True)


def measure_growth(dec, tree, extra_pages, steps, args, evict, stream):
    """Decode steps on a growing tree: before each step, every request gains
    one token (cap_tree_append on the host, cap_append_kv on the GPU) and the
    plan follows (cap_plan_refresh, or a new plan when it must).  Times each
    part apart; the step itself as in the main timing (cache flushed)."""
    import numpy as np
    import torch

    from decode_attention_prefix_amd import cap
    R, Hkv, D = tree.num_requests, tree.num_kv_heads, tree.head_dim
    dev = dec.device
    first_free = int(tree.num_pool_pages) - extra_pages
    free = list(range(first_free, int(tree.num_pool_pages)))
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)
    k_new = torch.randn((R, Hkv, D), generator=gen, device=dev).to(torch.bfloat16)
    v_new = torch.randn((R, Hkv, D), generator=gen, device=dev).to(torch.bfloat16)
    sp = stream.cuda_stream
    rec = {"append_host_us": [], "refresh_host_us": [], "append_kv_us": [], "plan_update_us": [],
           "step_us": []}
    counts = {"patch": 0, "whole": 0, "replan": 0}
    words = []
    for _ in range(steps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        cand = np.asarray(free[:R], np.int32)
        t0 = time.perf_counter()
        dest = cap.cap_tree_append(dec.tree, R, None, cand)
        rec["append_host_us"].append((time.perf_counter() - t0) * 1e6)
        taken = set((dest[(dest >= 0) & ((dest & 15) == 0)] >> 4).tolist())
        free = [p for p in free if p not in taken]
        d = torch.from_numpy(dest).to(dev)
        ev[0].record(stream)
        cap.cap_append_kv(dec.tree, d.data_ptr(), R, k_new.data_ptr(), v_new.data_ptr(), dec.k.data_ptr(),
                          dec.v.data_ptr(), sp)
        ev[1].record(stream)
        before = dec.stats["refreshes"]
        try:
            cap.cap_plan_refresh(dec.plan_h, sp)
            st = cap.cap_plan_get_stats(dec.plan_h)
            if st["refreshes"] > before:
                counts["whole" if st["refresh_full_copy"] else "patch"] += 1
                rec["refresh_host_us"].append(st["refresh_host_us"])
                words.append(st["refresh_words"])
            dec.stats = st
        except cap.CapError as e:
            if e.status != cap.CAP_ERR_REPLAN:
                raise
            dec.plan(**dec.plan_opts)
            counts["replan"] += 1
        ev[2].record(stream)
        if args.flush_mb > 0:
            evict()
        ev[3].record(stream)
        if args.fused:
            dec.fused_step()
        else:
            dec.decode()
            dec.merge()
        ev[4].record(stream)
        torch.cuda.synchronize(dev)
        rec["append_kv_us"].append(ev[0].elapsed_time(ev[1]) * 1e3)
        rec["plan_update_us"].append(ev[1].elapsed_time(ev[2]) * 1e3)
        rec["step_us"].append(ev[3].elapsed_time(ev[4]) * 1e3)
    med = {k: (round(statistics.median(v), 2) if v else None) for k, v in rec.items()}
    return {"steps": steps, "tokens_per_step": R, **{k + "_median": v for k, v in med.items()},
            "refresh_words_median": (statistics.median(words) if words else None),
            "plan_updates": counts,
            "note": "plan_update_us: stream time from the end of the K/V write to the end of the plan "
                    "update (its host work included while the stream waits on it)"}


def workload_for(cfg: int, control: bool, args, extra_pages: int = 0):
    """Seeded synthetic inputs of one tree shape (zero pool tails: the timed
    runs need no NaN poison), or its unshared control batch."""
    from decode_attention_prefix_amd import workloads as wl
    w = wl.make_config(cfg, seed=args.seed, tail_fill="zero", keep_tokens=control,
                       extra_pool_pages=extra_pages, permute_pages=not args.contiguous,
                       heads_divisor=args.tp_share)
    if control:
        w = wl.control_workload(w, tail_fill="zero")
    return w


def plan_opts(args) -> dict:
    opts = {"share_mode": args.share, "split_pages": args.split_pages}
    for k in ("shared_rows", "rounds", "order", "shared_cost", "share_margin"):
        if getattr(args, k):
            opts[k] = getattr(args, k)
    if args.dispatch:
        opts["item_dispatch"] = args.dispatch
    return opts


def plan_host_times(dec, opts, reps: int = 20) -> dict:
    """Host time of planning the tree again (medians over `reps`): a fresh
    cap_plan_step, and cap_plan_rebuild into an existing plan handle (its
    host memory reused, as a serving loop that plans every step would)."""
    from decode_attention_prefix_amd import cap
    fresh, rebuild = [], []
    p = cap.cap_plan_step(dec.tree, **opts)
    try:
        for _ in range(reps):
            q = cap.cap_plan_step(dec.tree, **opts)
            fresh.append(cap.cap_plan_get_stats(q)["plan_host_us"])
            cap.cap_plan_free(q)
            cap.cap_plan_rebuild(p, dec.tree, **opts)
            rebuild.append(cap.cap_plan_get_stats(p)["plan_host_us"])
    finally:
        cap.cap_plan_free(p)
    return {"plan_step_us": round(statistics.median(fresh), 1),
            "plan_rebuild_us": round(statistics.median(rebuild), 1)}


def measure(w, cfg: int, control: bool, args, dev, evict, stream, profiled: bool):
    """Time one workload: the whole step (decode + merge, or the fused
    launch) with HIP events around it, the decode kernel alone by events
    bound to its dispatch, the merge alone, and a plain read of the decode
    launch's bytes; caches evicted before each launch.  Returns (dict,
    decoder); the caller closes the decoder."""
    import torch

    from decode_attention_prefix_amd import cap
    from decode_attention_prefix_amd import workloads as wl
    from decode_attention_prefix_amd.decoder import TreeDecoder

    opts = plan_opts(args)
    st_tree = wl.tree_stats(w.tree)
    dec = TreeDecoder(w.tree, w.q, w.k_pool, w.v_pool, device=dev, **opts)
    plan = dec.stats
    sp = stream.cuda_stream
    uniq = st_tree["unique_kv_bytes"]
    fused = args.fused
    # the fused launch also writes the bf16 output
    alg_bytes_decode = uniq + st_tree["q_bytes"] + (st_tree["out_bytes"] if fused else 0)

    # a plain read of exactly the decode launch's algorithmic bytes, timed
    # like that launch (caches evicted, events around the one launch): what a
    # kernel that does nothing but stream those bytes reaches at this size,
    # launch latency, ramp-up and drain included
    sm_bytes = (alg_bytes_decode + 15) // 16 * 16
    probe = torch.empty(sm_bytes, dtype=torch.uint8, device=dev)
    sink = torch.empty(8192, dtype=torch.int32, device=dev)
    cap.cap_bench_fill(probe.data_ptr(), sm_bytes, 0x3F803F80, sp)
    sm_ms = []
    for _ in range(max(args.steps, 5)):
        evict()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        cap.cap_bench_read_stream(probe.data_ptr(), sm_bytes, sink.data_ptr(), sp)
        b.record(stream)
        b.synchronize()
        sm_ms.append(a.elapsed_time(b))
    sm_mean = statistics.fmean(sm_ms)
    del probe

    graph = dec.capture_step(fused=args.fused) if args.graph else None

    def one_step(evs=None):
        # events only around the whole step: an event recorded between the two
        # kernels would itself add a few microseconds of queue overhead
        if args.flush_mb > 0:
            evict()
        if evs is not None:
            evs[0].record(stream)
        if graph is not None:
            graph.replay()
        elif fused:
            dec.fused_step()
        else:
            dec.decode()
            dec.merge()
        if evs is not None:
            evs[1].record(stream)

    for _ in range(args.warmup):
        one_step()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for k in range(args.steps):
        one_step(events[k])
    torch.cuda.synchronize(dev)
    wall_s = time.perf_counter() - t0
    step_ms = [e[0].elapsed_time(e[1]) for e in events]
    mean_ms = statistics.fmean(step_ms)
    med_ms = statistics.median(step_ms)
    srt = sorted(step_ms)
    p90_ms = srt[min(len(srt) - 1, int(round(0.9 * (len(srt) - 1))))]

    # the dominant kernel alone, same inputs and cache state, for the roofline:
    # HIP events on the stream it runs on, around each launch
    kev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for k in range(args.steps):
        if args.flush_mb > 0:
            evict()
        kev[k][0].record(stream)
        if fused:
            dec.fused_step()
        else:
            dec.decode()
        kev[k][1].record(stream)
    torch.cuda.synchronize(dev)
    dec_ms = [e[0].elapsed_time(e[1]) for e in kev]
    # the same launches timed by HIP events bound to the kernel's own dispatch
    # (hipExtLaunchKernel): the kernel's execution alone, without the queueing
    # that the events recorded around the launch above include -- what the
    # rocprofv3 kernel trace reports, and what the roofline is taken on
    disp_ms = None
    if not fused:
        disp_ms = []
        for k in range(args.steps):
            if args.flush_mb > 0:
                evict()
            disp_ms.append(dec.decode_timed() * 1e-3)
    mrg_ms = None
    if not fused:
        mev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for k in range(args.steps):
            if args.flush_mb > 0:
                evict()
            dec.decode()
            mev[k][0].record(stream)
            dec.merge()
            mev[k][1].record(stream)
        torch.cuda.synchronize(dev)
        mrg_ms = [e[0].elapsed_time(e[1]) for e in mev]

    value = uniq / (mean_ms * 1e-3) / 1e9
    dec_ev_mean = statistics.fmean(dec_ms)                 # events around the launch
    dec_mean = statistics.fmean(disp_ms) if disp_ms else dec_ev_mean
    achieved = alg_bytes_decode / (dec_mean * 1e-3) / 1e9
    kernel_name = f"decode_kernel<{w.tree.head_dim}, {'true' if fused else 'false'}>"
    # committed profiles hold for the default plan of the same workload only
    pkey = "4c" if control and cfg == 4 else cfg
    traffic = load_traffic(pkey, kernel_name) if profiled else None
    trace_us = load_trace_us(pkey, kernel_name) if profiled else None
    counters = load_counters(pkey, kernel_name) if profiled else None
    r = {
        "value": round(value, 2),
        "ms_per_step": round(mean_ms, 5),
        "config": {
            "workload": ("control batch of " if control else "") + f"config {cfg}: " + wl.CONFIG_NAMES[cfg],
            "requests": w.tree.num_requests, "q_heads": w.tree.num_q_heads,
            "kv_heads": w.tree.num_kv_heads, "head_dim": w.tree.head_dim, "page_size": 16,
            "seed": args.seed, "nodes": w.tree.num_nodes,
            "pages": "tree order" if args.contiguous else "seeded permutation of the pool",
            **({"heads_share": f"1/{args.tp_share} of the heads (one GPU of a {args.tp_share}-way KV-head split)"}
               if args.tp_share != 1 else {}),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "kernel": kernel_name,
            "algorithmic_bytes_per_launch": alg_bytes_decode,
            "decode_us_mean": round(dec_mean * 1e3, 3),
            "timing": ("HIP events bound to the decode kernel's dispatch (hipExtLaunchKernel), mean over "
                       "the timed launches" if disp_ms else "HIP events on the stream around each launch"),
            "decode_us_events_around_launch": round(dec_ev_mean * 1e3, 3),
            # the same kernel's average in the committed rocprofv3 kernel trace
            # (start to end of the kernel, without the dispatch latency that
            # the events above include), and the fraction it gives
            "trace_avg_us": trace_us,
            "frac_by_trace": (round(alg_bytes_decode / (trace_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
                              if trace_us else None),
        },
        "pct_peak_hbm": round(100 * value / PEAK_HBM_GBS, 2),
        "req_heads_per_s": round(st_tree["request_heads"] / (mean_ms * 1e-3), 1),
        # useful FLOP of the step / its time / the bf16 dense peak
        "mfma_util": round(st_tree["useful_flop"] / (mean_ms * 1e-3) / 2.5e15, 5),
        # the decode kernel's matrix-core busy share and its other SQ figures,
        # from the committed rocprofv3 counter summary (rocprofv3's formulas)
        "counters": ({**counters, "source": os.path.relpath(COUNTERS_FILE.format(cfg=pkey), ROOT)}
                     if counters else None),
        "t_decode_us": {"mean": round(dec_mean * 1e3, 3),
                        "median": round(statistics.median(disp_ms or dec_ms) * 1e3, 3),
                        "events_around_launch_mean": round(dec_ev_mean * 1e3, 3)},
        "step_form": ("fused cap_decode_step" if fused else "cap_decode_attention + cap_merge_partials")
                     + (", replayed from a HIP graph" if args.graph else ""),
        "t_merge_us": ({"mean": round(statistics.fmean(mrg_ms) * 1e3, 3),
                        "median": round(statistics.median(mrg_ms) * 1e3, 3)} if mrg_ms else None),
        "t_step_us": {"mean": round(mean_ms * 1e3, 3), "median": round(med_ms * 1e3, 3),
                      "min": round(srt[0] * 1e3, 3), "p90": round(p90_ms * 1e3, 3)},
        "value_median_step": round(uniq / (med_ms * 1e-3) / 1e9, 2),
        "wall_ms_per_step_incl_flush": round(wall_s * 1e3 / args.steps, 4),
        "size_matched_read": {"bytes": sm_bytes, "us_mean": round(sm_mean * 1e3, 3),
                              "gbs": round(sm_bytes / (sm_mean * 1e-3) / 1e9, 1),
                              # both timed by events on the stream around the launch
                              "decode_over_read": round(dec_ev_mean / sm_mean, 4)},
        "bytes": {"unique_kv": uniq, "unshared_kv": st_tree["unshared_kv_bytes"],
                  "kv_streamed_by_items": plan["kv_bytes_streamed"],
                  "partial": plan["partial_bytes"], "q": st_tree["q_bytes"], "out": st_tree["out_bytes"]},
        "plan": {k: plan[k] for k in ("num_items", "num_shared_items", "num_tasks", "num_groups", "partial_rows",
                                      "max_partials_per_request", "max_pages_per_item")},
        "plan_host_us": plan_host_times(dec, opts),
    }
    return r, dec


def summary(r: dict) -> dict:
    """The figures of one workload kept in the per_config object."""
    return {
        "workload": r["config"]["workload"],
        "step_us": r["t_step_us"]["mean"], "step_us_median": r["t_step_us"]["median"],
        "unique_kv_gbs": r["value"], "pct_peak_hbm": r["pct_peak_hbm"],
        "req_heads_per_s": r["req_heads_per_s"],
        "decode_us": r["t_decode_us"]["mean"], "decode_frac": r["roofline"]["frac"],
        "decode_frac_by_trace": r["roofline"]["frac_by_trace"], "traffic": r["roofline"]["traffic"],
        "merge_us": r["t_merge_us"]["mean"] if r["t_merge_us"] else None,
        "decode_over_size_matched_read": r["size_matched_read"]["decode_over_read"],
        "bytes_unique_kv": r["bytes"]["unique_kv"], "bytes_partial": r["bytes"]["partial"],
        "plan_host_us": r["plan_host_us"],
        "counters": r["counters"],
    }


def cpu_baseline(w):
    """The C oracle on the whole workload, on this host's cores: median over
    repeated runs for about 10 s, and one run on one core."""
    import oracle
    from decode_attention_prefix_amd import workloads as wl
    uniq = wl.tree_stats(w.tree)["unique_kv_bytes"]
    ncores = len(os.sched_getaffinity(0))
    # bounded sample: the whole workload, run again until about 10 s of
    # CPU time has passed (at least 3 runs, at most 50), median run time
    runs = []
    t_all = time.perf_counter()
    while len(runs) < 3 or (time.perf_counter() - t_all < 10.0 and len(runs) < 50):
        t1 = time.perf_counter()
        oracle.decode(w.tree, w.q, w.k_pool, w.v_pool, nthreads=ncores)
        runs.append(time.perf_counter() - t1)
    t_or = statistics.median(runs)
    cores = oracle.threads()
    t1 = time.perf_counter()
    oracle.decode(w.tree, w.q, w.k_pool, w.v_pool, nthreads=1)
    t_one = time.perf_counter() - t1
    return {
        "value": round(uniq / t_or / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"whole workload ({w.tree.num_requests} requests), median of {len(runs)} runs, "
                  f"{t_or:.3f} s each",
        "cpu": cpu_model(),
        "one_core": {"value": round(uniq / t_one / 1e9, 4), "unit": "GB/s", "sample": f"one run, {t_one:.3f} s"},
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=15)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=None, choices=[0, 1, 2, 3, 4],
                    help="time this one tree shape (default: the random radix tree as the headline, with the "
                         "other shapes in per_config)")
    ap.add_argument("--per-config", default="1,2,3,4c",
                    help="with no --config: shapes timed after the headline and reported in per_config "
                         "(4c = the random radix tree's control batch; empty = none)")
    ap.add_argument("--control", action="store_true", help="time the unshared control batch of the config")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--flush-mb", type=int, default=1024)
    ap.add_argument("--share", type=int, default=-1, help="-1 auto, 0 fold all, 1 share all")
    ap.add_argument("--split-pages", type=int, default=0)
    ap.add_argument("--shared-rows", type=int, default=0,
                    help="groups with more query rows than this use shared workgroups (0: 16)")
    ap.add_argument("--rounds", type=float, default=0.0)
    ap.add_argument("--order", type=int, default=0, help="work-item order (planner option)")
    ap.add_argument("--shared-cost", type=float, default=0.0)
    ap.add_argument("--share-margin", type=float, default=0.0, help="planner option (0 = default)")
    ap.add_argument("--dispatch", type=int, default=0, choices=[0, 1],
                    help="0 one workgroup per item (default), 1 work queues (planner option item_dispatch)")
    ap.add_argument("--fused", action="store_true",
                    help="time the one-launch cap_decode_step instead of cap_decode_attention + "
                         "cap_merge_partials")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="replay the step from a HIP graph (captured once) instead of launching it")
    ap.add_argument("--read-probe-mb", type=int, default=2048)
    ap.add_argument("--tp-share", type=int, default=1,
                    help="keep 1/N of the query and KV heads (same tree): one GPU's share of an "
                         "N-way split by KV head")
    ap.add_argument("--contiguous", action="store_true",
                    help="physical pages in tree order instead of a seeded permutation of the pool")
    ap.add_argument("--growth-steps", type=int, default=16,
                    help="after the timed steps: decode steps that first grow the tree by one token "
                         "per request (host append, K/V write, plan refresh), timed apart (0 = none)")
    ap.add_argument("--rows", choices=["softmax", "layernorm"], default=None,
                    help="time a wide-row reduction-reuse workload instead of decode attention")
    ap.add_argument("--width", type=int, default=65536, help="row width for --rows")
    ap.add_argument("--row-mode", type=int, default=0, choices=[0, 1, 2, 3],
                    help="0 auto, 1 retained row, 2 two passes, 3 retained rows pipelined (for --rows)")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="also run one plain copy of this size (calibrates HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): this build has no "
              "multi-GPU path; the per-GPU share of a sharded run is the one-GPU workload.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from decode_attention_prefix_amd import cap

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.rows:
        bench_rows(args, dev)
        return

    suite = args.config is None
    cfg = 4 if suite else args.config
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    sink = torch.empty(8192, dtype=torch.int32, device=dev)
    flush = torch.empty(max(args.flush_mb, 1) << 20, dtype=torch.uint8, device=dev)
    cap.cap_bench_fill(flush.data_ptr(), flush.numel(), 0, sp)

    def evict():
        cap.cap_bench_read(flush.data_ptr(), flush.numel(), sink.data_ptr(), sp)

    # achievable HBM read rate (plain streaming read of a buffer >> caches)
    probe_bytes = args.read_probe_mb << 20
    probe = torch.empty(probe_bytes, dtype=torch.uint8, device=dev)
    cap.cap_bench_fill(probe.data_ptr(), probe_bytes, 0x3F803F80, sp)
    read_ms = []
    for _ in range(5):
        evict()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        cap.cap_bench_read_stream(probe.data_ptr(), probe_bytes, sink.data_ptr(), sp)
        b.record(stream)
        b.synchronize()
        read_ms.append(a.elapsed_time(b))
    read_gbs = probe_bytes / (min(read_ms) * 1e-3) / 1e9
    del probe

    # the committed profiles were taken with the default plan of each workload
    profiled = (args.tp_share == 1 and not args.contiguous and args.seed == 0 and args.share == -1
                and not args.split_pages and not args.shared_rows and not args.rounds and not args.order
                and not args.shared_cost and not args.share_margin and not args.dispatch and not args.fused
                and not args.graph)
    t_gen = time.perf_counter()
    growth = args.growth_steps if not args.control else 0
    R_cfg = {0: 4, 1: 64, 2: 128, 3: 32, 4: 256}[cfg]
    extra_pages = R_cfg * (growth // 16 + 3) if growth else 0
    w = workload_for(cfg, args.control, args, extra_pages)
    t_gen = time.perf_counter() - t_gen
    r, dec = measure(w, cfg, args.control, args, dev, evict, stream, profiled)
    result = {
        "metric": METRIC,
        "value": r["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        **{k: v for k, v in r.items() if k not in ("value", "ms_per_step")},
        "read_roofline_gbs": round(read_gbs, 1),
        "pct_measured_read_roofline": round(100 * r["value"] / read_gbs, 2),
        "flush_mb": args.flush_mb,
        "gen_s": round(t_gen, 2),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w)
    if growth:
        result["growth"] = measure_growth(dec, w.tree, extra_pages, growth, args, evict, stream)
    dec.close()
    del dec
    if args.copy_probe_mb > 0:
        nb = args.copy_probe_mb << 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty(nb, dtype=torch.uint8, device=dev)
        cap.cap_bench_fill(src.data_ptr(), nb, 1, sp)
        evict()
        cap.cap_bench_copy(dst.data_ptr(), src.data_ptr(), nb, sp)
        torch.cuda.synchronize(dev)
        result["copy_probe_bytes"] = nb
        del src, dst

    if suite and args.per_config.strip():
        per = {}
        for key in [k.strip() for k in args.per_config.split(",") if k.strip()]:
            control = key.endswith("c")
            c = int(key.rstrip("c"))
            if c == cfg and control:
                # the headline's control batch: the same requests, unshared
                wc = workload_for(c, True, args)
            else:
                wc = workload_for(c, control, args)
            rc, dc = measure(wc, c, control, args, dev, evict, stream, profiled)
            dc.close()
            del dc, wc
            torch.cuda.empty_cache()
            per[key] = summary(rc)
        if "4c" in per and cfg == 4:
            per["4c"]["sharing_speedup"] = round(per["4c"]["step_us"] / r["t_step_us"]["mean"], 3)
        result["per_config"] = per
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
