"""Benchmark of the ring all-reduce hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

A step is one ring all-reduce (R-1 reduce-scatter hops, then R-1 all-gather
hops, over S slices) of the data-parallel gradient bucket: 8 virtual ranks x
25 Mi bf16 elements (50 MiB per rank), values normal(0, 1e-3), fp32 adds with
per-hop bf16 rounding.  Inputs are resident in HBM before the timed region.

Printed: one JSON line with
  value       bus bandwidth (nccl-tests convention: (b*N/t) * 2(R-1)/R), GB/s
  hbm         algorithmic HBM bytes of the ring (reduce 3b, copy 2b per
              element per hop) / time, and the fraction of 8 TB/s
  roofline    the reduce kernel alone: algorithmic bytes per launch / mean
              launch duration, measured with HIP events on its own stream
  gemm        slowdown of a concurrent 8192^3 bf16 GEMM while all-reduces run
              on a second stream, with kernel copies vs SDMA copies
  cpu_baseline the CPU oracle on the same workload (1 thread)
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

HBM_PEAK_GBS = 8000.0
METRIC = "all-reduce busBW GB/s and % HBM peak on 1 MI355X; concurrent-GEMM slowdown %"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(a):
    import numpy as np
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def ring_bytes(R, count, esize, fused=True):
    """Algorithmic HBM bytes of one ring all-reduce on one GPU: a reduce hop
    reads two operands and writes one (3b per element), a copy hop reads one
    and writes one (2b).  With the last reduce-scatter hop forwarding its
    result (fused), that hop writes twice and all-gather has R-2 hops."""
    if fused:
        return esize * count * (3 * (R - 1) + 1 + 2 * (R - 2))
    return esize * count * 5 * (R - 1)


def time_steps(fn, steps, stream=None):
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


_OWN_QUEUES = []


def own_queue_stream(i):
    """The i-th torch stream with a hardware queue of its own.  Plain streams
    share the runtime's few hardware queues round-robin, so unrelated streams
    can end up serialised in one in-order queue; a CU-masked stream (mask:
    all CUs) is given its own queue.  The streams are created once and
    reused: every extra hardware queue counts, and with some twenty of them
    the hardware scheduler time-slices queues and a GEMM alone runs 1.65x
    slower on MI355X."""
    while len(_OWN_QUEUES) <= i:
        _OWN_QUEUES.append(_new_own_queue_stream())
    return _OWN_QUEUES[i]


def _new_own_queue_stream():
    import ctypes
    import torch
    hip = ctypes.CDLL("libamdhip64.so")  # the runtime torch already loaded
    hip.hipExtStreamCreateWithCUMask.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint32,
                                                 ctypes.POINTER(ctypes.c_uint32)]
    n = torch.cuda.get_device_properties(0).multi_processor_count
    words = (n + 31) // 32
    mask = (ctypes.c_uint32 * words)(*([0xFFFFFFFF] * words))
    s = ctypes.c_void_p()
    if hip.hipExtStreamCreateWithCUMask(ctypes.byref(s), words, mask) != 0:
        raise RuntimeError("hipExtStreamCreateWithCUMask failed")
    return torch.cuda.ExternalStream(s.value)


def contention_rate(intervals, window_ms, n_cu):
    """HOCCL Eq. 1 over one window [0, window_ms] in which compute is active
    throughout: the integral of the compute units held by communication
    kernels, over n_cu times the window.  intervals: (start, end, cus) per
    kernel in ms from the window's start; at any moment the kernels running
    hold the sum of their cus, at most n_cu.  Computed by sweeping the
    interval ends."""
    edges = sorted([(max(0.0, s), cu) for s, e, cu in intervals if e > 0 and s < window_ms] +
                   [(min(window_ms, e), -cu) for s, e, cu in intervals if e > 0 and s < window_ms])
    held, level, last = 0.0, 0.0, 0.0
    for t, d in edges:
        held += min(n_cu, level) * (t - last)
        level += d
        last = t
    return held / (n_cu * window_ms)


PAIRS = 15  # interleaved GEMM-alone / loaded window pairs per overlap configuration


def ci95(xs):
    """(mean, lower, upper) of the two-sided 95% t-interval of the mean."""
    a = np.asarray(xs, dtype=np.float64)
    n = a.size
    m = float(a.mean()) if n else float("nan")
    if n < 2:
        return m, m, m
    try:
        from scipy.stats import t as student_t
        q = float(student_t.ppf(0.975, n - 1))
    except ImportError:  # normal approximation
        q = 1.96
    h = q * float(a.std(ddof=1)) / np.sqrt(n)
    return m, m - h, m + h


def diff_ci95(a, b):
    """(mean, lower, upper) of mean(a) - mean(b), Welch's 95% interval."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    d = float(a.mean() - b.mean())
    va, vb = a.var(ddof=1) / a.size, b.var(ddof=1) / b.size
    se = float(np.sqrt(va + vb))
    if se == 0.0:
        return d, d, d
    df = (va + vb) ** 2 / (va ** 2 / (a.size - 1) + vb ** 2 / (b.size - 1))
    try:
        from scipy.stats import t as student_t
        q = float(student_t.ppf(0.975, df))
    except ImportError:
        q = 1.96
    return d, d - q * se, d + q * se


def run_label(r):
    """Short name of an overlap run: copy mode, CU budget, SDMA engines."""
    if r["copy_mode"] == "kernel":
        return f"kernel/B{r['cu_budget']}"
    tail = "deadline" if "dma_deadline" in r else (f"E{r['dma_engines']}" if r["dma_engines"] != "all" else "Eall")
    if r.get("dma_sync") == "stream_flags":
        tail += "/flags"
    return f"sdma/B{r['cu_budget']}/{tail}"


def pareto(points):
    """Labels of the points no other point beats on both axes (collective
    time under load, GEMM slowdown: lower is better on each), by time."""
    out = []
    for lab, t, sd in points:
        if not any((t2 <= t and s2 <= sd) and (t2 < t or s2 < sd) for _, t2, s2 in points):
            out.append((t, lab))
    return [lab for _, lab in sorted(out)]


def sdma_verdict(runs):
    """Kernel copies against SDMA copies under a concurrent GEMM, from the
    per-pair slowdowns of each overlap run (host-function gates only):
    - equal budget: at each CU budget B both modes were run at, SDMA on all
      engines minus kernel copies, with Welch's 95% interval;
    - matched time: each SDMA run against the kernel run whose collectives
      took the nearest time under load;
    - the Pareto set over (collective time under load, GEMM slowdown)."""
    rs = [r for r in runs if r.get("dma_sync") in (None, "host_func")]
    kern = {r["cu_budget"]: r for r in rs if r["copy_mode"] == "kernel"}
    sdma_all = {r["cu_budget"]: r for r in rs if r["copy_mode"] == "sdma" and r["dma_engines"] == "all"
                and "dma_deadline" not in r}
    equal = []
    for B in sorted(set(kern) & set(sdma_all), reverse=True):
        d, lo, hi = diff_ci95(sdma_all[B]["pairs_pct"], kern[B]["pairs_pct"])
        equal.append({"cu_budget": B, "kernel_pct": round(kern[B]["slowdown_mean_pct"], 2),
                      "sdma_pct": round(sdma_all[B]["slowdown_mean_pct"], 2),
                      "sdma_minus_kernel_pp": [round(d, 2), round(lo, 2), round(hi, 2)],
                      "sdma_lower": bool(hi < 0), "sdma_higher": bool(lo > 0)})
    matched = []
    for r in rs:
        if r["copy_mode"] != "sdma" or r["cu_budget"] != 256:
            continue
        k = min(kern.values(), key=lambda x: abs(x["collectives_under_load_ms"] - r["collectives_under_load_ms"]))
        d, lo, hi = diff_ci95(r["pairs_pct"], k["pairs_pct"])
        matched.append({"sdma": run_label(r), "kernel": run_label(k),
                        "coll_ms": [round(r["collectives_under_load_ms"], 2),
                                    round(k["collectives_under_load_ms"], 2)],
                        "slowdown_pct": [round(r["slowdown_mean_pct"], 2), round(k["slowdown_mean_pct"], 2)],
                        "sdma_minus_kernel_pp": [round(d, 2), round(lo, 2), round(hi, 2)],
                        "sdma_lower": bool(hi < 0)})
    front = pareto([(run_label(r), r["collectives_under_load_ms"], r["slowdown_mean_pct"]) for r in rs])
    full = next((e for e in equal if e["cu_budget"] == 256), None)
    return {"equal_budget": equal, "matched_time": matched, "pareto": front,
            "target_sdma_lower_at_full_cus": None if full is None else full["sdma_lower"],
            "sdma_lower_at_some_matched_time": any(m["sdma_lower"] for m in matched),
            "sdma_on_pareto": [lab for lab in front if lab.startswith("sdma")]}


def overlap_runs(ccr, collective, runs, gemm_dims, n_gemm, n_coll):
    """Fixed-work overlap protocol.  G back-to-back GEMMs on stream g, alone
    and then with n_coll calls of `collective(ctx, stream)` issued on
    stream c over the same window.  Both streams get hardware queues of their
    own and are released together by an event after a short GPU sleep, so
    the host has enqueued everything before either starts; every mode does
    the same communication work.  Reported per run: the GEMMs' slowdown,
    the time the collectives took under load, and the makespan (time until
    both the GEMMs and the collectives are done) against the GEMMs alone."""
    import torch
    M, N, K = gemm_dims
    A = torch.randn(M, K, dtype=torch.bfloat16, device="cuda")
    B = torch.randn(K, N, dtype=torch.bfloat16, device="cuda")
    C = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    g, c, s0 = own_queue_stream(0), own_queue_stream(1), own_queue_stream(2)

    def gemms():
        for _ in range(n_gemm):
            torch.matmul(A, B, out=C)

    def window(ctx=None, events=False):
        torch.cuda.synchronize()
        go = torch.cuda.Event()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        with torch.cuda.stream(s0):
            torch.cuda._sleep(20_000_000)
            go.record(s0)
        g.wait_event(go)
        c.wait_event(go)
        with torch.cuda.stream(g):
            ev[0].record(g)
            gemms()
            ev[1].record(g)
        if ctx is not None:
            with torch.cuda.stream(c):
                ev[2].record(c)
                for _ in range(n_coll):
                    collective(ctx, c)
                ev[3].record(c)
        torch.cuda.synchronize()
        gemm = ev[0].elapsed_time(ev[1])
        if ctx is None:
            return gemm, 0.0, gemm
        coll = ev[2].elapsed_time(ev[3])
        span = max(ev[0].elapsed_time(ev[1]), ev[0].elapsed_time(ev[3]))
        return (gemm, coll, span, ev) if events else (gemm, coll, span)

    n_cu = torch.cuda.get_device_properties(0).multi_processor_count

    def contention(ctx):
        """HOCCL Eq. 1 for the collective: the integral over the GEMMs' active
        time of the compute units its kernels hold, over n_cu times that
        time.  One more window, with every collective kernel bracketed by
        events attached to its launch; the GEMMs run back to back, so
        compute is active from the first GEMM's start to the last one's end."""
        ccr.ccr_profile_enable(ctx, True)
        gemm, _, _, ev = window(ctx, events=True)
        iv = np.concatenate([ccr.ccr_profile_intervals(ctx, k, ev[0])
                             for k in ("reduce", "copy_kernel", "reduce_forward")])
        ccr.ccr_profile_enable(ctx, False)
        return contention_rate(iv, gemm, n_cu)

    with torch.cuda.stream(g):
        gemms()
    window()
    alone = sorted(window()[0] for _ in range(3))[1]
    out = {"gemm": f"{M}x{N}x{K} bf16 x{n_gemm}", "gemm_alone_ms": round(alone, 3),
           "collectives_per_window": n_coll, "runs": []}
    for conf in runs:
        if conf.get("dma_deadline_us") == "window":
            # each collective may take its share of the GEMMs' window alone
            conf = dict(conf, dma_deadline_us=int(alone * 1e3 / n_coll))
        with ccr.Context(0, ccr.Config(**conf)) as ctx:
            collective(ctx, c)  # first use starts the SDMA proxy
            torch.cuda.synchronize()
            t1 = time_steps(lambda: collective(ctx, c), 3)
            # A/B interleaved: GEMM alone, then with the collectives, nine times;
            # each run is compared with its own alone windows, so slow drift of
            # the GEMM's own time (clocks, temperature) does not count as slowdown
            a_ms, b_runs = [], []
            for _ in range(PAIRS):
                a_ms.append(window()[0])
                b_runs.append(window(ctx))
            alone_i = sorted(a_ms)[PAIRS // 2]
            gemm, coll, span = sorted(b_runs)[PAIRS // 2]
            # paired slowdowns: each loaded window against the alone window just before it
            pairs_pct = [100.0 * (b[0] / a - 1.0) for a, b in zip(a_ms, b_runs)]
            mean, lo, hi = ci95(pairs_pct)
            coll_ms = sorted(b[1] for b in b_runs)[PAIRS // 2]
            i_coll = contention(ctx)
            paced = None
            if conf["copy_mode"] == "sdma" and conf.get("dma_deadline_us"):
                gbs, used = ccr.ccr_dma_rate(ctx)
                paced = {"deadline_us": conf["dma_deadline_us"], "engine_gbs": round(gbs, 1),
                         "engines_used": used}
            run = {
                "copy_mode": conf["copy_mode"], "cu_budget": conf.get("cu_budget", 0) or 256,
                "dma_sync": conf.get("dma_sync", "host_func") if conf["copy_mode"] == "sdma" else None,
                "dma_engines": (conf.get("dma_engines", 0) or "all") if conf["copy_mode"] == "sdma" else None,
                "gemm_alone_ms": round(alone_i, 3),
                "gemm_ms": round(gemm, 3), "slowdown_pct": round(100.0 * (gemm / alone_i - 1.0), 2),
                "slowdown_mean_pct": round(mean, 3), "slowdown_ci95_pct": [round(lo, 3), round(hi, 3)],
                "pairs_pct": [round(x, 3) for x in pairs_pct],
                "slowdown_pct_spread": [round(min(pairs_pct), 2), round(max(pairs_pct), 2)],
                "collective_alone_ms": round(t1 * 1e3, 4),
                "collectives_under_load_ms": round(coll_ms, 3),
                "makespan_ms": round(span, 3),
                "makespan_over_gemm_alone_pct": round(100.0 * (span / alone_i - 1.0), 2),
                "contention_rate": round(i_coll, 4),
                **({"dma_deadline": paced} if paced else {})}
            run["label"] = run_label(run)
            log(f"  {run['label']}: slowdown {mean:.2f}% [{lo:.2f}, {hi:.2f}], "
                f"collectives {coll_ms:.2f} ms under load")
            out["runs"].append(run)
    out["verdict"] = sdma_verdict(out["runs"])
    return out


def compact_verdict(o):
    """A few hundred characters of an overlap run's verdict: kernel against
    SDMA at full CUs (GEMM slowdown %, mean over the pairs, and the SDMA
    minus kernel difference with its 95% interval), each SDMA run against
    the kernel run of the nearest collective time under load, and the
    Pareto set."""
    v = o["verdict"]
    full = next((e for e in v["equal_budget"] if e["cu_budget"] == 256), None)
    return {"pairs": PAIRS,
            "full_cus": None if full is None else
            {"kernel_pct": full["kernel_pct"], "sdma_pct": full["sdma_pct"],
             "sdma_minus_kernel_pp_ci95": full["sdma_minus_kernel_pp"]},
            "matched_time": [f"{m['sdma']} {m['coll_ms'][0]}ms {m['slowdown_pct'][0]}% vs {m['kernel']} "
                             f"{m['coll_ms'][1]}ms {m['slowdown_pct'][1]}%: {m['sdma_minus_kernel_pp'][0]} "
                             f"[{m['sdma_minus_kernel_pp'][1]}, {m['sdma_minus_kernel_pp'][2]}] pp"
                             for m in v["matched_time"]],
            "pareto": v["pareto"],
            "sdma_lower_at_full_cus": v["target_sdma_lower_at_full_cus"],
            "sdma_lower_at_some_matched_time": v["sdma_lower_at_some_matched_time"]}


def reduce_hops_by_position(iv, bytes_per_launch, calls):
    """The plain reduce hops of `calls` all-reduces split by position: the
    first reduce-scatter hop, whose two operands were last written six or
    more hops earlier (out of the 256 MB MALL by then), and the later ones,
    whose incoming operand is the previous hop's output, read back from the
    MALL.  iv: (n, 3) intervals in issue order."""
    if calls <= 0 or len(iv) == 0 or len(iv) % calls:
        return None
    per = len(iv) // calls
    d = (iv[:, 1] - iv[:, 0]).reshape(calls, per)  # ms
    out = {}
    for name, sel, bound, note in (
            ("first_hop", d[:, :1], "hbm", "both operands last written 6 or more hops earlier: read from HBM"),
            ("later_hops", d[:, 1:], "hbm+mall",
             "the incoming operand is the previous hop's output, read back from the 256 MB MALL")):
        if sel.size == 0:
            continue
        us = float(sel.mean()) * 1e3
        gbs = bytes_per_launch / (us * 1e-6) / 1e9
        out[name] = {"bound": bound, "achieved": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "mean_launch_us": round(us, 3), "launches": int(sel.size), "note": note}
    return out


def kernel_means(rows):
    """Mean duration (ns) per kernel name in a rocprofv3 kernel trace."""
    acc = {}
    for r in rows:
        d = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        n, t = acc.get(r["Kernel_Name"], (0, 0))
        acc[r["Kernel_Name"]] = (n + 1, t + d)
    return {k: t / n for k, (n, t) in acc.items()}


def _releases(name):
    """The GPU sleep that releases both streams of a loaded window."""
    n = name.lower()
    return "sleep" in n or "spin_kernel" in n


def contention_from_trace(rows, n_cu=256, allowed=256, alone=None):
    """HOCCL Eq. 1 from a rocprofv3 kernel trace of one loaded window: the
    compute units the collective's kernels hold while the compute kernels
    run, over n_cu times the compute kernels' active time.  rows: the trace's
    records (dicts with Kernel_Name, Start_Timestamp, End_Timestamp,
    Grid_Size_X, Workgroup_Size_X).  The window starts after the last GPU
    sleep kernel (which releases both streams); compute is every other
    kernel that is not the library's, active from the first one's start to
    the last one's end.
    - interval_bound: a collective kernel holds min(its workgroups, allowed)
      compute units for its whole traced interval (as the event-based
      figure does); a kernel starved behind the compute kernels stretches
      over much of the window, so this is an upper bound;
    - work_estimate (when `alone` maps kernel names to their durations in
      ns with nothing else running): a kernel holds those units only for its
      unloaded duration, the compute-unit time it needs, counted in
      proportion to the part of its interval inside the window."""
    recs = [(int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"],
             int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))) for r in rows]
    rel = [e for b, e, n, _ in recs if _releases(n)]
    t_from = max(rel) if rel else min(b for b, _, _, _ in recs)
    recs = [x for x in recs if x[0] >= t_from]
    coll = [x for x in recs if "ccr::" in x[2]]
    comp = [x for x in recs if "ccr::" not in x[2] and not _releases(x[2])]
    if not comp:
        return None
    t0 = min(b for b, _, _, _ in comp)
    t1 = max(e for _, e, _, _ in comp)
    win = (t1 - t0) * 1e-6
    iv = [((b - t0) * 1e-6, (e - t0) * 1e-6, min(wg, allowed)) for b, e, _, wg in coll]
    out = {"interval_bound": round(contention_rate(iv, win, n_cu), 4),
           "compute_active_ms": round(win, 3), "compute_kernels": len(comp),
           "collective_kernels": len(coll),
           "collective_kernel_ms": round(sum(e - b for b, e, _, _ in coll) * 1e-6, 3)}
    if alone:
        work = 0.0  # compute-unit nanoseconds
        for b, e, name, wg in coll:
            inside = max(0, min(e, t1) - max(b, t0))
            if inside <= 0 or e <= b:
                continue
            need = min(e - b, alone.get(name, e - b))
            work += need * (inside / (e - b)) * min(wg, allowed)
        out["work_estimate"] = round(work / (n_cu * (t1 - t0)), 4)
    return out


def slowdown_key(r):
    """Name of a full-CU overlap run in the GEMM-slowdown summary."""
    if "dma_deadline" in r:
        return "sdma_deadline"
    if r["dma_engines"] in (None, "all"):
        return r["copy_mode"]
    return f"sdma_{r['dma_engines']}_engines"


def back_to_back_ms(fn, calls, warm=5):
    """Time per call of `calls` calls enqueued back to back between two
    events (how nccl-tests times a collective), after `warm` calls."""
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(calls):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / calls


def event_times(fn, reps=20, warm=5, before=None):
    """Event times (ms) of `reps` calls of fn, each alone, after `warm`
    untimed calls; `before` (untimed) runs ahead of each timed call, e.g. a
    scratch write that evicts the caches."""
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        if before is not None:
            before()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return ts


def median_ms(fn, reps=10, warm=3, before=None):
    """Median event time of fn (see event_times)."""
    ts = event_times(fn, reps, warm, before)
    return sorted(ts)[len(ts) // 2]


def spread(ts):
    """p10 and p90 of event times, for a workload figure reported as its median."""
    p = percentiles(ts)
    return {"p10_ms": p["p10_ms"], "p90_ms": p["p90_ms"], "n": p["n"]}


def bf16_modes(ccr, xs):
    """The gradient bucket with both bf16 accumulation modes: time per
    all-reduce, and the error against the float64 sum of the same bf16
    inputs, max |y - ref| / max |ref| (the accuracy bar is 1e-2)."""
    import torch
    ref = np.zeros(xs[0].size, np.float64)
    for x in xs:
        ref += (x.astype(np.uint32) << 16).view(np.float32)
    scale = np.abs(ref).max()
    pristine = [to_dev(x) for x in xs]
    bufs = [p.clone() for p in pristine]
    out = {}
    for mode in ("per_hop", "fp32_partials"):
        with ccr.Context(0, ccr.Config(bf16_acc=mode)) as ctx:
            ms = median_ms(lambda: ccr.ccr_allreduce(ctx, bufs), 10,
                           before=lambda: [b.copy_(p) for b, p in zip(bufs, pristine)])
            for b, p in zip(bufs, pristine):
                b.copy_(p)
            ccr.ccr_allreduce(ctx, bufs)
            torch.cuda.synchronize()
        y = bufs[0].float().cpu().numpy().astype(np.float64)
        out[mode] = {"ms": round(ms, 4), "max_err_over_max_ref": float(np.abs(y - ref).max() / scale)}
    return out


def size_sweep(ccr, R=8, sizes_mib=(2, 4, 8, 16, 64, 256, 1024)):
    """The pages' message-size sweep (nccl-tests style), at R = 8 bf16 ranks:
    busBW of the all-reduce and of the all-gather alone, with kernel and
    with SDMA copies, per-rank sizes in MiB; up to 2 MiB the kernel
    all-reduce replays from the context's graph cache; up to 16 MiB the eager
    all-reduce is timed beside it."""
    import torch
    out = []
    for mib in sizes_mib:
        N = (mib << 20) // 2
        bufs = [torch.randn(N, device="cuda").mul_(1e-3).to(torch.bfloat16) for _ in range(R)]
        row = {"mib_per_rank": mib}
        for mode in ("kernel", "sdma"):
            with ccr.Context(0, ccr.Config(copy_mode=mode)) as ctx:
                reps = 10 if mib <= 64 else 4
                ar = median_ms(lambda: ccr.ccr_allreduce(ctx, bufs), reps, warm=2)
                ag = median_ms(lambda: ccr.ccr_all_gather(ctx, bufs), reps, warm=2)
            row[f"allreduce_{mode}_busbw"] = round(2 * N / (ar * 1e-3) * 2 * (R - 1) / R / 1e9, 1)
            row[f"allgather_{mode}_busbw"] = round(2 * N / (ag * 1e-3) * (R - 1) / R / 1e9, 1)
        if mib <= 16:
            # up to 2 MiB per rank the 8-rank all-reduce above is replayed from
            # the context's graph cache; the same calls launched eagerly:
            with ccr.Context(0, ccr.Config(graph_cache=False)) as ctx:
                ar = median_ms(lambda: ccr.ccr_allreduce(ctx, bufs), 10, warm=2)
            row["allreduce_kernel_eager_busbw"] = round(2 * N / (ar * 1e-3) * 2 * (R - 1) / R / 1e9, 1)
        out.append(row)
        del bufs
    torch.cuda.empty_cache()
    return out


def moe_buffers(ccr, m):
    """Inputs, routing, plan and every buffer of one expert-parallel
    dispatch / combine of workload m, on cuda:0."""
    import torch
    R, T, H, E, K = m.R, m.tokens, m.hidden, m.experts, m.topk
    xs = [torch.randn(T, H, device="cuda").to(torch.bfloat16) for _ in range(R)]
    logits = [torch.randn(T, E, device="cuda") for _ in range(R)]
    with ccr.Context(0) as ctx:
        topk = [torch.empty(T, K, dtype=torch.int32, device="cuda") for _ in range(R)]
        src_tok = [torch.empty(T * K, dtype=torch.int32, device="cuda") for _ in range(R)]
        slot = [torch.empty(T * K, dtype=torch.int32, device="cuda") for _ in range(R)]
        route_ms = median_ms(lambda: [ccr.ccr_moe_topk(ctx, logits[r], topk[r]) for r in range(R)], 10)
        ecnt = np.stack([ccr.ccr_moe_plan(ctx, topk[r], E, R, src_tok[r], slot[r]) for r in range(R)])
    rows = [int(ecnt[:, (E // R) * d:(E // R) * (d + 1)].sum()) for d in range(R)]
    return {"xs": xs, "src_tok": src_tok, "slot": slot, "ecnt": ecnt, "route_ms": route_ms,
            "send": [torch.empty(T * K, H, dtype=torch.bfloat16, device="cuda") for _ in range(R)],
            "recv": [torch.empty(n, H, dtype=torch.bfloat16, device="cuda") for n in rows],
            "exp": [torch.empty(n, H, dtype=torch.bfloat16, device="cuda") for n in rows],
            "out": [torch.empty(T, K, H, dtype=torch.bfloat16, device="cuda") for _ in range(R)]}


def moe_probe(ccr, workloads, steps):
    """Only the fused dispatch and combine of the MoE dispatch workload,
    `steps` times each (the run behind the gather kernel's profiles)."""
    import torch
    m = workloads.MOE_DISPATCH_BF16
    b = moe_buffers(ccr, m)
    with ccr.Context(0) as ctx:
        for _ in range(steps):
            ccr.ccr_moe_dispatch_fused(ctx, b["xs"], b["src_tok"], b["ecnt"], m.topk, b["exp"])
            ccr.ccr_moe_combine_fused(ctx, b["exp"], b["slot"], b["ecnt"], m.tokens, m.topk, b["out"])
        torch.cuda.synchronize()
    log(f"moe probe: {steps} fused dispatch + combine")


def loaded_window_probe(ccr, workloads, mode, n_gemm=20, n_coll=6):
    """One loaded window only (the run behind the contention-rate trace):
    n_gemm back-to-back 8192^3 bf16 GEMMs on one stream and n_coll bucket
    all-reduces (full CUs, kernel or SDMA copies) on another, released
    together by an event after a GPU sleep.  Prints the event-based
    contention bound of the same window."""
    import torch
    w = workloads.DP_BUCKET_BF16
    bufs = [to_dev(x) for x in workloads.ring_inputs(w)]
    A = torch.randn(8192, 8192, dtype=torch.bfloat16, device="cuda")
    B = torch.randn(8192, 8192, dtype=torch.bfloat16, device="cuda")
    C = torch.empty(8192, 8192, dtype=torch.bfloat16, device="cuda")
    g, c, s0 = own_queue_stream(0), own_queue_stream(1), own_queue_stream(2)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    with ccr.Context(0, ccr.Config(copy_mode=mode)) as ctx:
        with torch.cuda.stream(g):
            for _ in range(2):
                torch.matmul(A, B, out=C)
        ccr.ccr_allreduce(ctx, bufs, stream=c)
        torch.cuda.synchronize()
        ccr.ccr_profile_enable(ctx, True)
        go = torch.cuda.Event()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        with torch.cuda.stream(s0):
            torch.cuda._sleep(20_000_000)
            go.record(s0)
        g.wait_event(go)
        c.wait_event(go)
        with torch.cuda.stream(g):
            ev[0].record(g)
            for _ in range(n_gemm):
                torch.matmul(A, B, out=C)
            ev[1].record(g)
        for _ in range(n_coll):
            ccr.ccr_allreduce(ctx, bufs, stream=c)
        torch.cuda.synchronize()
        iv = np.concatenate([ccr.ccr_profile_intervals(ctx, k, ev[0])
                             for k in ("reduce", "copy_kernel", "reduce_forward")])
        ccr.ccr_profile_enable(ctx, False)
    gemm = ev[0].elapsed_time(ev[1])
    print(json.dumps({"loaded_window": mode, "gemm_ms": round(gemm, 3),
                      "event_bound_contention_rate": round(contention_rate(iv, gemm, n_cu), 4)}), flush=True)


PROBE_WORKLOADS = ("ring_allreduce_r4_1m_f32", "rs_ag_r32_8m_f32", "pp_sendrecv_4x2048x4096_bf16",
                   "moe_dispatch_combine_three_stage")


def workload_probe(ccr, workloads, name, steps):
    """Only `steps` calls of one of the other workloads, kernel copies, full
    CUs (the runs behind their kernel-trace profiles)."""
    import torch
    if name in ("ring_allreduce_r4_1m_f32", "rs_ag_r32_8m_f32"):
        w = workloads.RING_SMALL_F32 if name == "ring_allreduce_r4_1m_f32" else workloads.RS_AG_R32_F32
        bufs = [torch.rand(w.count, device="cuda") * 2 - 1 for _ in range(w.R)]
        with ccr.Context(0, ccr.Config(slices=w.slices)) as ctx:
            for _ in range(steps):
                if name == "ring_allreduce_r4_1m_f32":
                    ccr.ccr_allreduce(ctx, bufs)
                else:
                    ccr.ccr_reduce_scatter(ctx, bufs)
                    ccr.ccr_all_gather(ctx, bufs)
            torch.cuda.synchronize()
            if name == "ring_allreduce_r4_1m_f32":
                # references of the same size in the same trace: torch's copy of
                # one rank's 4 MiB (the bytes of one copy hop), and a kernel of
                # 512 one-wave workgroups that only records its CU ids (the
                # launch alone, at the copy hop's workgroup count)
                dst = torch.empty_like(bufs[0])
                ids = torch.zeros(512, 3, dtype=torch.int32, device="cuda")
                for _ in range(steps):
                    dst.copy_(bufs[0])
                    ccr._check(ccr._lib.ccr_probe_cu_ids(ctx.handle, ids.data_ptr(), 512, None))
                torch.cuda.synchronize()
                # the same call and the same empty kernel replayed from HIP
                # graphs, so that the GPU dispatches them back to back with no
                # host in the loop (the trace's gaps are then the GPU's own)
                g_call, g_empty = launch_floor_graphs(ccr, ctx, bufs, ids)
                for _ in range(max(1, steps // 10)):
                    g_call.replay()
                    g_empty.replay()
                torch.cuda.synchronize()
    elif name == "pp_sendrecv_4x2048x4096_bf16":
        pw = workloads.PP_STAGING_BF16
        mbs = [torch.randn(pw.rows, pw.cols, device="cuda").to(torch.bfloat16)
               for _ in range(pw.microbatches)]
        outs = [torch.empty_like(x) for x in mbs]
        cfg = ccr.Config(staging_chunk_bytes=pw.chunk_bytes, staging_slots=pw.slots)
        with ccr.Context(0, cfg) as ctx:
            for _ in range(steps):
                ccr.ccr_sendrecv_batch(ctx, mbs, outs)
            torch.cuda.synchronize()
    else:
        m = workloads.MOE_DISPATCH_BF16
        b = moe_buffers(ccr, m)
        with ccr.Context(0) as ctx:
            for _ in range(steps):
                ccr.ccr_moe_dispatch(ctx, b["xs"], b["src_tok"], b["ecnt"], m.topk, b["send"],
                                     b["recv"], b["exp"])
                ccr.ccr_moe_combine(ctx, b["exp"], b["slot"], b["ecnt"], m.tokens, m.topk,
                                    b["recv"], b["send"], b["out"])
            torch.cuda.synchronize()
    log(f"workload probe: {steps} calls of {name}")


def launch_floor_graphs(ccr, ctx, bufs, ids, calls=10):
    """Two HIP graphs captured on a side stream: `calls` all-reduce calls of
    `bufs`, and 5 * `calls` launches in a row of the empty 512-workgroup probe
    kernel (it only records CU ids into `ids`), i.e. `calls` chains of as many
    launches as the 4-rank call makes.  Replayed, the GPU runs them back to
    back without waiting for the host."""
    import torch
    ccr._check(ccr._lib.ccr_probe_cu_ids(ctx.handle, ids.data_ptr(), 512, None))  # side stream made eagerly
    torch.cuda.synchronize()
    gs = torch.cuda.Stream()
    g_call, g_empty = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_call, stream=gs):
        for _ in range(calls):
            ccr.ccr_allreduce(ctx, bufs)
    with torch.cuda.graph(g_empty, stream=gs):
        for _ in range(5 * calls):
            ccr._check(ccr._lib.ccr_probe_cu_ids(ctx.handle, ids.data_ptr(), 512, gs.cuda_stream))
    torch.cuda.synchronize()
    return g_call, g_empty


def graph_per_call_us(g, calls, reps=10):
    """Median over `reps` replays of one replay's event time, per call (us)."""
    ts = event_times(g.replay, reps=reps, warm=2)
    return round(sorted(ts)[len(ts) // 2] * 1e3 / calls, 2)


def workload_timings(ccr, workloads):
    """The other workloads, for context (each is also a full-size parity
    test): per call, 5 untimed warm-up calls, then 20 calls each timed alone
    with events; the median, p10 and p90, and the figures of merit."""
    import torch
    out = {}
    for w, how in ((workloads.RING_SMALL_F32, "allreduce"), (workloads.RS_AG_R32_F32, "rs_then_ag")):
        bufs = [torch.rand(w.count, device="cuda") * 2 - 1 for _ in range(w.R)]
        b, R, N = 4, w.R, w.count
        cold = cold_ts = None
        b2b = host_us = floor = None
        with ccr.Context(0, ccr.Config(slices=w.slices)) as ctx:
            if how == "allreduce":
                ts = event_times(lambda: ccr.ccr_allreduce(ctx, bufs))
                algo = b * N * (3 * (R - 1) + 1 + 2 * (R - 2))
                # per call as nccl-tests times it: calls back to back between two events
                b2b = back_to_back_ms(lambda: ccr.ccr_allreduce(ctx, bufs), 100)
                # host time to enqueue one call (its five launches), through the binding
                host_us = host_call_us(ccr, lambda: ccr.ccr_allreduce(ctx, bufs))
                # the GPU alone: the call, and 5 launches of an empty kernel of
                # the copy hop's 512 workgroups, each replayed from a graph
                ids = torch.zeros(512, 3, dtype=torch.int32, device="cuda")
                g_call, g_empty = launch_floor_graphs(ccr, ctx, bufs, ids)
                floor = {"graph_replay_us_per_call": graph_per_call_us(g_call, 10),
                         "empty_5_launches_us": round(5 * graph_per_call_us(g_empty, 50), 2)}
                del g_call, g_empty
                if R * N * b <= (128 << 20):  # fits the 256 MB MALL: also time it cold
                    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
                    cold_ts = event_times(lambda: ccr.ccr_allreduce(ctx, bufs),
                                          before=lambda: scratch.fill_(1))
                    cold = sorted(cold_ts)[len(cold_ts) // 2]
                    del scratch
            else:
                ts = event_times(lambda: (ccr.ccr_reduce_scatter(ctx, bufs),
                                          ccr.ccr_all_gather(ctx, bufs)))
                algo = b * N * 5 * (R - 1)
        ms = sorted(ts)[len(ts) // 2]
        out[w.name] = {"ms": round(ms, 4), **spread(ts), "cold_ms": None if cold is None else round(cold, 4),
                       **({"cold": spread(cold_ts)} if cold_ts else {}),
                       **({"back_to_back_ms": round(b2b, 4),
                           "back_to_back_hbm_frac": round(algo / (b2b * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                           "host_us_per_call": host_us, "launch_floor": floor}
                          if b2b else {}),
                       "busbw_gbs": round(b * N / (ms * 1e-3) * 2 * (R - 1) / R / 1e9, 1),
                       "algorithmic_gbs": round(algo / (ms * 1e-3) / 1e9, 1),
                       "hbm_frac": round(algo / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "slices": w.slices}
        del bufs
    m = workloads.MOE_DISPATCH_BF16
    R, T, H, E, K = m.R, m.tokens, m.hidden, m.experts, m.topk
    b = moe_buffers(ccr, m)
    xs, src_tok, slot, ecnt = b["xs"], b["src_tok"], b["slot"], b["ecnt"]
    send, recv, exp, outb, route_ms = b["send"], b["recv"], b["exp"], b["out"], b["route_ms"]
    moved = R * T * K * H * 2  # bytes of rows each stage moves over all ranks
    res = {"route_topk_ms_all_ranks": round(route_ms, 4), "rows_per_rank": T * K,
           "exchange_bytes": moved}
    for mode in ("kernel", "sdma"):
        with ccr.Context(0, ccr.Config(copy_mode=mode)) as ctx:
            d_ts = event_times(lambda: ccr.ccr_moe_dispatch(ctx, xs, src_tok, ecnt, K, send, recv, exp))
            c_ts = event_times(lambda: ccr.ccr_moe_combine(ctx, exp, slot, ecnt, T, K, recv, send, outb))
        d_ms, c_ms = sorted(d_ts)[len(d_ts) // 2], sorted(c_ts)[len(c_ts) // 2]
        # three stages (pack, exchange, unpack), each reading and writing `moved` bytes
        res[mode] = {"dispatch_ms": round(d_ms, 4), "combine_ms": round(c_ms, 4),
                     "dispatch": spread(d_ts), "combine": spread(c_ts),
                     "dispatch_algorithmic_gbs": round(3 * 2 * moved / (d_ms * 1e-3) / 1e9, 1),
                     "exchange_algbw_gbs": round(moved / (d_ms * 1e-3) / 1e9, 1)}
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    flush = lambda: scratch.fill_(1)  # noqa: E731
    with ccr.Context(0) as ctx:
        d_ts = event_times(lambda: ccr.ccr_moe_dispatch_fused(ctx, xs, src_tok, ecnt, K, exp))
        c_ts = event_times(lambda: ccr.ccr_moe_combine_fused(ctx, exp, slot, ecnt, T, K, outb))
        d_ms, c_ms = sorted(d_ts)[len(d_ts) // 2], sorted(c_ts)[len(c_ts) // 2]
        # cold: a 512 MiB scratch write before each call evicts the MALL
        dc_ts = event_times(lambda: ccr.ccr_moe_dispatch_fused(ctx, xs, src_tok, ecnt, K, exp), before=flush)
        cc_ts = event_times(lambda: ccr.ccr_moe_combine_fused(ctx, exp, slot, ecnt, T, K, outb), before=flush)
        k_cold = None
        with ccr.Context(0, ccr.Config(copy_mode="kernel")) as kctx:
            k_cold = event_times(lambda: ccr.ccr_moe_dispatch(kctx, xs, src_tok, ecnt, K, send, recv, exp),
                                 before=flush)
        gbs = {}
        for name, fn in (("dispatch", lambda: ccr.ccr_moe_dispatch_fused(ctx, xs, src_tok, ecnt, K, exp)),
                         ("combine", lambda: ccr.ccr_moe_combine_fused(ctx, exp, slot, ecnt, T, K, outb))):
            ccr.ccr_profile_enable(ctx, True)
            for _ in range(5):
                fn()
            g = ccr.ccr_profile_read(ctx, "moe_gather")
            gbs[name] = (round(g["bytes"] / (g["ms"] * 1e-3) / 1e9, 1) if g["ms"] else None,
                         round(g["ms"] / max(1, g["launches"]) * 1e3, 2))
        ccr.ccr_profile_enable(ctx, False)
    # one gather: every row read once and written once
    res["fused"] = {"dispatch_ms": round(d_ms, 4), "combine_ms": round(c_ms, 4),
                    "dispatch": spread(d_ts), "combine": spread(c_ts),
                    "dispatch_algorithmic_gbs": round(2 * moved / (d_ms * 1e-3) / 1e9, 1),
                    "exchange_algbw_gbs": round(moved / (d_ms * 1e-3) / 1e9, 1),
                    "dispatch_gather_kernel": {"gbs": gbs["dispatch"][0], "us": gbs["dispatch"][1]},
                    "combine_gather_kernel": {"gbs": gbs["combine"][0], "us": gbs["combine"][1]},
                    "cold": {"dispatch_ms": round(sorted(dc_ts)[len(dc_ts) // 2], 4), "dispatch": spread(dc_ts),
                             "combine_ms": round(sorted(cc_ts)[len(cc_ts) // 2], 4), "combine": spread(cc_ts),
                             "note": "512 MiB scratch write before each call"}}
    res["kernel"]["cold_dispatch_ms"] = round(sorted(k_cold)[len(k_cold) // 2], 4)
    out[m.name] = res
    # pipeline-parallel activations through the staging slots, each copy mode
    pw = workloads.PP_STAGING_BF16
    mbs = [torch.randn(pw.rows, pw.cols, device="cuda").to(torch.bfloat16) for _ in range(pw.microbatches)]
    outs = [torch.empty_like(x) for x in mbs]
    payload = sum(x.numel() * x.element_size() for x in mbs)
    pp = {"payload_bytes": payload, "chunk_bytes": pw.chunk_bytes, "slots": pw.slots}
    for mode in ("kernel", "sdma"):
        with ccr.Context(0, ccr.Config(copy_mode=mode, staging_chunk_bytes=pw.chunk_bytes,
                                       staging_slots=pw.slots)) as ctx:
            ts = event_times(lambda: ccr.ccr_sendrecv_batch(ctx, mbs, outs))
            cold_ts = event_times(lambda: ccr.ccr_sendrecv_batch(ctx, mbs, outs), before=flush)
            b2b = back_to_back_ms(lambda: ccr.ccr_sendrecv_batch(ctx, mbs, outs), 50)
        ms = sorted(ts)[len(ts) // 2]
        cms = sorted(cold_ts)[len(cold_ts) // 2]
        # every chunk is copied in (fill) and out (drain): 2 reads + 2 writes per byte
        pp[mode] = {"ms": round(ms, 4), **spread(ts), "cold_ms": round(cms, 4), "cold": spread(cold_ts),
                    "cold_algorithmic_gbs": round(4 * payload / (cms * 1e-3) / 1e9, 1),
                    "back_to_back_ms": round(b2b, 4),
                    "back_to_back_algorithmic_gbs": round(4 * payload / (b2b * 1e-3) / 1e9, 1),
                    "algbw_gbs": round(payload / (ms * 1e-3) / 1e9, 1),
                    "algorithmic_gbs": round(4 * payload / (ms * 1e-3) / 1e9, 1)}
    out[pw.name] = pp
    del scratch
    return out


def oracle_timings(workloads):
    """The CPU oracle on the other workloads, one host core, each at its full
    size (inputs generated beforehand, outside the timing; one call each)."""
    import oracle
    out = {}

    def once(fn):
        t = time.perf_counter()
        fn()
        return round((time.perf_counter() - t) * 1e3, 1)

    w = workloads.RING_SMALL_F32
    xs = workloads.ring_inputs(w)
    out[w.name] = once(lambda: oracle.ring_allreduce(xs, S=w.slices))
    w = workloads.RS_AG_R32_F32
    xs = workloads.ring_inputs(w)
    out[w.name] = once(lambda: oracle.ring_all_gather(oracle.ring_reduce_scatter(xs, S=w.slices),
                                                      S=w.slices))
    del xs
    pw = workloads.PP_STAGING_BF16
    mbs = workloads.staging_inputs(pw)
    out[pw.name] = once(lambda: oracle.staged_copy(mbs, pw.chunk_bytes, pw.slots))
    m = workloads.MOE_DISPATCH_BF16
    xs, logits = workloads.moe_inputs(m)
    out[m.name] = once(lambda: oracle.moe_dispatch(xs, [oracle.moe_topk(l, m.topk) for l in logits],
                                                   m.experts))
    return {k: {"oracle_ms": v, "cores": 1} for k, v in out.items()}


def schedule_timings(ccr, workloads):
    """Stage decomposition (host only) of a skewed expert-parallel dispatch
    over a modelled two-node, 16-GPU MI355X cluster: the stage count, the
    modelled time of the schedule (sum of stage times, HOCCL Eq. 11) beside
    a lower bound that no schedule beats, and the host time per call."""
    w = workloads.SCHED_MOE_2X8
    t = w.topology
    C = np.ascontiguousarray(workloads.moe_traffic(w), np.int64)
    node = np.array(t.node(), np.int32)
    peer = np.array(t.peer(), np.int32)
    entries, times = ccr.ccr_schedule_stages(C, node, peer, t.bw_scaleup, t.bw_rdma)
    reps = []
    for _ in range(20):
        t0 = time.perf_counter()
        ccr.ccr_schedule_stages(C, node, peer, t.bw_scaleup, t.bw_rdma)
        reps.append(time.perf_counter() - t0)
    T = ccr.ccr_traffic_matrix(C, node, peer)
    cross = node[:, None] != node[None, :]
    # bytes / (GB/s) = ns.  Each GPU moves its inter-node bytes at most one
    # flow at a time per direction, and a scale-up cell's bytes over one link.
    rdma_ns = max(np.where(cross, C, 0).sum(axis=1).max(), np.where(cross, C, 0).sum(axis=0).max()) / t.bw_rdma
    up_ns = np.where(cross, 0, T).max() / t.bw_scaleup
    model_ns = float(sum(int(l) / int(b) for l, b in times.tolist()))
    bound_ns = float(max(rdma_ns, up_ns))
    return {"workload": w.name, "topology": t.name, "gpus": t.G,
            "flows": int((C > 0).sum()), "stages": int(len(times)),
            "rdma_stages": int(len(set(entries["stage"][entries["kind"] == 0].tolist()))),
            "modelled_ms": round(model_ns / 1e6, 4), "lower_bound_ms": round(bound_ns / 1e6, 4),
            "modelled_over_bound": round(model_ns / bound_ns, 4) if bound_ns else None,
            "host_us_per_call": round(float(np.median(reps)) * 1e6, 1)}


def host_call_us(ccr, call, reps=50, windows=7):
    """Host time per enqueue (HOCCL Fig. 9 measures CPU launch time per op):
    the median over `windows` loops of `reps` calls each, so that one
    preemption of the host thread does not decide the figure."""
    import torch
    per = []
    for _ in range(windows):
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(reps):
            call()
        per.append((time.perf_counter() - t) / reps)
    torch.cuda.synchronize()
    return round(sorted(per)[len(per) // 2] * 1e6, 2)


COUNTERS = os.path.join(ROOT, "profiles", "ring_allreduce_dp_bucket_r8_bf16_hbm_counters.md")
# the sources of the streaming kernels the counters measured
KERNELS = [os.path.join(ROOT, "collective_communication_reduce_amd", "csrc", f)
           for f in ("ccr_device.h", "ccr_kernels.hip", "ccr_ring.hip")]


def kernel_source_sha256(paths=None):
    """sha256 over the streaming kernels' sources, concatenated in order."""
    import hashlib
    h = hashlib.sha256()
    for p in paths or KERNELS:
        h.update(open(p, "rb").read())
    return h.hexdigest()


def measured_traffic(key="reduce_hop_traffic_bytes_per_launch"):
    """HBM bytes per launch from the committed FETCH_SIZE/WRITE_SIZE summary,
    or None when the kernel source has changed since the counters were
    taken."""
    try:
        fields = dict(l.split(": ", 1) for l in open(COUNTERS).read().splitlines() if ": " in l
                      and not l.startswith(("|", "#", "`")))
        sha = kernel_source_sha256()
    except OSError:
        return None
    if fields.get("kernel_source_sha256", "").strip() != sha:
        return None
    return int(float(fields[key]))


def cu_occupancy(ccr, budgets=(0, 64, 32, 16), nblocks=4096):
    """Distinct compute units (XCC, SE, CU hardware ids) that a burst of
    one-wave workgroups on the collective's stream lands on, per CU budget."""
    out = {}
    for b in budgets:
        with ccr.Context(0, ccr.Config(cu_budget=b)) as ctx:
            ids = ccr.ccr_probe_cu_ids(ctx, nblocks).cpu().numpy()
        cus = {tuple(r) for r in ids.tolist()}
        out[str(b or 256)] = {"cus": len(cus), "xccs": len({r[0] for r in cus})}
    return out


def restored_steps(fn, bufs, steps):
    """Per-step times (ms) of `fn` with every input restored from a pristine
    device copy before each step, outside the timed region, so each step
    reduces the same bits.  Events on the current stream bracket each step."""
    import torch
    pristine = [b.clone() for b in bufs]
    times = []
    for _ in range(steps):
        for b, p in zip(bufs, pristine):
            b.copy_(p)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    for b, p in zip(bufs, pristine):
        b.copy_(p)
    return times


def percentiles(ts):
    a = np.sort(np.asarray(ts, dtype=np.float64))
    return {"median_ms": round(float(np.median(a)), 4), "p10_ms": round(float(np.percentile(a, 10)), 4),
            "p90_ms": round(float(np.percentile(a, 90)), 4), "n": int(a.size)}


def copy_roofline(ccr, nbytes=1 << 30, reps=5):
    """The library's copy kernel on one plain nbytes copy at full CUs: the
    practical streaming ceiling the reduce hop is compared with."""
    import torch
    a = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    with ccr.Context(0) as ctx:
        ccr.ccr_alltoall_rows(ctx, [a], [b], [[nbytes // 16]], 16)
        ccr.ccr_profile_enable(ctx, True)
        for _ in range(reps):
            ccr.ccr_alltoall_rows(ctx, [a], [b], [[nbytes // 16]], 16)
        st = ccr.ccr_profile_read(ctx, "copy_kernel")
        ccr.ccr_profile_enable(ctx, False)
    del a, b
    return st["bytes"] / (st["ms"] * 1e6)


def copy_probe(ccr, nbytes, reps):
    """A plain copy of nbytes through the library's copy kernel, reps times
    (the calibration run for the HBM traffic counters)."""
    import torch
    a = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    with ccr.Context(0) as ctx:
        for _ in range(reps):
            ccr.ccr_alltoall_rows(ctx, [a], [b], [[nbytes // 16]], 16)
        torch.cuda.synchronize()
    assert torch.equal(a, b)
    log(f"copy probe: {reps} x {nbytes} bytes")


def cpu_baseline(xs, R, count, esize, S, budget_s=12.0):
    import oracle
    t0 = time.perf_counter()
    n = 0
    while True:
        oracle.ring_allreduce(xs, S=S)
        n += 1
        if time.perf_counter() - t0 >= budget_s or n >= 20:
            break
    t = (time.perf_counter() - t0) / n
    bus = esize * count / t * 2 * (R - 1) / R / 1e9
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    out = {"value": bus, "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"the full workload, {n} all-reduce(s), single-threaded C oracle",
           "ms_per_step": t * 1e3, "host_cpus": os.cpu_count(), "cpu_model": model}
    # The same oracle arithmetic on T host cores: each all-reduce's element
    # range cut into T parts, every part run through all hops on a thread
    # of its own (oracle.ring_allreduce_threads: bit for bit the one-thread
    # result, pinned by the oracle tests), timed per call.
    T = min(16, os.cpu_count() or 1)
    if T > 1:
        oracle.ring_allreduce_threads(xs, T, S=S)  # warm the pool's first call
        t0 = time.perf_counter()
        calls = 0
        while True:
            oracle.ring_allreduce_threads(xs, T, S=S)
            calls += 1
            if time.perf_counter() - t0 >= budget_s or calls >= 40:
                break
        tt = (time.perf_counter() - t0) / calls
        out["threads"] = {"cores": T, "value": esize * count / tt * 2 * (R - 1) / R / 1e9,
                          "ms_per_step": tt * 1e3,
                          "sample": f"{calls} all-reduces of the full workload, each split over {T} "
                                    "threads by element range (the same per-element operations in "
                                    "the same order)"}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--slices", type=int, default=None)
    ap.add_argument("--overlap", type=int, default=0)
    ap.add_argument("--bf16-acc", choices=("per_hop", "fp32_partials"), default="per_hop",
                    help="bf16 accumulation of the timed all-reduce (default: per_hop)")
    ap.add_argument("--copy-mode", choices=("kernel", "sdma"), default="kernel",
                    help="all-gather copies of the timed all-reduce (default: kernel)")
    ap.add_argument("--no-gemm", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain BYTES copy through the copy kernel (counter calibration)")
    ap.add_argument("--ring-only", action="store_true",
                    help="only the timed all-reduce steps and the per-launch pass (for profiler runs)")
    ap.add_argument("--moe-probe", action="store_true",
                    help="only run --steps fused MoE dispatch + combine calls (gather kernel profiles)")
    ap.add_argument("--workload-probe", choices=PROBE_WORKLOADS, default=None,
                    help="only run --steps calls of one of the other workloads (kernel-trace profiles)")
    ap.add_argument("--loaded-window", choices=("kernel", "sdma"), default=None,
                    help="only run one GEMM + bucket all-reduce window (the contention-rate trace)")
    ap.add_argument("--trace-contention", metavar="KERNEL_TRACE_CSV", default=None,
                    help="no GPU: HOCCL Eq. 1 of the loaded window in a rocprofv3 kernel trace")
    ap.add_argument("--alone-trace", metavar="KERNEL_TRACE_CSV", default=None,
                    help="with --trace-contention: a trace of the same kernels with nothing else "
                         "running, for the work-based estimate")
    args = ap.parse_args()
    if args.trace_contention:
        import csv
        rows = list(csv.DictReader(open(args.trace_contention)))
        alone = kernel_means(list(csv.DictReader(open(args.alone_trace)))) if args.alone_trace else None
        print(json.dumps(contention_from_trace(rows, alone=alone)), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the R ranks are virtual ranks in one GPU's HBM; "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch

    import collective_communication_reduce_amd as ccr
    import workloads

    if args.copy_probe:
        copy_probe(ccr, args.copy_probe, max(1, args.steps))
        return
    if args.moe_probe:
        moe_probe(ccr, workloads, max(1, args.steps))
        return
    if args.workload_probe:
        workload_probe(ccr, workloads, args.workload_probe, max(1, args.steps))
        return
    if args.loaded_window:
        loaded_window_probe(ccr, workloads, args.loaded_window)
        return

    w = workloads.DP_BUCKET_BF16
    R, count, esize = w.R, w.count, 2
    S = args.slices or w.slices
    log(f"bench: {w.name}: generating inputs")
    xs = workloads.ring_inputs(w)
    bufs = [to_dev(x) for x in xs]
    cfg = dict(slices=S, overlap=bool(args.overlap), copy_mode=args.copy_mode, bf16_acc=args.bf16_acc)
    ctx = ccr.Context(0, ccr.Config(**cfg))
    step = lambda: ccr.ccr_allreduce(ctx, bufs)  # noqa: E731
    log(f"bench: warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"bench: timing {args.steps} steps")
    t = time_steps(step, args.steps)
    bus = esize * count / t * 2 * (R - 1) / R / 1e9
    algo = ring_bytes(R, count, esize, fused=True) / t / 1e9

    log("bench: per-launch reduce kernel timing")
    ccr.ccr_profile_enable(ctx, True)
    ref_ev = torch.cuda.Event(enable_timing=True)
    ref_ev.record()
    for _ in range(args.steps):
        step()
    red = ccr.ccr_profile_read(ctx, "reduce")
    fwd = ccr.ccr_profile_read(ctx, "reduce_forward")
    cpy = ccr.ccr_profile_read(ctx, "copy_kernel")
    dma = ccr.ccr_profile_read(ctx, "sdma")
    red_iv = ccr.ccr_profile_intervals(ctx, "reduce", ref_ev)
    ccr.ccr_profile_enable(ctx, False)
    red_gbs = red["bytes"] / (red["ms"] * 1e6)
    cpy_gbs = cpy["bytes"] / (cpy["ms"] * 1e6) if cpy["ms"] else None
    by_position = reduce_hops_by_position(red_iv, red["bytes"] // max(1, red["launches"]), args.steps)

    # Every part after the timed steps is context: a part that fails (e.g. no
    # usable SDMA engine on a machine) is reported under "errors" instead of
    # taking the headline line down with it.
    errors = {}

    def guarded(name, fn):
        try:
            return fn()
        except Exception as e:  # noqa: BLE001
            log(f"bench: {name} failed: {e}")
            errors[name] = f"{type(e).__name__}: {e}"
            return None

    restored = copy_gbs = None
    if not args.ring_only:
        log("bench: per-step times with inputs restored before each step")
        restored = guarded("restored_inputs",
                           lambda: percentiles(restored_steps(step, bufs, max(20, args.steps))))
        log("bench: plain 1 GiB copy (copy roofline)")
        copy_gbs = guarded("copy_roofline", lambda: copy_roofline(ccr))
    if args.ring_only:
        args.no_gemm = args.no_cpu = True

    gemm = ag_only = pp = occ = launch = None
    if not args.no_gemm:
        log("bench: concurrent GEMM, gradient-bucket all-reduce")
        # kernel copies over CU budgets, SDMA copies over the same budgets
        # (reduce kernels budgeted) and over engine counts at full CUs
        runs = [dict(cfg, copy_mode=m, cu_budget=b) for b in (0, 64, 32, 16) for m in ("kernel", "sdma")]
        runs.insert(2, dict(cfg, copy_mode="kernel", cu_budget=128))
        runs += [dict(cfg, copy_mode="sdma", dma_engines=e) for e in (8, 4, 2, 1)]
        runs.append(dict(cfg, copy_mode="sdma", dma_deadline_us="window"))
        runs.append(dict(cfg, copy_mode="sdma", dma_sync="stream_flags"))
        gemm = guarded("gemm_slowdown", lambda: overlap_runs(
            ccr, lambda ctx, st: ccr.ccr_allreduce(ctx, bufs, stream=st), runs, (8192, 8192, 8192), 20, 6))
        log("bench: concurrent GEMM, the bucket's all-gather alone (the copy paths isolated)")
        # the reduce-scatter runs on compute units in either mode; all-gather
        # calls alone compare the two copy paths on the same bytes
        ag_only = guarded("gemm_slowdown_all_gather_only", lambda: overlap_runs(
            ccr, lambda ctx, st: ccr.ccr_all_gather(ctx, bufs, stream=st),
            [dict(cfg, copy_mode="kernel"), dict(cfg, copy_mode="sdma"),
             dict(cfg, copy_mode="sdma", dma_engines=4), dict(cfg, copy_mode="sdma", dma_engines=2)],
            (8192, 8192, 8192), 20, 6))
        log("bench: concurrent GEMM, pipeline-parallel send/recv through staging")
        pw = workloads.PP_STAGING_BF16
        mbs = [torch.randn(pw.rows, pw.cols, device="cuda").to(torch.bfloat16)
               for _ in range(pw.microbatches)]
        outs = [torch.empty_like(x) for x in mbs]
        stg = dict(staging_chunk_bytes=pw.chunk_bytes, staging_slots=pw.slots)
        pp = guarded("pp_staging_gemm_slowdown", lambda: overlap_runs(
            ccr, lambda ctx, st: ccr.ccr_sendrecv_batch(ctx, mbs, outs, stream=st),
            [dict(stg, copy_mode="kernel", cu_budget=b) for b in (0, 64, 32, 16)] +
            [dict(stg, copy_mode="sdma"), dict(stg, copy_mode="sdma", dma_engines=4),
             dict(stg, copy_mode="sdma", dma_engines=2), dict(stg, copy_mode="sdma", dma_engines=1),
             dict(stg, copy_mode="sdma", dma_deadline_us="window")],
            (4096, 4096, 16384), 20, 20))
        if pp is not None:
            pp["workload"] = pw.name
        log("bench: compute units reached under each CU budget; host time per call")
        occ = guarded("cu_occupancy", lambda: cu_occupancy(ccr))

        def host_costs():
            out = {}
            for m in ("kernel", "sdma"):
                with ccr.Context(0, ccr.Config(**dict(cfg, copy_mode=m))) as c2:
                    ccr.ccr_allreduce(c2, bufs)
                    out[f"allreduce_{m}"] = host_call_us(ccr, lambda: ccr.ccr_allreduce(c2, bufs), 20)
                with ccr.Context(0, ccr.Config(**dict(stg, copy_mode=m))) as c2:
                    ccr.ccr_sendrecv_batch(c2, mbs[:1], outs[:1])
                    out[f"sendrecv_16MiB_{m}"] = host_call_us(
                        ccr, lambda: ccr.ccr_sendrecv_batch(c2, mbs[:1], outs[:1]), 20)
            return out
        launch = guarded("host_us_per_call", host_costs)

    others = None
    if not args.no_gemm:
        log("bench: the other workloads (context)")
        others = guarded("other_workloads", lambda: workload_timings(ccr, workloads)) or {}
        others["stage_schedule"] = guarded("stage_schedule", lambda: schedule_timings(ccr, workloads))
        log("bench: bf16 accumulation modes on the bucket")
        others["dp_bucket_bf16_accumulation"] = guarded("bf16_modes", lambda: bf16_modes(ccr, xs))
        log("bench: message-size sweep")
        others["size_sweep_r8_bf16"] = guarded("size_sweep", lambda: size_sweep(ccr))

    cpu = None
    if not args.no_cpu:
        log("bench: CPU oracle baseline")
        cpu = guarded("cpu_baseline", lambda: cpu_baseline(xs, R, count, esize, S))
        if others is not None and cpu is not None:
            log("bench: CPU oracle on the other workloads")
            cpu["other_workloads"] = guarded("cpu_other_workloads", lambda: oracle_timings(workloads))

    line = {
        "metric": METRIC, "value": round(bus, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(t * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "ranks": R, "count_per_rank": count, "slices": S,
                   "overlap": bool(args.overlap), "copy_mode": args.copy_mode,
                   "values": "normal(0, 1e-3)",
                   "accumulation": "fp32 add, bf16 per hop" if args.bf16_acc == "per_hop"
                   else "fp32 partials between hops, bf16 at the last hop"},
        "algbw_gbs": round(esize * count / t / 1e9, 2),
        "hbm": {"algorithmic_gbs": round(algo, 1), "frac_of_8tbs": round(algo / HBM_PEAK_GBS, 4)},
        "roofline": {"bound": "hbm", "achieved": round(red_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(red_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic() if args.bf16_acc == "per_hop" else None,
                     "kernel": "ring_hop_kernel<kReduceBf16, 2, 8>: one reduce-scatter hop, all 8 ranks, incoming operand loaded non-temporally"
                               if args.bf16_acc == "per_hop" else
                               "partial_kernel<kFirst/kMid/kLast*, 16>: the reduce-scatter hops with fp32 partials",
                     "launches": red["launches"],
                     "bytes_per_launch": red["bytes"] // max(1, red["launches"]),
                     "mean_launch_us": round(red["ms"] * 1e3 / max(1, red["launches"]), 3),
                     "by_position": by_position},
        "protocol": {"timed_region": f"{args.steps} back-to-back in-place all-reduces, host clock, "
                                     "synchronised on both sides",
                     "restored_inputs": None if restored is None else dict(
                         restored, note="inputs restored by a device copy before each step, "
                                        "outside HIP events around the step")},
        "copy_roofline": None if copy_gbs is None else {
            "gbs": round(copy_gbs, 1), "frac_of_8tbs": round(copy_gbs / HBM_PEAK_GBS, 4),
            "reduce_hop_frac_of_copy": round(red_gbs / copy_gbs, 4),
            "what": "copy kernel, one 1 GiB copy, full CUs"},
        "reduce_forward_kernel": None if not fwd["ms"] else {
            "achieved": round(fwd["bytes"] / (fwd["ms"] * 1e6), 1), "launches": fwd["launches"],
            "mean_launch_us": round(fwd["ms"] * 1e3 / max(1, fwd["launches"]), 3)},
        "sdma_copies": None if not dma["launches"] else {
            "jobs": dma["launches"], "bytes": dma["bytes"], "ms": round(dma["ms"], 4),
            "gbs": round(dma["bytes"] / (dma["ms"] * 1e6), 1) if dma["ms"] else None},
        "copy_kernel": None if cpy_gbs is None else {
            "achieved": round(cpy_gbs, 1), "launches": cpy["launches"],
            "mean_launch_us": round(cpy["ms"] * 1e3 / max(1, cpy["launches"]), 3)},
        "gemm_slowdown_pct": None if gemm is None else {
            slowdown_key(r): r["slowdown_mean_pct"] for r in gemm["runs"]
            if r["cu_budget"] == 256 and r["dma_sync"] in (None, "host_func")},
        "gemm_slowdown": gemm,
        "gemm_slowdown_all_gather_only": ag_only,
        "pp_staging_gemm_slowdown": pp,
        "cu_occupancy": occ,
        "host_us_per_call": launch,
        "other_workloads": others,
        "cpu_baseline": cpu,
        **({"errors": errors} if errors else {}),
    }
    # last, so that a tail of the output line still shows it
    line["sdma_vs_kernel"] = {k: compact_verdict(v) for k, v in (("bucket", gemm),
                                                                  ("bucket_all_gather_only", ag_only),
                                                                  ("pp_staging", pp))
                              if v is not None}
    ctx.close()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
