#!/usr/bin/env python3
"""Benchmark of the sparse-KV hot-cache decode step on one MI355X.

Metric: selected rows per second of decode steps — S*L*K rows gathered per
step — plus the gather's HBM bandwidth and the miss fetch's PCIe bandwidth.
Default workload: the full-model shape of the page "From 1M Total to 15+ ×
1M Contexts: GLM-5.3 KV Cache Offloading" — 78 layers, a selection every 4th
layer reused by the next 3, history 50,023 positions growing by one per step,
32,768 hot slots per layer, top-2,048 (sections "Separate historical capacity
from the current working set" and "Six interleaved pairs establish the
nearly lossless result").  Inputs are seeded synthetic data
(cache_gather_amd.workload), resident in HBM / pinned host RAM before timing.

One step = one hc_step call = the whole path: top-K scan and cut, lookup, LRU,
host->HBM miss fetch, gather + dequant.  W warmup steps (the first is the cold
step that fills the caches) are followed by exactly K timed steps.  The steps
run three times, each time on a fresh context over the same inputs: the first
pass has nothing but the steps inside its timed region and gives `value` and
`ms_per_step`; the second attaches HIP events to each stage's first and last
kernel dispatch and gives the per-kernel times behind `stage_us` and
`roofline`; the third, untimed, writes the trace, from which the miss counts
and the gather's own counts of the rows it moved come.

Prints one JSON line on stdout.  `roofline` is for the kernel that takes the
most time per step; `cpu_baseline` times the CPU oracle on a short prefix of
the same workload (the oracle is test infrastructure, used here only for
that baseline).
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "selected rows/s per decode step (50K hist, K=2048); gather HBM + fetch PCIe GB/s"
HBM_PEAK_GBS = 8000.0
PCIE_PEAK_GBS = 63.0      # PCIe Gen5 x16, 32 GT/s x 16 lanes x 128/130, one direction
ROW, OUT_ROW = 656, 1152


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(name):
    path = os.path.join(ROOT, "cache_gather_amd", "csrc", name)
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def traffic_from_profile(kernel_file, workload):
    """Per-launch HBM bytes measured by rocprofv3 FETCH_SIZE / WRITE_SIZE,
    from profiles/traffic_<kernel>_<workload>.md, or None if absent or taken
    on a different version of the kernel source."""
    stem = kernel_file.replace(".hip", "")
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.md" % (stem, workload))
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source_sha256_16:\s*([0-9a-f]{16})", text)
    b = re.search(r"bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not b or m.group(1) != kernel_source_hash(kernel_file):
        return None
    return float(b.group(1))


def time_oracle(wl, rows, n_steps, threads):
    """Seconds per step of the oracle on the first n_steps of the workload."""
    import numpy as np
    import oracle
    from cache_gather_amd import workload as W
    model = oracle.Model(wl.n_sessions, wl.n_layers, wl.layers_per_select, wl.top_k,
                         wl.cache_slots, wl.hcap, rows)
    sc = W.Scores(wl)
    times = []
    for t in range(n_steps):
        s = sc.step(t)
        t0 = time.perf_counter()
        model.step(t, list(s), wl.hist_len(t).astype(np.int64), gather=True, info=False,
                   nthreads=threads)
        times.append(time.perf_counter() - t0)
        log("cpu baseline (%d thread%s): step %d took %.2f s" % (
            threads, "" if threads == 1 else "s", t, times[-1]))
    model.close()
    return times


def run_cpu_baseline(wl, rows, n_steps, threads=0, single_steps=3):
    """The oracle as it stands, on the first n_steps of the workload with
    `threads` threads (0: one per selection group, at most 16, the machine's CPU
    share), and on the first single_steps steps with one thread; each rate is
    taken over the steps after step 0 (the cold fill)."""
    if threads <= 0:
        threads = max(1, min(16, os.cpu_count() or 1, wl.n_units))
    rows_per_step = wl.n_sessions * wl.n_layers * wl.top_k
    times = time_oracle(wl, rows, n_steps, threads)
    warm = times[1:] if len(times) > 1 else times
    res = {
        "value": rows_per_step * len(warm) / sum(warm),
        "unit": "rows/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "first %d decode steps of %s on %d threads (at most one per selection "
                  "group); rate over steps 1-%d, cold step 0 took %.2f s" % (
                      n_steps, wl.name, threads, n_steps - 1, times[0]),
        "nproc": os.cpu_count(),
        "cpu_model": cpu_model(),
    }
    if single_steps > 1 and threads != 1:
        t1 = time_oracle(wl, rows, single_steps, 1)
        res["single_thread"] = {
            "value": rows_per_step * (len(t1) - 1) / sum(t1[1:]),
            "unit": "rows/s", "cores": 1,
            "sample": "first %d decode steps on one thread; rate over steps 1-%d, cold step 0 "
                      "took %.2f s" % (single_steps, single_steps - 1, t1[0])}
    return res


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def copy_ceiling(torch, dev):
    """Read+write rate (GB/s) of a plain 256 MiB device-to-device copy, median
    of 5, each preceded by a read of an unrelated 1 GiB buffer: the copy starts
    with neither its source nor dirty lines in the 256 MB Infinity Cache, the
    state a gather of 1.6 GiB of slots meets."""
    n = 256 << 20
    a = torch.ones(n, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    flush = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ts = []
    for _ in range(5):
        flush.view(torch.int64).sum()
        ev[0].record()
        b.copy_(a)
        ev[1].record()
        torch.cuda.synchronize()
        ts.append(ev[0].elapsed_time(ev[1]))
    ms = sorted(ts)[2]
    del a, b, flush
    return round(2 * n / (ms * 1e-3) / 1e9, 1)


def memory_ceilings(torch, dev):
    """Reference rates of the chip's memory paths, measured with torch's own
    kernels only (so that they rest on nothing of this package): the plain
    device copy; a 64 MiB copy after 1 GiB of reads and after 1 GiB of
    ordinary stores, whose dirty lines its reads must evict from the 256 MB
    Infinity Cache; a gather of 159,744 random 704-B rows out
    of a 1.8 GB array (the slot reads of the 78-layer step, without the
    dequantisation: read and write 704 B per row); and a contiguous 256 MiB
    copy from pinned host memory.  Medians of 7, kernel time by events."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(prep, fn, reps=7):
        ts = []
        for _ in range(reps):
            prep()
            ev[0].record()
            fn()
            ev[1].record()
            torch.cuda.synchronize()
            ts.append(ev[0].elapsed_time(ev[1]) * 1e3)
        return sorted(ts)[reps // 2]

    out = {"copy_256mib_gbs": copy_ceiling(torch, dev)}
    flush = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    acc = torch.zeros((), dtype=torch.int64, device=dev)
    src = torch.ones(64 << 20, dtype=torch.uint8, device=dev)
    dst64 = torch.empty_like(src)

    def after_reads():
        acc.add_(flush.view(torch.int64).sum())

    def after_stores():
        flush.fill_(1)

    def copy64():
        dst64.copy_(src)
    us_r = timed(after_reads, copy64)
    us_w = timed(after_stores, copy64)
    out["copy_64mib_after_reads_us"] = round(us_r, 2)
    out["copy_64mib_after_stores_us"] = round(us_w, 2)
    out["copy_64mib_after_reads_gbs"] = round(2 * (64 << 20) / us_r / 1e3, 1)
    del src, dst64
    rows = torch.ones((78 * 32768, 704), dtype=torch.uint8, device=dev)
    g = torch.Generator(device="cpu").manual_seed(7)
    idx = torch.randint(0, rows.shape[0], (78 * 2048,), generator=g).to(dev)
    dst = torch.empty((idx.numel(), 704), dtype=torch.uint8, device=dev)
    us_g = timed(after_reads, lambda: torch.index_select(rows, 0, idx, out=dst))
    out["row_gather_704b_us"] = round(us_g, 2)
    out["row_gather_704b_gbs"] = round(2 * 704 * idx.numel() / us_g / 1e3, 1)
    del rows, dst, flush
    host = torch.ones(256 << 20, dtype=torch.uint8).pin_memory()
    dev_buf = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    us_h = timed(lambda: None, lambda: dev_buf.copy_(host, non_blocking=True), reps=5)
    out["host_to_device_256mib_gbs"] = round((256 << 20) / us_h / 1e3, 1)
    return out


def replacement_probe(hc, W, np, torch, reps=10):
    """The page's probe (section "GPU cache management has hazards too"): a
    full hot cache of 32,768 slots whose reference bits are all set, then one
    gather of 2,048 rows with 1% (20) misses.  Each repetition builds the
    state on a fresh context (16 steps of disjoint 2,048-position blocks fill
    every slot; fills set the bits) and times the probe step's kernels with
    HIP events.  One layer, one session, history 131,072 positions."""
    K, C, H = 2048, 32768, 131072
    wl = W.Workload("replacement_probe", 1, 1, 1, H, 17, C, K, (1.0,), (1.0,), 77)
    rows = W.fill_rows(wl, 0, 0)
    stride = (wl.hcap + 3) // 4 * 4
    dev = torch.device("cuda", 0)
    preload_kernels(hc, torch)
    blocks = torch.zeros((C // K, stride), dtype=torch.float32, device=dev)
    for t in range(C // K):
        blocks[t, t * K:(t + 1) * K] = 1.0
    rng = np.random.default_rng(3)
    probes = []
    for r in range(reps):
        x = np.zeros(stride, np.float32)
        x[np.sort(rng.choice(C, K - 20, replace=False))] = 1.0
        x[np.sort(rng.choice(np.arange(C, H), 20, replace=False))] = 1.0
        probes.append(torch.from_numpy(x).to(dev))
    out_res = {}
    for name, policy in (("lru", hc.LRU), ("circular", hc.CIRCULAR), ("clock", hc.CLOCK)):
        stage = {k: [] for k in hc.STAGES}
        misses = []
        for r in range(reps):
            cache = hc.HotCache(1, 1, 1, C, K, wl.hcap, 0, replacement=policy)
            np.copyto(cache.host_rows(0, 0), rows)
            out, sel, tr = cache.alloc_outputs(trace=True)
            for t in range(C // K):
                cache.step(blocks[t], stride, [H], out, sel)
            hc.hc_profile_enable(cache.ctx, 1)
            cache.step(probes[r], stride, [H], out, sel, tr)
            ms, n, _ = hc.hc_profile_read(cache.ctx)
            misses.append(int(tr[0, 1].item()))
            for k in hc.STAGES:
                stage[k].append(ms[k] * 1e3)
            cache.close()
        med = {k: round(float(np.median(v)), 2) for k, v in stage.items()}
        out_res[name] = {"stage_us_median": med,
                         "select_plus_gather_us": round(med["select"] + med["gather"], 2),
                         "misses": int(np.median(misses))}
    return {"metric": "replacement probe: us per 2,048-row step, full cache, all reference "
                      "bits set, 1% misses",
            "unit": "us", "higher_is_better": False, "n_gpus": 1, "reps": reps,
            "config": {"workload": "replacement_probe", "cache_slots": C, "top_k": K,
                       "history": H, "layers": 1},
            "policies": out_res,
            "page_context_w7900d": {"clock_ms": [1.03, 1.07], "circular_ms": 0.032}}


def preload_kernels(hc, torch):
    """Steps on tiny throwaway contexts — one query, two queries, and a ring
    append with its copyback — so that loading the kernels' code objects is
    not counted in the cold step."""
    for q in (1, 2):
        c = hc.HotCache(1, 1, 1, 64, 8, 64, 0, ring_rows=2, copyback_rows=1, queries=q)
        out, sel, _ = c.alloc_outputs()
        sc = torch.zeros(64 * q, dtype=torch.float32, device="cuda")
        rows = torch.zeros((1, 1, ROW), dtype=torch.uint8, device="cuda")
        c.step(sc, 64, [63], out, sel)
        c.append(rows, [63])
        c.step(sc, 64, [64], out, sel)
        torch.cuda.synchronize()
        c.close()


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--workload", default="model78_50k")
    ap.add_argument("--cpu-steps", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="threads of the CPU oracle baseline (0: one per selection group, "
                         "at most 16)")
    ap.add_argument("--cpu-single-steps", type=int, default=3,
                    help="steps of the one-thread oracle leg of the CPU baseline (0: none)")
    ap.add_argument("--cpu-only", action="store_true",
                    help="time only the CPU oracle baseline on --workload (first --cpu-steps "
                         "steps, --cpu-threads threads); no GPU work")
    ap.add_argument("--ring", type=int, default=0, metavar="ROWS",
                    help="decode with a recent ring of ROWS rows per layer: every step first "
                         "appends the new position's row of every layer, and batches of "
                         "--copyback-rows rows are copied back to host RAM")
    ap.add_argument("--copyback-rows", type=int, default=64)
    ap.add_argument("--queries", type=int, default=1, metavar="Q",
                    help="query rows per round (MTP verification: Q = MTP depth + 1); every "
                         "query selects its own top-K and the cache round runs on their union")
    ap.add_argument("--replacement-probe", action="store_true",
                    help="time the page's replacement probe instead: a full 32,768-slot hot "
                         "cache with every reference bit set, then one 2,048-row step with 1%% "
                         "misses, for LRU, circular and clock replacement")
    ap.add_argument("--ceilings", action="store_true",
                    help="print reference rates of the memory paths (device copy, a 64 MiB copy "
                         "after reads / after stores, random 704-B row gather, pinned host to "
                         "device copy), measured with torch's kernels only, and exit")
    ap.add_argument("--attend", type=int, default=0, metavar="HEADS",
                    help="follow every step with MLA decode attention of HEADS heads over the "
                         "selected rows, once through the bf16 buffer and once fused (the step "
                         "skips the buffer, attention reads the slots)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device-to-device copy (reference for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE readings)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU; runs on several GPUs are not supported "
              "(asked for --gpus %d, WORLD_SIZE=%d)" % (args.gpus, world),
              file=sys.stderr)
        sys.exit(2)
    if args.warmup < 1 or args.steps < 1:
        sys.exit("need --warmup >= 1 (the cold step) and --steps >= 1")

    if args.cpu_only:
        from cache_gather_amd import workload as W
        wl = W.ALL[args.workload]
        t0 = time.time()
        rows = W.fill_all_rows(wl)
        log("host rows generated in %.1fs" % (time.time() - t0))
        res = run_cpu_baseline(wl, rows, args.cpu_steps, args.cpu_threads, args.cpu_single_steps)
        print(json.dumps({"metric": "oracle rows/s (CPU)", "workload": wl.name,
                          "cpu_baseline": res, "ms_per_step": round(
                              wl.n_sessions * wl.n_layers * wl.top_k / res["value"] * 1e3, 2),
                          "nproc": os.cpu_count(), "cpu_model": cpu_model()}), flush=True)
        return

    import numpy as np
    import torch
    from cache_gather_amd import hc
    from cache_gather_amd import workload as W

    if args.replacement_probe:
        print(json.dumps(replacement_probe(hc, W, np, torch)), flush=True)
        return
    if args.ceilings:
        print(json.dumps({"metric": "memory ceilings", "ceilings": memory_ceilings(torch, "cuda:0")}),
              flush=True)
        return

    base = W.ALL[args.workload]
    total = args.warmup + args.steps
    wl = base.with_(steps=max(base.steps, total))
    dev = torch.device("cuda", 0)
    S, L, K, U = wl.n_sessions, wl.n_layers, wl.top_k, wl.n_units
    log("workload %s: S=%d L=%d R=%d K=%d C=%d H0=%d, %d warmup + %d timed steps" % (
        wl.name, S, L, wl.layers_per_select, K, wl.cache_slots, wl.hist0, args.warmup,
        args.steps))

    preload_kernels(hc, torch)
    t0 = time.time()
    rows = W.fill_all_rows(wl)
    log("host rows generated (%.1f GiB) in %.1fs" % (
        S * L * wl.hcap * ROW / 2 ** 30, time.time() - t0))

    # With a ring, prefill rows [0, H0 - 1) are in host RAM and step t appends
    # position H0 - 1 + t (the newest token) before it runs, so hist_len(t) is
    # the same as without a ring; the appended rows wait in HBM.
    first = wl.hist0 - 1
    d_new = None
    if args.ring:
        d_new = torch.empty((total, S, L, ROW), dtype=torch.uint8, device=dev)
        for t in range(total):
            d_new[t].copy_(torch.from_numpy(np.stack([np.stack([rows[s][l][first + t]
                                                                for l in range(L)])
                                                      for s in range(S)])))

    stride = (wl.hcap + 3) // 4 * 4
    t0 = time.time()
    scores = W.Scores(wl)
    Q = args.queries
    d_scores = torch.empty((total, U * Q, stride), dtype=torch.float32, device=dev)
    for t in range(total):
        d_scores[t].copy_(torch.from_numpy(scores.step(t, stride, queries=Q)))
    torch.cuda.synchronize()
    log("scores for %d steps resident in HBM (%.2f GiB) in %.1fs" % (
        total, d_scores.numel() * 4 / 2 ** 30, time.time() - t0))

    att = None
    if args.attend:
        import math
        d_q = torch.empty((total,) + W.queries(wl, 0, args.attend, Q).shape, dtype=torch.int16,
                          device=dev)
        for t in range(total):
            d_q[t].copy_(torch.from_numpy(W.queries(wl, t, args.attend, Q).view(np.int16)))
        att = {"heads": args.attend, "scale": 1.0 / math.sqrt(576.0), "q": d_q}

    def run_pass(kernel_events, variant=None, with_trace=False):
        """A fresh context over the same inputs: cold step, warmup, then the
        timed steps.  With kernel_events, each stage of the timed steps carries
        a pair of HIP events attached to its first and last dispatch (the
        kernels' own begin and end).  With with_trace, every step writes its
        trace (a debugging output of the ABI, from which the miss counts and
        the gather's own movement counts come; the counting adds atomics to
        the gather, so no timed pass writes one).  The pass that produces
        `value` has neither."""
        cache = hc.HotCache(S, L, wl.layers_per_select, wl.cache_slots, K, wl.hcap, 0,
                            ring_rows=args.ring,
                            copyback_rows=args.copyback_rows if args.ring else 0, queries=Q)
        for s in range(S):
            for l in range(L):
                h = cache.host_rows(s, l)
                if args.ring:
                    h[:first] = rows[s][l][:first]
                    h[first:] = 0
                else:
                    np.copyto(h, rows[s][l])
        out, sel, _ = cache.alloc_outputs()
        trace = (torch.empty((total, U, hc.trace_ints(Q * K)), dtype=torch.int32, device=dev)
                 if with_trace else None)
        append_ev = ([(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                      for _ in range(total)] if args.ring and kernel_events else None)

        if variant:
            work, att_out = cache.attention_buffers(att["heads"])

        def step(t):
            tr = trace[t] if trace is not None else None
            if variant == "fused":
                cache.step(d_scores[t], stride, wl.hist_len(t), None, sel, tr)
                cache.attend_cached(att["q"][t], att["heads"], att["scale"], work, att_out)
                return
            if variant == "buffer":
                cache.step(d_scores[t], stride, wl.hist_len(t), out, sel, tr)
                cache.attend(att["q"][t], att["heads"], att["scale"], out, work, att_out)
                return
            if args.ring:
                timed_append = append_ev is not None and t >= args.warmup
                if timed_append:
                    append_ev[t][0].record()
                cache.append(d_new[t], [first + t] * S)
                if timed_append:
                    append_ev[t][1].record()
            cache.step(d_scores[t], stride, wl.hist_len(t), out, sel, tr)

        # cold step (every row misses), then the rest of the warmup
        hc.hc_profile_enable(cache.ctx, 1)
        torch.cuda.synchronize()
        c0 = time.perf_counter()
        step(0)
        torch.cuda.synchronize()
        cold_ms = (time.perf_counter() - c0) * 1e3
        cold_stage_ms, _, _ = hc.hc_profile_read(cache.ctx)
        for t in range(1, args.warmup):
            step(t)
        # timed region: exactly --steps steps
        hc.hc_profile_enable(cache.ctx, args.steps if kernel_events else 0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(args.warmup, total):
            step(t)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        res = {"elapsed": elapsed, "cold_ms": cold_ms, "cold_stage_ms": cold_stage_ms,
               "trace": trace.cpu().numpy() if trace is not None else None,
               "last_out": out, "last_sel": sel}
        if args.ring:
            f0 = time.perf_counter()
            status, counts = cache.flush()
            res["flush_ms"] = (time.perf_counter() - f0) * 1e3
            res["flush_ok"] = status == 0 and all(int(c) == first + total for c in counts)
            if append_ev is not None:
                res["append_us"] = np.array([append_ev[t][0].elapsed_time(append_ev[t][1]) * 1e3
                                             for t in range(args.warmup, total)])
        if kernel_events:
            stage_ms, n_prof, per_step = hc.hc_profile_read(cache.ctx, args.steps)
            assert n_prof == args.steps
            res["stage_avg"] = {k: v / n_prof for k, v in stage_ms.items()}
            res["step_kernel_us"] = per_step.sum(axis=1) * 1e3
            res["gather_us"] = per_step[:, list(hc.STAGES).index("gather")] * 1e3
            res["elapsed_with_events"] = elapsed
        cache.close()
        del trace
        return res

    if att:
        res_att = {}
        for variant in ("buffer", "fused"):
            r = run_pass(False, variant)
            res_att[variant] = {"ms_per_step": round(r["elapsed"] * 1e3 / args.steps, 5)}
        heads = att["heads"]
        rows = S * L * Q * K
        flops = 2.0 * rows * heads * (576 + 512)
        for v in res_att.values():
            v["attention_tflops_incl_step"] = round(flops / (v["ms_per_step"] * 1e-3) / 1e12, 2)
        print(json.dumps({
            "metric": "decode step + MLA attention over the selected rows (ms per step)",
            "unit": "ms", "higher_is_better": False, "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "dtype": "bf16 (fp32 accumulate)", "data": "synthetic",
            "config": {"workload": wl.name, "heads": heads, "queries": Q, "top_k": K,
                       "layers": L, "attention_gflop_per_step": round(flops / 1e9, 2)},
            "variants": res_att}), flush=True)
        return
    timed = run_pass(False)
    kernels_pass = run_pass(True)
    trace_pass = run_pass(False, with_trace=True)
    elapsed = timed["elapsed"]
    cold_ms, cold_stage_ms = timed["cold_ms"], timed["cold_stage_ms"]
    stage_avg = kernels_pass["stage_avg"]
    step_kernel_us = kernels_pass["step_kernel_us"]
    # the passes ran the same steps on fresh contexts: same last selection and output
    for other in (kernels_pass, trace_pass):
        if not (torch.equal(timed["last_sel"], other["last_sel"])
                and torch.equal(timed["last_out"], other["last_out"])):
            raise SystemExit("the passes disagree")
    del timed["last_out"], kernels_pass["last_out"], trace_pass["last_out"]

    ms_per_step = elapsed * 1e3 / args.steps
    rows_per_step = S * L * Q * K       # every query row's K rows of every layer
    value = rows_per_step / (ms_per_step / 1e3)

    # misses per step from the trace (n_miss of each unit x layers of its group)
    tr = trace_pass["trace"]
    layers_of_group = np.array([min(wl.layers_per_select, L - g * wl.layers_per_select)
                                for g in range(wl.n_groups)] * S)
    miss_rows = (tr[:, :, 1] * layers_of_group[None, :]).sum(axis=1)   # per step
    timed_miss_rows = miss_rows[args.warmup:]
    fetch_bytes = float(timed_miss_rows.mean()) * ROW
    # the rows as the gather's own lanes counted them while moving them (trace
    # fields 4-7: read from host RAM, read from HBM, slot fills, output rows)
    moved = tr[args.warmup:, :, 4:8].sum(axis=1).astype(np.float64).mean(axis=0)
    gather_bytes = float(rows_per_step) * (ROW + OUT_ROW)
    hist_len_mean = float(np.mean([wl.hist0 + t for t in range(args.warmup, total)]))
    scan_bytes = U * hist_len_mean * 4   # one fp32 read per position per pass

    # The gather kernel also performs the miss fetch: its HBM bytes are the hit
    # reads + miss slot writes (656 B per row either way) + 1,152 B output per
    # row; its PCIe bytes are 656 B per missing row.  Both rates use its time.
    kernels = {
        "gather": ("k_gather.hip", "hbm", gather_bytes, HBM_PEAK_GBS, "gather"),
        "fetch": ("k_gather.hip", "pcie", fetch_bytes, PCIE_PEAK_GBS, "gather"),
        "topk_scan": ("k_topk.hip", "hbm", scan_bytes, HBM_PEAK_GBS, "topk_scan"),
        "select": ("k_select.hip", "hbm", U * (wl.cache_slots * 8 + K * 16), HBM_PEAK_GBS,
                   "select"),
    }

    # Per timed step: is the gather launch held by HBM or by PCIe?  Each step
    # goes to the resource it drives closer to its peak.
    g_us = kernels_pass["gather_us"]
    hbm_frac_step = gather_bytes / (g_us * 1e-6) / 1e9 / HBM_PEAK_GBS
    pcie_frac_step = timed_miss_rows * ROW / (g_us * 1e-6) / 1e9 / PCIE_PEAK_GBS
    regimes = {}
    for name, mask, frac in (("hbm_bound", hbm_frac_step >= pcie_frac_step, hbm_frac_step),
                             ("pcie_bound", hbm_frac_step < pcie_frac_step, pcie_frac_step)):
        if mask.any():
            peak = HBM_PEAK_GBS if name == "hbm_bound" else PCIE_PEAK_GBS
            nbytes = (gather_bytes * mask.sum() if name == "hbm_bound"
                      else float(timed_miss_rows[mask].sum()) * ROW)
            gbs = nbytes / (g_us[mask].sum() * 1e-6) / 1e9
            regimes[name] = {"steps": int(mask.sum()),
                             "gather_us_mean": round(float(g_us[mask].mean()), 2),
                             "achieved_gbs": round(gbs, 2), "frac": round(gbs / peak, 4)}

    def roofline(stage):
        src, bound, nbytes, peak, timed_as = kernels[stage]
        ms = stage_avg[timed_as]
        achieved = nbytes / (ms * 1e-3) / 1e9 if ms > 0 else 0.0
        traffic = traffic_from_profile(src, wl.name) if stage == "gather" else None
        return {"kernel": stage, "bound": bound, "achieved": round(achieved, 2),
                "peak": peak, "unit": "GB/s", "frac": round(achieved / peak, 4),
                "traffic": traffic, "algorithmic_bytes": nbytes,
                "avg_launch_us": round(ms * 1e3, 2)}

    dominant = max(stage_avg, key=stage_avg.get)
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "sessions": S, "layers": L,
                   "layers_per_select": wl.layers_per_select, "history0": wl.hist0,
                   "cache_slots": wl.cache_slots, "top_k": K,
                   "rows_per_step": rows_per_step,
                   "output": "bf16 [S][L][Q][K][576]" if Q > 1 else "bf16 [S][L][K][576]"},
        "roofline": roofline(dominant),
        "roofline_gather": roofline("gather"),
        "roofline_fetch": roofline("fetch"),
        "dominant_kernel": dominant,
        "gather_regimes": regimes,
        "stage_us": {k: round(v * 1e3, 2) for k, v in stage_avg.items()},
        "kernel_sum_us": round(sum(stage_avg.values()) * 1e3, 2),
        "kernel_timing": "HIP events attached to each stage's first and last kernel dispatch "
                         "(hipExtLaunchKernel) in a second pass over the same steps",
        "ms_per_step_with_kernel_events": round(
            kernels_pass["elapsed_with_events"] * 1e3 / args.steps, 5),
        "gather_hbm_gbs": roofline("gather")["achieved"],
        "fetch_pcie_gbs": roofline("fetch")["achieved"],
        "miss_rows_per_step": round(float(timed_miss_rows.mean()), 1),
        "moved_per_step_counted": {"host_read_bytes": round(moved[0] * ROW, 1),
                                   "hbm_read_rows": round(moved[1], 1),
                                   "slot_fill_rows": round(moved[2], 1),
                                   "output_rows": round(moved[3], 1)},
        "step_kernel_us": {"median": round(float(np.median(step_kernel_us)), 2),
                           "p99": round(float(np.percentile(step_kernel_us, 99)), 2),
                           "max": round(float(step_kernel_us.max()), 2),
                           "mean": round(float(step_kernel_us.mean()), 2)},
        "cold_step_ms": round(cold_ms, 3),
        "cold_step_kernel_us": {k: round(v * 1e3, 2) for k, v in cold_stage_ms.items()},
        "cold_step_miss_rows": int(miss_rows[0]),
        "cold_step_fetch_pcie_gbs": round(int(miss_rows[0]) * ROW / (
            cold_stage_ms["gather"] * 1e-3) / 1e9, 2),
        "cpu_baseline": None,
    }
    if Q > 1:
        result["config"]["queries"] = Q
        # fetch bytes count one PCIe read per distinct missing position; further
        # query rows of the same missing position read host RAM again
    if args.ring:
        B = args.copyback_rows
        timed_t = np.arange(args.warmup, total)
        copies = (timed_t + 1) % B == 0     # t + 1 rows appended after step t
        a_us = kernels_pass["append_us"]
        plain = float(a_us[~copies].mean()) if (~copies).any() else None
        with_copy = float(a_us[copies].mean()) if copies.any() else None
        batch_bytes = S * L * B * ROW
        result["config"]["ring_rows"] = args.ring
        result["config"]["copyback_rows"] = B
        result["recent_ring"] = {
            "append_us_mean": round(plain, 2) if plain is not None else None,
            "append_with_copyback_us": round(with_copy, 2) if with_copy is not None else None,
            "copybacks_in_timed_steps": int(copies.sum()),
            "copyback_bytes": batch_bytes,
            "copyback_pcie_write_gbs": (round(batch_bytes / ((with_copy - plain) * 1e-6) / 1e9, 2)
                                        if plain is not None and with_copy is not None else None),
            "flush_ms": round(timed["flush_ms"], 3),
            "flush_host_count_ok": bool(timed["flush_ok"] and kernels_pass["flush_ok"]),
        }
    del d_scores
    result["hbm_copy_ceiling_gbs"] = copy_ceiling(torch, dev)
    if args.calibrate_copy:
        a = torch.ones(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    if not args.no_cpu_baseline and (Q > 1 or args.ring):
        log("cpu baseline: timed only for the single-query step without a ring")
    elif not args.no_cpu_baseline:
        log("cpu baseline: oracle on the first %d steps ..." % args.cpu_steps)
        result["cpu_baseline"] = run_cpu_baseline(wl, rows, args.cpu_steps, args.cpu_threads,
                                                  args.cpu_single_steps)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
