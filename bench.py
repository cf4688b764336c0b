#!/usr/bin/env python3
"""Bench of the per-GPU reduction hot path on one MI355X.

Headline (`value`): achieved HBM GB/s of the two-stage reduce at the 8 MB
message cap, W=8 rank buffers of 4,194,304 bf16, as run by one rank
(reduce-scatter of its 1/8 shard + all-gather of all 8 shards), with all
buffers resident in HBM and rotated over enough buffer sets that every launch
reads from HBM rather than the 256 MB Infinity Cache.  One step = one launch.

Timing: K launches are captured in a HIP graph (no host launch overhead in
the timed region) and replayed between two HIP events on the launch stream;
ms_per_step = elapsed / K.  The same events time every other row of the hot
path (one-stage reduce, fused all-reduce + residual + RMSNorm, LL / LL128
pack and decode, Lamport, two-shot fused, streaming), reported under "rows"
as the median over 5 replays with their coefficient of variation (a row
above 5 % is timed again, then flagged); the fused M=1 latency is also
reported per call.

`roofline.traffic` comes from the rocprofv3 counter summary committed under
profiles/ (FETCH_SIZE + WRITE_SIZE per dispatch, scaled by a plain copy of
known size) and is null when the kernel source changed since it was taken.

`cpu_baseline` times the CPU oracle (plain C) on the same per-rank two-stage
work: single-threaded for about 10 s, then on every host core of this GPU's
share at once (up to 16 threads, each doing whole steps) for about 3 s; the
all-core aggregate is `value`, the single-thread rate `single_core`.

Context row: the launch floor (a one-pack reduce).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
                       [--rows all|none|stream|wire|sets] [--eager] [--calib-copy] [--warm]
                       [--trace-summary DIR]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("achieved HBM GB/s (% of peak) for W=8 8MB reduce; "
          "µs/call M=1 fused AR+RMSNorm")
HBM_PEAK_GBPS = 8000.0
MALL_BYTES = 256 << 20
# The W rank buffers (and staging buffers) of one set are carved from one
# allocation with this gap after each, so that the W streams read at the same
# offset do not all start at addresses equal modulo 32 KiB, which on one
# MI355X puts them on the same HBM channels (on W real GPUs they would sit in
# W different HBMs).
RANK_GAP = 4096 + 512
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "reduce_2stage_w8_8MiB_counters.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "ar_rmsnorm_amd", "csrc", f)
                  for f in ("reduce.hip", "device.h", "index_map.h")]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10,
                   help="headline steps timed; a step is one call on each rotated buffer set")
    p.add_argument("--warmup", type=int, default=2, help="untimed headline steps first")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--rows", choices=["all", "none", "stream", "wire", "sets"], default="all",
                   help="which rows besides the headline: all, none, or only the streaming, "
                        "the wire-format or the rotated-set rows")
    p.add_argument("--eager", action="store_true",
                   help="time eager launches instead of a HIP graph replay")
    p.add_argument("--calib-copy", action="store_true",
                   help="also run a plain 256 MiB device copy (counter calibration)")
    p.add_argument("--trace-summary", metavar="DIR",
                   help="no GPU work: summarize the rocprofv3 kernel trace (kernel_trace.csv) "
                        "under DIR per kernel and launch shape, and the back-to-back spacing "
                        "of the headline kernel's dispatches")
    p.add_argument("--counter-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="no GPU work: HBM bytes per dispatch from two rocprofv3 --pmc runs "
                        "(FETCH_SIZE, then WRITE_SIZE) of a bench run with --calib-copy, scaled "
                        "by what each counter reads for the trailing 256 MiB copies")
    p.add_argument("--warm", action="store_true",
                   help="also time the headline call on one reused buffer set (its bytes "
                        "then come from the Infinity Cache); off by default so that a "
                        "kernel trace of the bench holds only the cold headline launches")
    return p.parse_args()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(source_hash: str):
    """HBM bytes per launch from the committed counter summary, or None."""
    try:
        text = open(PROFILE_COUNTERS).read()
    except OSError:
        return None
    m = re.search(r"^source_hash:\s*(\S+)", text, re.M)
    t = re.search(r"^hbm_bytes_per_launch:\s*([0-9.]+)", text, re.M)
    if not m or not t or m.group(1) != source_hash:
        return None
    return float(t.group(1))


TRACE_SUMMARY = os.path.join(ROOT, "profiles", "hot_path_kernel_trace.txt")


def profiled_headline(source_hash: str, nbytes: int):
    """The headline kernel's per-dispatch durations from the committed kernel
    trace of the driver's command (written by --trace-summary), while the
    kernel sources still hash to the value recorded there."""
    try:
        text = open(TRACE_SUMMARY).read()
    except OSError:
        return None
    m = re.search(r"^reduce kernel sources hash: (\S+)", text, re.M)
    if not m or m.group(1) != source_hash:
        return None
    vals = {}
    for key in ("headline_dispatch_mean_us", "headline_dispatch_median_us",
                "headline_dispatches"):
        t = re.search(rf"^{key}: ([\d.]+)", text, re.M)
        if not t:
            return None
        vals[key] = float(t.group(1))
    n = int(vals["headline_dispatches"])
    med, mean = vals["headline_dispatch_median_us"], vals["headline_dispatch_mean_us"]
    return {"source": "profiles/hot_path_kernel_trace.txt", "dispatches": n,
            "median_us": med, "mean_us": mean,
            "frac_from_mean": round(nbytes / (mean * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "note": "per-dispatch durations under rocprofv3, which starts no dispatch "
                    "before the previous one's traced end"}


WIRE_COUNTERS = os.path.join(ROOT, "profiles", "wire_16Mi_counters.txt")


def wire_traffic():
    """Scaled HBM bytes per dispatch of the wire kernels from the committed
    counter summary (written by --counter-summary), keyed by (kernel, grid
    lanes); empty when the kernel sources changed since it was taken."""
    try:
        text = open(WIRE_COUNTERS).read()
    except OSError:
        return {}
    m = re.search(r"^kernel sources sha256\[:16\]: (\S+)", text, re.M)
    if not m or m.group(1) != all_source_hash():
        return {}
    out = {}
    for line in text.splitlines():
        t = re.match(r"\s*\d+\s+\d+\s+[\d.]+\s+[\d.]+\s+(\d+)\s+\S+\s+\S+\s+(ar::.+?) "
                     r"\[(\d+), \d+\] #\d+$", line)
        if t:
            out.setdefault((t.group(2), int(t.group(3))), float(t.group(1)))
    return out


def trace_summary(d: str) -> str:
    """Per-dispatch statistics from a rocprofv3 --kernel-trace CSV: for every
    kernel and launch shape the dispatch count and the median, mean, min,
    P5, P95, max and coefficient of variation of the durations (end - start);
    then, for the headline kernel, the spacing of dispatches that follow one
    another directly: start-to-start interval, duration, and the gap from one
    dispatch's end to the next one's start."""
    import csv
    import glob
    import numpy as np
    import gzip
    files = (glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
             + glob.glob(os.path.join(d, "**", "*kernel_trace.csv.gz"), recursive=True))
    if not files:
        raise SystemExit(f"bench.py: no kernel_trace.csv under {d}")
    recs = []
    for f in files:
        with (gzip.open(f, "rt") if f.endswith(".gz") else open(f)) as fh:
            recs += list(csv.DictReader(fh))
    groups = {}
    for r in recs:
        name = r["Kernel_Name"]
        name = name[5:] if name.startswith("void ") else name
        key = (name.split("(")[0][:80], r["Grid_Size_X"], r["Grid_Size_Y"],
               r["Workgroup_Size_X"])
        groups.setdefault(key, []).append(
            (int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    out = ["per kernel of the library and launch shape: dispatches, then duration statistics "
           "in us (median, mean, min, P5, P95, max) and the coefficient of variation",
           "%6s %9s %9s %8s %8s %9s %9s %6s  %s" % ("n", "median", "mean", "min", "p5", "p95",
                                                   "max", "cv", "kernel [grid x, grid y, wg]")]
    stats = {}
    for key, v in groups.items():
        a = np.array([(e - b) / 1000.0 for b, e in v])
        stats[key] = a
    for key, a in sorted(stats.items(), key=lambda kv: -np.median(kv[1])):
        if not key[0].startswith("ar::"):
            continue            # the library's kernels only (torch's fills and copies stage)
        out.append("%6d %9.3f %9.3f %8.3f %8.3f %9.3f %9.3f %6.3f  %s [%s, %s, %s]" % (
            len(a), np.median(a), a.mean(), a.min(), np.percentile(a, 5),
            np.percentile(a, 95), a.max(), a.std() / a.mean(), *key))
    # The headline's own dispatches: the first uninterrupted run of the
    # two-stage W=8 kernel's most frequent launch shape in start order (the
    # bench times the headline first; later rows with the same shape, such
    # as the rotated-set sweep, come after other kernels).  Their duration
    # statistics, and the spacing of directly consecutive pairs.
    allv = sorted((b, e, key) for key, v in groups.items() for b, e in v)
    cand = [k for k in groups if "reduce_2stage_kernel<8, true, true" in k[0]]
    head = sorted(cand, key=lambda k: -len(groups[k]))[:1]
    for hk in head:
        seg, started = [], False
        for b, e, k in allv:
            if k == hk:
                seg.append((b, e))
                started = True
            elif started and "ar::" in k[0]:
                break
        du = np.array([(e - b) / 1000.0 for b, e in seg])
        iv = np.array([(b1 - b0) / 1000.0 for (b0, _), (b1, _) in zip(seg, seg[1:])])
        gp = np.array([(b1 - e0) / 1000.0 for (_, e0), (b1, _) in zip(seg, seg[1:])])
        out.append("")
        out.append(f"headline dispatches {hk[0]} [{hk[1]}, {hk[2]}, {hk[3]}]: the first "
                   f"uninterrupted run of that shape, {len(seg)} dispatches (us)")
        out.append("  %-24s median %8.3f  mean %8.3f  min %8.3f  p5 %8.3f  p95 %8.3f  max %8.3f"
                   "  cv %6.3f" % ("duration", np.median(du), du.mean(), du.min(),
                                   np.percentile(du, 5), np.percentile(du, 95), du.max(),
                                   du.std() / du.mean()))
        for name, a in (("start-to-start interval", iv), ("end-to-next-start gap", gp)):
            if len(a):
                out.append("  %-24s median %8.3f  mean %8.3f  p5 %8.3f  p95 %8.3f" % (
                    name, np.median(a), a.mean(), np.percentile(a, 5), np.percentile(a, 95)))
        out.append(f"headline_dispatch_mean_us: {du.mean():.3f}")
        out.append(f"headline_dispatch_median_us: {np.median(du):.3f}")
        out.append(f"headline_dispatches: {len(seg)}")
    return "\n".join(out)


ALL_SOURCES = [os.path.join(ROOT, "ar_rmsnorm_amd", "csrc", f)
               for f in ("reduce.hip", "wire.hip", "stream.hip", "copy.hip", "device.h",
                         "index_map.h", "stream_plan.h")]


def all_source_hash() -> str:
    h = hashlib.sha256()
    for f in ALL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def algorithmic_bytes():
    """What a launch must move, by (kernel, grid lanes), for the kernels the
    counter runs cover: the headline (the method's bytes and the bytes the
    kernel moves), the wire formats at 16 Mi (+13) fp32, W=4, and the plain
    copy."""
    n, W = 4_194_304, 8
    shard = n // 8 // W * 16
    out = {("ar::reduce_2stage_kernel<8, true, true, 256, 1, 2>", 256 * 256 + 7 * 128 * 256):
           (W * shard + 2 * shard + 2 * (W - 1) * shard, "moved; the method's count is "
            f"{(3 * W + 1) * shard}")}
    for nn in (16_777_216, 16_777_229):
        ll, l128 = -(-4 * nn // 8), -(-4 * nn // 120)
        out[("ar::ll_unpack_reduce_kernel<4>", -(-ll // 128) * 128)] = (4 * ll * 16 + 4 * nn, "")
        out[("ar::ll128_unpack_reduce_kernel<4>", -(-8 * l128 // 256) * 256)] = (
            4 * l128 * 128 + 4 * nn, "")
        out[("ar::ll_pack_kernel", -(-ll // 256) * 256)] = (4 * nn + ll * 16, "")
        out[("ar::ll128_pack_kernel", -(-16 * ((l128 + 1) // 2) // 256) * 256)] = (
            4 * nn + l128 * 128, "")
    for mib in (12, 256):
        out[("ar::copy_kernel", (mib << 20) // 16)] = (2 * (mib << 20), "")
    return out


def counter_summary(fetch_dir: str, write_dir: str) -> str:
    """HBM bytes per dispatch of every kernel and grid in two rocprofv3 --pmc
    runs (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each counter scaled
    by its reading for the run's last three dispatches, plain 256 MiB copies
    of the library's copy kernel (262,144 KiB read + 262,144 KiB written)."""
    import csv
    import glob
    import numpy as np

    def load(d):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"bench.py: no counter_collection.csv under {d}")
        recs = []
        for f in files:
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    name = r["Kernel_Name"]
                    name = (name[5:] if name.startswith("void ") else name).split("(")[0]
                    recs.append((int(r["Dispatch_Id"]), name, int(r["Grid_Size"]),
                                 int(r["Workgroup_Size"]), float(r["Counter_Value"])))
        recs.sort()
        return recs

    f, w = load(fetch_dir), load(write_dir)
    kib = 256 * 1024
    cal_f = [x[4] for x in f if x[1] == "ar::copy_kernel" and x[2] == (256 << 20) // 16][-3:]
    cal_w = [x[4] for x in w if x[1] == "ar::copy_kernel" and x[2] == (256 << 20) // 16][-3:]
    if len(cal_f) < 3 or len(cal_w) < 3:
        raise SystemExit("bench.py: the runs end without the three calibration copies "
                         "(run the bench with --calib-copy)")
    sf, sw = kib / float(np.mean(cal_f)), kib / float(np.mean(cal_w))

    def groups(d):
        # per launch shape, split into segments: runs of that shape not
        # interrupted by another kernel of the library (each bench row's
        # dispatches form one; an eager bench run also starts every timed
        # row with a one-workgroup copy, which ends the previous row's run
        # and is left out of the table), labelled #1, #2, ... in dispatch
        # order
        g, last, seen = {}, None, {}
        for _, name, grid, wg, v in d[:-3]:
            key = (name, grid, wg)
            if not name.startswith("ar::"):
                continue
            if name == "ar::copy_kernel" and grid == 256:
                last = None
                continue
            if key != last:
                seen[key] = seen.get(key, 0) + 1
                last = key
            g.setdefault((name, grid, wg, seen[key]), []).append(v)
        return g

    gf, gw = groups(f), groups(w)
    alg = algorithmic_bytes()
    out = [f"kernel sources sha256[:16]: {all_source_hash()}",
           f"calibration (last three 256 MiB copies): FETCH_SIZE KiB "
           f"{[round(x, 1) for x in cal_f]} -> scale {sf:.4f}; WRITE_SIZE KiB "
           f"{[round(x, 1) for x in cal_w]} -> scale {sw:.4f}",
           "%6s %6s %12s %12s %14s %14s %8s  %s" % ("n(f)", "n(w)", "fetch MiB", "write MiB",
                                                   "scaled bytes", "algorithmic", "ratio",
                                                   "kernel [grid lanes, wg]")]
    head = None
    for key in sorted(gf, key=lambda k: (k[0], k[1], k[3])):
        name, grid, wg, seg = key
        if key not in gw:
            continue
        fb = float(np.mean(gf[key])) * sf * 1024
        wb = float(np.mean(gw[key])) * sw * 1024
        a = alg.get((name, grid))
        out.append("%6d %6d %12.2f %12.2f %14.0f %14s %8s  %s [%d, %d] #%d" % (
            len(gf[key]), len(gw[key]), fb / 2 ** 20, wb / 2 ** 20, fb + wb,
            a[0] if a else "-", f"{(fb + wb) / a[0]:.4f}" if a else "-", name, grid, wg, seg))
        if name.startswith("ar::reduce_2stage_kernel<8, true, true") and a and head is None:
            head = (fb + wb, a)
    if head:
        out += ["", f"source_hash: {kernel_source_hash()}",
                f"hbm_bytes_per_launch: {head[0]:.0f}",
                f"headline traffic / bytes moved: {head[0] / head[1][0]:.4f} ({head[1][1]})"]
    return "\n".join(out)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def log(msg: str) -> None:
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.trace_summary:
        print(trace_summary(args.trace_summary))
        return
    if args.counter_summary:
        print(counter_summary(*args.counter_summary))
        return
    if args.gpus != 1:
        print(f"bench.py: libar runs on one GPU only; --gpus {args.gpus} is not "
              "supported (the W rank buffers all live in one GPU's HBM)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    if not torch.cuda.is_available():
        raise SystemExit("bench.py: no GPU visible")
    from ar_rmsnorm_amd import libar as ar
    from ar_rmsnorm_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    marker = []

    def row_marker():
        """One 16-byte library copy (a one-workgroup copy_kernel dispatch)
        ahead of every eagerly timed row, so that a counter summary can tell
        apart consecutive rows that share a launch shape."""
        if not marker:
            marker.extend(torch.zeros(2, 4, dtype=torch.int32, device=dev).unbind(0))
        ar.ar_copy(marker[0], marker[1])

    def graph_time(fns, steps, warmup):
        """Average ms per call of the calls fns[i % len(fns)], timed over a
        HIP graph of `steps` back-to-back launches replayed between events."""
        if args.eager:
            row_marker()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(max(warmup, len(fns))):
                fns[i % len(fns)]()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        if args.eager:
            start = torch.cuda.Event(enable_timing=True)
            stop = torch.cuda.Event(enable_timing=True)
            start.record()
            for i in range(steps):
                fns[i % len(fns)]()
            stop.record()
            stop.synchronize()
            return start.elapsed_time(stop) / steps
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                fns[i % len(fns)]()
        g.replay()                     # warm the graph itself
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        start.record()
        g.replay()
        stop.record()
        stop.synchronize()
        ms = start.elapsed_time(stop) / steps
        del g
        return ms

    def graph_time_stats(fns, steps, warmup, extra=10):
        """graph_time for the timed `steps` launches, then `extra` further
        replays of the same graph, each timed on its own, for the spread:
        returns (ms per launch of the timed replay, per-replay ms per launch)."""
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(max(warmup, len(fns))):
                fns[i % len(fns)]()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                fns[i % len(fns)]()
        g.replay()                     # warm the graph itself
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(extra + 2)]
        ev[0].record()
        g.replay()
        ev[1].record()
        for r in range(extra):
            g.replay()
            ev[r + 2].record()
        ev[-1].synchronize()
        ms = ev[0].elapsed_time(ev[1]) / steps
        each = [ev[r + 1].elapsed_time(ev[r + 2]) / steps for r in range(extra)]
        del g
        return ms, each

    def rank_buffers(count, nbytes, dtype, fill=None, gap=RANK_GAP):
        """`count` buffers of `nbytes` each, `gap` bytes apart in one
        allocation (fill[i] copied into buffer i when given)."""
        stride = -(-nbytes // 256) * 256 + gap
        arena = torch.empty(count * stride + 4096, dtype=torch.uint8, device=dev)
        start = (-arena.data_ptr()) % 4096
        bufs = [arena[start + i * stride: start + i * stride + nbytes].view(dtype)
                for i in range(count)]
        if fill is not None:
            for b, f in zip(bufs, fill):
                b.copy_(f.view(-1))
        return bufs

    def sets_for(touched_bytes):
        """Buffer sets so that one rotation touches > 2x the Infinity Cache."""
        return max(2, -(-2 * MALL_BYTES // max(touched_bytes, 1)) + 1)

    # ------------------------------------------------------------------
    # headline: two-stage reduce, W=8 x 8 MiB, per rank (rank 0: RS + AG)
    # ------------------------------------------------------------------
    cfg = synth.REDUCE_CAP
    W, n = cfg["W"], cfg["n"]
    xs = synth.reduce_cap()
    P = n // 8
    part, rem = P // W, P % W
    shard = part * 16
    # algorithmic bytes of one rank's call, as the method states it: RS reads
    # the W slices of its shard and writes the shard to tmp; AG reads all W
    # staged shards and writes them to out.  The kernel moves one shard less
    # each way (its own shard goes from registers to out): moved_bytes.
    bytes_2stage = W * shard + shard + W * shard + W * shard
    moved_2stage = W * shard + 2 * shard + (W - 1) * shard + (W - 1) * shard
    nsets = sets_for(moved_2stage)
    base = [to_dev(x) for x in xs]
    sets = []
    for k in range(nsets):
        ins = rank_buffers(W, 2 * n, torch.int16, base)
        tmps = rank_buffers(W, (part + rem) * 16, torch.int16)
        out = torch.empty(n, dtype=torch.int16, device=dev)
        for r in range(1, W):               # the peers' shards, staged untimed
            ar.ar_reduce_2stage(ins, tmps, r, None, flags=ar.AR_STAGE_RS)
        sets.append((ins, tmps, out))
    torch.cuda.synchronize()
    calls = [(lambda s=s: ar.ar_reduce_2stage(s[0], s[1], 0, s[2])) for s in sets]
    # one step = the call on each of the nsets cold buffer sets (a batch of
    # nsets messages); --steps K steps are timed as K * nsets launches
    steps = max(1, args.steps)
    launches = steps * nsets
    log(f"two-stage W=8 8MiB: {nsets} buffer sets staged; {args.warmup} warm-up steps, "
        f"timing {steps} steps = {launches} launches")
    if args.eager:
        ms_launch = graph_time(calls, launches, args.warmup * nsets)
        each = [ms_launch]
    else:
        ms_launch, each = graph_time_stats(calls, launches, args.warmup * nsets)
    ms = ms_launch * nsets                  # per step
    gbps = bytes_2stage / (ms_launch * 1e-3) / 1e9
    log(f"two-stage: {ms_launch * 1e3:.3f} us/launch, {gbps:.1f} GB/s "
        f"({moved_2stage / (ms_launch * 1e-3) / 1e9:.1f} GB/s moved)")
    us = np.sort(np.array(each) * 1e3)
    stats = {
        "spread_over": f"{len(us)} further replays of the timed graph of {launches} launches, "
                       "us per launch",
        "median_us": round(float(np.median(us)), 3),
        "p5_us": round(float(np.percentile(us, 5)), 3),
        "p95_us": round(float(np.percentile(us, 95)), 3),
        "min_us": round(float(us[0]), 3), "max_us": round(float(us[-1]), 3),
        "cv": round(float(np.std(us) / np.mean(us)), 4),
    }
    log(f"two-stage per-replay: {stats}")
    src_hash = kernel_source_hash()
    traffic = traffic_from_profile(src_hash)
    # the per-launch floor on this device, measured the same way: a one-stage
    # reduce of a single 16-byte pack, launched back to back in a graph
    fd = [to_dev(x[:8]) for x in synth.reduce_small()]
    fo = torch.empty_like(fd[0])
    floor_ms = graph_time([lambda: ar.ar_reduce_1stage(fd, fo)], 200, args.warmup)
    above = ms_launch - floor_ms
    log(f"launch floor {floor_ms * 1e3:.3f} us; headline above it: {above * 1e3:.3f} us")

    result = {
        "metric": METRIC,
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "storage_dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "two-stage reduce at the 8 MB cap: W=8 rank buffers of "
                        "4,194,304 bf16 ~U(-1,1), one rank's reduce-scatter of its 1/8 "
                        "shard + all-gather of the 8 shards, HBM-resident, cold",
            "W": W, "n": n,
            "step": f"one call on each of {nsets} rotated buffer sets ({nsets} launches)",
            "launches_per_step": nsets,
            "launches_timed": launches,
            "us_per_launch": round(ms_launch * 1e3, 3),
            "bytes_per_launch": bytes_2stage,
            "bytes_moved_per_launch": moved_2stage,
            "layout": f"per set, the 8 inputs and the 8 staging shards each in one "
                      f"allocation, {RANK_GAP} B apart",
            "buffer_sets_rotated": nsets,
        },
        "pct_of_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "timing_stats": stats,
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(gbps / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "kernel": "reduce_2stage_kernel<8,true,true,256,1,2>",
            "kernel_us": round(ms_launch * 1e3, 3),
            "kernel_us_timer": "HIP events around the graph replay on the launch stream, "
                               "divided by the launches it holds",
            "bytes_per_launch": bytes_2stage,
            "bytes_moved_per_launch": moved_2stage,
            "achieved_moved": round(moved_2stage / (ms_launch * 1e-3) / 1e9, 1),
            "source_hash": src_hash,
            "profiled": profiled_headline(src_hash, bytes_2stage),
            "launch_floor_us": round(floor_ms * 1e3, 3),
            "achieved_above_launch_floor": round(bytes_2stage / (above * 1e-3) / 1e9, 1)
            if above > 0 else None,
            "note": "achieved = the method's bytes per launch (26,214,400) / us per launch; "
                    "achieved_moved counts the bytes the kernel moves (own shard not "
                    "re-read); achieved_above_launch_floor divides the method's bytes by "
                    "the time above a one-pack launch",
        },
    }
    # the same call on one buffer set, launch after launch: its 24 MiB stay in
    # the 256 MB Infinity Cache, so this is a cache rate, not HBM bandwidth
    warm_ms = graph_time(calls[:1], launches, args.warmup) if args.warm else None
    del sets, calls
    torch.cuda.empty_cache()

    # ------------------------------------------------------------------
    # the other rows of the hot path
    # ------------------------------------------------------------------
    rows = {}
    if warm_ms is not None:
        rows["2stage_W8_n4194304_per_rank_warm"] = {
            "us_per_call": round(warm_ms * 1e3, 3), "bytes": bytes_2stage,
            "GBps": round(bytes_2stage / (warm_ms * 1e-3) / 1e9, 1),
            "note": "one buffer set reused: served from the Infinity Cache, not HBM"}
        log(f"row 2stage_W8_n4194304_per_rank_warm: {warm_ms * 1e3:.3f} us")

    def row(name, nbytes, fns, steps=None, extra=None, oracle_fn=None):
        """Time one row on the GPU: the median over 5 replays of a graph of
        back-to-back calls, with the replays' coefficient of variation; a row
        whose CV exceeds 5 % is timed once more and flagged if it still does.
        With the CPU leg on, also time the oracle doing the same work
        (repeated until ~0.3 s, single-threaded)."""
        # at least 40 launches per replay, so the 5 timed replays hold >= 200
        # dispatches (the per-dispatch statistics come from the kernel trace)
        k = max(steps or 60, 40)
        k = -(-k // len(fns)) * len(fns)
        if args.eager:
            t, cv, reruns = graph_time(fns, k, args.warmup), None, 0
        else:
            for reruns in range(2):
                first, each = graph_time_stats(fns, k, args.warmup, extra=4)
                reps = np.array([first] + each)
                t, cv = float(np.median(reps)), float(np.std(reps) / np.mean(reps))
                if cv <= 0.05:
                    break
        r = {"us_per_call": round(t * 1e3, 3), "bytes": nbytes,
             "GBps": round(nbytes / (t * 1e-3) / 1e9, 1),
             "frac_hbm": round(nbytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
        if cv is not None:
            r["cv_over_5_replays"] = round(cv, 4)
            if cv > 0.05:
                r["cv_flag"] = f"CV above 5 % after {reruns + 1} timings"
        if extra:
            r.update(extra)
        if oracle_fn is not None and not args.no_cpu:
            reps, t0 = 0, time.perf_counter()
            while True:
                oracle_fn()
                reps += 1
                el = time.perf_counter() - t0
                if el >= 0.3 or reps >= 50:
                    break
            r["oracle_ms"] = round(el / reps * 1e3, 3)
            r["oracle_GBps"] = round(nbytes * reps / el / 1e9, 3)
        rows[name] = r
        log(f"row {name}: {r['us_per_call']} us, {r['GBps']} GB/s"
            + (f"; oracle {r['oracle_ms']} ms" if "oracle_ms" in r else ""))
        return r

    orc = None
    if not args.no_cpu:
        import oracle as orc

    if args.rows == "all":
        # fused all-reduce + residual + RMSNorm, W=4, N=2048, M in {1, 16, 128}
        fc = synth.FUSED
        for M in fc["Ms"]:
            fx, fr, fw = synth.fused(M)
            nb = (fc["W"] + 3) * M * fc["N"] * 2 + 2 * fc["N"]
            d = [to_dev(x) for x in fx]
            dr, dw = to_dev(fr), to_dev(fw)
            ro = torch.empty_like(dr)
            no = torch.empty_like(dr)
            call = (lambda d=d, dr=dr, dw=dw, ro=ro, no=no:
                    ar.ar_fused_residual_rmsnorm(d, dr, dw, ro, no, fc["eps"]))
            row(f"fused_W4_M{M}_N2048", nb, [call], steps=200,
                oracle_fn=orc and (lambda fx=fx, fr=fr, fw=fw:
                                   orc.fused_residual_rmsnorm(fx, fr, fw, fc["eps"])))
        result["fused_m1_us_per_call"] = rows["fused_W4_M1_N2048"]["us_per_call"]

        # Lamport data-as-flag form of the same operator: rank 0's push into
        # the W comm buffers, rank 0's reader (the peers' pushes staged once),
        # and the whole per-rank call (push then read).  A repeated call with
        # one flag is idempotent: it rewrites and rereads one region and
        # resets another.
        for M in fc["Ms"]:
            fx, fr, fw = synth.fused(M)
            Wf, N = fc["W"], fc["N"]
            d = [to_dev(x) for x in fx]
            dr, dw = to_dev(fr), to_dev(fw)
            ro, no = torch.empty_like(dr), torch.empty_like(dr)
            comms = [torch.empty(ar.ar_lamport_comm_bytes(Wf, M, N) // 4, dtype=torch.int32,
                                 device=dev) for _ in range(Wf)]
            for c in comms:
                ar.ar_lamport_fill(c, Wf, M, N)
            for r in range(Wf):
                ar.ar_lamport_push(d[r], r, comms, 1)
            mat = M * N * 2
            push = (lambda d=d, comms=comms: ar.ar_lamport_push(d[0], 0, comms, 1))
            read = (lambda comms=comms, dr=dr, dw=dw, ro=ro, no=no:
                    ar.ar_lamport_fused_residual_rmsnorm(comms[0], Wf, dr, dw, ro, no,
                                                         fc["eps"], 1))
            hc = None
            if orc:
                hc = [orc.lamport_comm(Wf, M, N) for _ in range(Wf)]
                for r in range(Wf):
                    orc.lamport_push(fx[r], r, hc, 1)
            row(f"lamport_push_W4_M{M}_N2048", mat + Wf * mat, [push], steps=200,
                oracle_fn=orc and (lambda fx=fx, hc=hc: orc.lamport_push(fx[0], 0, hc, 1)))
            row(f"lamport_read_W4_M{M}_N2048", Wf * mat + 2 * mat + 2 * N + 2 * mat + Wf * mat,
                [read], steps=200,
                oracle_fn=orc and (lambda hc=hc, fr=fr, fw=fw:
                                   orc.lamport_fused_residual_rmsnorm(hc[0], Wf, fr, fw,
                                                                      fc["eps"], 1)))
            # the whole per-rank call in one launch: push to the W buffers,
            # poll the W - 1 peer slots, reduce, normalise, reset
            oneshot = (lambda d=d, comms=comms, dr=dr, dw=dw, ro=ro, no=no:
                       ar.ar_lamport_oneshot_residual_rmsnorm(d[0], 0, comms, dr, dw, ro, no,
                                                              fc["eps"], 1))
            row(f"lamport_oneshot_W4_M{M}_N2048",
                mat + Wf * mat + (Wf - 1) * mat + mat + 2 * N + 2 * mat + Wf * mat,
                [oneshot], steps=200)
            del comms
        result["lamport_m1_us_per_call"] = rows["lamport_oneshot_W4_M1_N2048"]["us_per_call"]

        # the Lamport exchange of all W ranks in one launch: each rank's reader
        # polls slots that other workgroups of the launch are still pushing,
        # so the re-read path is timed.  Flags run through 0..5 (a multiple of
        # 3), so every graph replay finds its regions reset as a live run would.
        for M in fc["Ms"]:
            fx, fr, fw = synth.fused(M)
            Wf, N = fc["W"], fc["N"]
            d = [to_dev(x) for x in fx]
            dr, dw = to_dev(fr), to_dev(fw)
            ros = [torch.empty_like(dr) for _ in range(Wf)]
            nos = [torch.empty_like(dr) for _ in range(Wf)]
            comms = [torch.empty(ar.ar_lamport_comm_bytes(Wf, M, N) // 4, dtype=torch.int32,
                                 device=dev) for _ in range(Wf)]
            for c in comms:
                ar.ar_lamport_fill(c, Wf, M, N)
            bad = torch.zeros(1, dtype=torch.int32, device=dev)
            mat = M * N * 2
            calls = [(lambda f=f, d=d, comms=comms, dr=dr, dw=dw, ros=ros, nos=nos, bad=bad:
                      ar.ar_lamport_all_ranks_residual_rmsnorm(d, comms, dr, dw, ros, nos,
                                                               fc["eps"], f, ar.AR_MAX_SPINS,
                                                               bad)) for f in range(6)]
            r = row(f"lamport_all_ranks_W4_M{M}_N2048",
                    Wf * (mat + Wf * mat + (Wf - 1) * mat + mat + 2 * mat + Wf * mat) + 2 * N,
                    calls, steps=60)
            torch.cuda.synchronize()
            r["bad_chunks"] = int(bad.item())
            r["note"] = ("the W ranks' one-launch calls as one launch of M x W workgroups; "
                         "bytes = per rank: its rows, the W pushes, W - 1 peer slots, the "
                         "residual, two outputs, the W-slot reset")
            del comms

        # the grid of shapes the fused operator's source page benchmarks
        # (M in {1, 8, 128} x N in {2048, 4096, 8192}, W=4, the same buffers
        # every call as in its CUDA-graph replays): the one-shot fused call
        # and the one-launch Lamport call, median of 5 graph replays each
        def med_us(fns, steps=200):
            if args.eager:
                return round(graph_time(fns, steps, args.warmup) * 1e3, 3)
            first, each = graph_time_stats(fns, steps, args.warmup, extra=4)
            return round(float(np.median([first] + each)) * 1e3, 3)

        grid = {}
        for N in (2048, 4096, 8192):
            for M in (1, 8, 128):
                Wf = fc["W"]
                gx, gr, gw = synth.fused_inputs(Wf, M, N, [1000 + fc["id"], M, N])
                d = [to_dev(x) for x in gx]
                dr, dw = to_dev(gr), to_dev(gw)
                ro, no = torch.empty_like(dr), torch.empty_like(dr)
                comms = [torch.empty(ar.ar_lamport_comm_bytes(Wf, M, N) // 4,
                                     dtype=torch.int32, device=dev) for _ in range(Wf)]
                for c in comms:
                    ar.ar_lamport_fill(c, Wf, M, N)
                for r in range(Wf):
                    ar.ar_lamport_push(d[r], r, comms, 1)
                one = med_us([lambda d=d, dr=dr, dw=dw, ro=ro, no=no:
                              ar.ar_fused_residual_rmsnorm(d, dr, dw, ro, no, fc["eps"])])
                lam = med_us([lambda d=d, comms=comms, dr=dr, dw=dw, ro=ro, no=no:
                              ar.ar_lamport_oneshot_residual_rmsnorm(d[0], 0, comms, dr, dw,
                                                                     ro, no, fc["eps"], 1)])
                grid[f"M{M}_N{N}"] = {"one_shot_fused_us": one, "lamport_one_launch_us": lam}
                log(f"fused grid M={M} N={N}: one-shot {one} us, Lamport {lam} us")
                del comms
        rows["fused_grid_W4_warm"] = {
            "us_per_call": grid,
            "note": "same buffers every call (warm), as the source page's CUDA-graph method"}

        # one-shot against two-shot fused, one rank's call, at the workload's
        # M=128 and at a large M (2048 rows of 8192); cold buffer sets
        for M, N in ((128, 2048), (2048, 8192)):
            Wf = fc["W"]
            if (M, N) == (128, 2048):
                fx, fr, fw = synth.fused(M)
            else:
                fx, fr, fw = synth.fused_inputs(Wf, M, N, [1000 + fc["id"], M, N])
            mat, rowb = M * N * 2, N * 2
            part, rem = M // Wf, M % Wf
            own = part                       # rank 0 owns rows [0, part)
            one_bytes = (Wf + 3) * mat + 2 * N
            two_bytes = (Wf * own * rowb + own * rowb + 2 * N + 4 * own * rowb
                         + 4 * (M - own) * rowb)
            base_x = [to_dev(x) for x in fx]
            base_r, dw = to_dev(fr), to_dev(fw)
            s1 = []
            for k in range(sets_for(one_bytes)):
                xx = [b.view(M, N) for b in rank_buffers(Wf, mat, torch.int16, base_x)]
                rr = base_r if k == 0 else base_r.clone()
                s1.append((xx, rr, torch.empty_like(rr), torch.empty_like(rr)))
            if M != 128:
                row(f"fused_W4_M{M}_N{N}", one_bytes,
                    [lambda q=q: ar.ar_fused_residual_rmsnorm(q[0], q[1], dw, q[2], q[3],
                                                              fc["eps"]) for q in s1],
                    steps=8 * len(s1))
            del s1
            s2 = []
            for k in range(sets_for(two_bytes)):
                xx = [b.view(M, N) for b in rank_buffers(Wf, mat, torch.int16, base_x)]
                rr = base_r if k == 0 else base_r.clone()
                tmps = rank_buffers(Wf, 4 * (part + rem) * N, torch.int16)
                for r in range(1, Wf):
                    ar.ar_fused_residual_rmsnorm_2stage(xx, tmps, r, rr, dw, None, None,
                                                        fc["eps"], flags=ar.AR_STAGE_RS)
                s2.append((xx, rr, tmps, torch.empty_like(rr), torch.empty_like(rr)))
            row(f"fused2_W4_M{M}_N{N}_per_rank", two_bytes,
                [lambda q=q: ar.ar_fused_residual_rmsnorm_2stage(q[0], q[2], 0, q[1], dw, q[3],
                                                                 q[4], fc["eps"])
                 for q in s2],
                steps=8 * len(s2),
                oracle_fn=orc and (lambda fx=fx, fr=fr, fw=fw:
                                   orc.fused_2stage_scatter(fx, 0, fr, fw, fc["eps"])))
            del s2, base_x
            torch.cuda.empty_cache()

        def fused_crossover(Wf, N, Ms):
            cross = {}
            for M in Ms:
                fx, fr, fw = synth.fused_inputs(Wf, M, N, [1000 + fc["id"], Wf, M, N])
                mat = M * N * 2
                part, rem = M // Wf, M % Wf
                base_x = [to_dev(x) for x in fx]
                base_r, dw = to_dev(fr), to_dev(fw)
                nsets_f = sets_for((Wf + 3) * mat)
                s1, s2 = [], []
                for k in range(nsets_f):
                    xx = [b.view(M, N) for b in rank_buffers(Wf, mat, torch.int16, base_x)]
                    rr = base_r if k == 0 else base_r.clone()
                    tmps = rank_buffers(Wf, 4 * (part + rem) * N, torch.int16)
                    for r in range(1, Wf):
                        ar.ar_fused_residual_rmsnorm_2stage(xx, tmps, r, rr, dw, None, None,
                                                            fc["eps"], flags=ar.AR_STAGE_RS)
                    s1.append((xx, rr, torch.empty_like(rr), torch.empty_like(rr)))
                    s2.append((xx, rr, tmps, torch.empty_like(rr), torch.empty_like(rr)))
                k = max(8 * nsets_f, 40)
                k = -(-k // nsets_f) * nsets_f
                t1 = graph_time([lambda q=q: ar.ar_fused_residual_rmsnorm(
                    q[0], q[1], dw, q[2], q[3], fc["eps"]) for q in s1], k, args.warmup)
                t2 = graph_time([lambda q=q: ar.ar_fused_residual_rmsnorm_2stage(
                    q[0], q[2], 0, q[1], dw, q[3], q[4], fc["eps"]) for q in s2], k, args.warmup)
                cross[str(M)] = {"one_shot_us": round(t1 * 1e3, 3),
                                 "two_shot_us": round(t2 * 1e3, 3),
                                 "library_picks_two_shot": ar.ar_fused_prefers_two_shot(Wf, M, N)}
                del s1, s2, base_x
                torch.cuda.empty_cache()
            won = [int(m) for m, v in cross.items() if v["two_shot_us"] < v["one_shot_us"]]
            lost = [int(m) for m, v in cross.items() if v["two_shot_us"] >= v["one_shot_us"]]
            # the smallest M from which the two-shot call won at every larger M tried
            from_m = min((m for m in won if all(x < m for x in lost)), default=None)
            rows[f"fused_one_vs_two_shot_W{Wf}_N{N}"] = {
                "us_per_call": cross, "two_shot_faster_from_M": from_m}
            log(f"fused one-shot vs two-shot, W={Wf} N={N}: {cross}")

        # where the two-shot fused form overtakes the one-shot form for one
        # rank's call on this device: W = 2, 4, 8, N = 2048 and 8192, M from W
        # rows up (cold sets, graph-timed); the crossover M is reported, and
        # what ar_fused_prefers_two_shot picks for each shape beside it
        for Wf in (2, 4, 8):
            for N in (2048, 8192):
                Ms = [m for m in (2, 4, 8, 12, 16, 24, 32, 64, 128, 512, 2048) if m >= Wf]
                if Wf == 2:
                    Ms = [2, 16, 128, 2048]
                fused_crossover(Wf, N, Ms)

        # one-stage reduce: small, decode shape, and the cap message
        for name, maker in (("1stage_W2_n8192", synth.reduce_small),
                            ("1stage_W8_n8192", synth.reduce_decode)):
            xx = maker()
            d = [to_dev(x) for x in xx]
            o = torch.empty_like(d[0])
            row(name, (len(d) + 1) * d[0].numel() * 2,
                [lambda d=d, o=o: ar.ar_reduce_1stage(d, o)], steps=200,
                oracle_fn=orc and (lambda xx=xx: orc.reduce_1stage(xx)))
        # the per-launch floor: a one-stage reduce of a single 16-byte pack
        d = [to_dev(x[:8]) for x in synth.reduce_small()]
        o = torch.empty_like(d[0])
        row("launch_floor_1stage_W2_n8", 48, [lambda d=d, o=o: ar.ar_reduce_1stage(d, o)],
            steps=200)
        nb = (W + 1) * n * 2
        k1 = sets_for(nb)
        s1 = []
        for k in range(k1):
            ins = rank_buffers(W, 2 * n, torch.int16, base)
            s1.append((ins, torch.empty(n, dtype=torch.int16, device=dev)))
        row("1stage_W8_n4194304", nb,
            [lambda s=s: ar.ar_reduce_1stage(s[0], s[1]) for s in s1], steps=8 * k1,
            oracle_fn=orc and (lambda: orc.reduce_1stage(xs)),
            extra={"layout": f"rank buffers {RANK_GAP} B apart in one allocation"})
        del s1
        # the same call on buffers from separate allocations (each 2 MiB aligned
        # by the allocator, so all eight streams start on the same channels)
        s1 = []
        for k in range(k1):
            s1.append(([b.clone() for b in base], torch.empty(n, dtype=torch.int16, device=dev)))
        row("1stage_W8_n4194304_separate_allocations", nb,
            [lambda s=s: ar.ar_reduce_1stage(s[0], s[1]) for s in s1], steps=8 * k1)
        del s1
        # the rank-buffer gap: with 0 or 32 KiB between the 8 MiB buffers the
        # W streams read at the same offset start on the same HBM channels
        for gap in (0, 32768, 2048, RANK_GAP):
            s1 = []
            for k in range(k1):
                s1.append((rank_buffers(W, 2 * n, torch.int16, base, gap=gap),
                           torch.empty(n, dtype=torch.int16, device=dev)))
            row(f"1stage_W8_n4194304_gap{gap}", nb,
                [lambda s=s: ar.ar_reduce_1stage(s[0], s[1]) for s in s1], steps=8 * k1,
                extra={"layout": f"rank buffers {gap} B apart in one allocation"})
            del s1

        # the same per-rank two-stage call over message sizes of 1 to 32 MiB per
        # rank buffer (cold sets): a straight-line fit of us per launch against
        # bytes splits the launch into a fixed part and a streaming rate
        fit_x, fit_y = [], []
        for mib in (1, 2, 4, 8, 16, 32):
            nm = mib << 19                      # bf16 elements of `mib` MiB
            pm = nm // 8 // W
            nbm = (3 * W + 1) * pm * 16
            movedm = (W + 2 + 2 * (W - 1)) * pm * 16
            rep = -(-nm // n) if nm > n else 1
            src = [torch.cat([b] * rep)[:nm] for b in base] if nm >= n else [b[:nm] for b in base]
            sm = []
            for k in range(sets_for(movedm)):
                ins = rank_buffers(W, 2 * nm, torch.int16, src)
                tmps = rank_buffers(W, pm * 16, torch.int16)
                for r in range(1, W):
                    ar.ar_reduce_2stage(ins, tmps, r, None, flags=ar.AR_STAGE_RS)
                sm.append((ins, tmps, torch.empty(nm, dtype=torch.int16, device=dev)))
            rr = row(f"2stage_W8_n{nm}_per_rank", nbm,
                     [lambda s=s: ar.ar_reduce_2stage(s[0], s[1], 0, s[2]) for s in sm],
                     steps=8 * len(sm), extra={"bytes_moved": movedm, "sets": len(sm)})
            fit_x.append(nbm)
            fit_y.append(rr["us_per_call"])
            del sm, src
            torch.cuda.empty_cache()
        slope, icept = np.polyfit(np.array(fit_x, float), np.array(fit_y, float), 1)
        rows["2stage_W8_size_fit"] = {
            "fixed_us": round(float(icept), 3),
            "streaming_GBps": round(1e-3 / float(slope), 1),
            "points": {str(x): y for x, y in zip(fit_x, fit_y)},
            "note": "least-squares line through us per launch against the method's bytes "
                    "per launch, 1 to 32 MiB per rank buffer, cold sets"}
        log(f"two-stage size fit: {rows['2stage_W8_size_fit']}")

        # achievable-copy reference: a plain 16-byte copy kernel (ar_copy), cold
        # sets, moving the headline's bytes (12 MiB read + 12 MiB written) and
        # 512 MiB (256 + 256)
        for half_mib in (12, 256):
            nbc = half_mib << 20
            cs = []
            for k in range(sets_for(2 * nbc)):
                cs.append((torch.empty(nbc, dtype=torch.uint8, device=dev),
                           torch.empty(nbc, dtype=torch.uint8, device=dev)))
            for a, _ in cs:
                a.fill_(1)
            row(f"copy_{2 * half_mib}MiB_traffic", 2 * nbc,
                [lambda q=q: ar.ar_copy(q[0], q[1]) for q in cs], steps=8 * len(cs),
                extra={"note": "ar_copy of %d MiB into %d MiB, cold sets" % (half_mib, half_mib)})
            del cs
            torch.cuda.empty_cache()

    if args.rows in ("all", "sets"):
        # what the rotated buffer sets measure: the headline call over 1 to 40
        # sets (one rotation touches 24 MiB per set; the Infinity Cache holds
        # 256 MB), each set with its own 8 input and 8 staging buffers
        sweep = {}
        cap_packs = n // 8 // W + (n // 8) % W       # staging packs per shard
        for count in (1, 2, 3, 4, 6, 12, 23, 40):
            sw = []
            for k in range(count):
                ins = rank_buffers(W, 2 * n, torch.int16, base)
                tmps = rank_buffers(W, cap_packs * 16, torch.int16)
                for r in range(1, W):
                    ar.ar_reduce_2stage(ins, tmps, r, None, flags=ar.AR_STAGE_RS)
                sw.append((ins, tmps, torch.empty(n, dtype=torch.int16, device=dev)))
            k = -(-230 // count) * count
            t = graph_time([lambda q=q: ar.ar_reduce_2stage(q[0], q[1], 0, q[2]) for q in sw],
                           k, args.warmup)
            sweep[str(count)] = round(t * 1e3, 3)
            log(f"headline over {count} rotated sets: {t * 1e3:.3f} us")
            del sw
            torch.cuda.empty_cache()
        rows["2stage_W8_n4194304_rotated_sets_us_per_launch"] = sweep

    if args.rows in ("all", "wire"):
        # wire formats: W=4 fp32 payloads of 16 Mi values (and the +13 tail);
        # every row rotates buffer sets so each call streams from HBM
        wc = synth.WIRE
        # counter-measured HBM bytes per dispatch (profiles/), by kernel and
        # grid lanes, attached to the rows while the kernel sources match
        wt = wire_traffic()

        def add_traffic(r, kernel, lanes, wg, nbytes):
            tb = wt.get((kernel, -(-lanes // wg) * wg))
            if tb:
                r["traffic"] = tb
                r["traffic_over_algorithmic"] = round(tb / nbytes, 4)

        for nn in (wc["n"], wc["n"] + wc["tail"]):
            host_payloads = synth.wire(nn)
            payloads = [torch.from_numpy(p).to(dev) for p in host_payloads]
            for fmt, lsize, lines_fn, pack, unpack in (
                    ("ll128", 128, ar.ll128_lines, ar.ll128_pack, ar.ll128_unpack_reduce),
                    ("ll", 16, ar.ll_lines, ar.ll_pack, ar.ll_unpack_reduce)):
                opack = orc and (orc.ll128_pack if fmt == "ll128" else orc.ll_pack)
                ounpack = orc and (orc.ll128_unpack_reduce if fmt == "ll128"
                                   else orc.ll_unpack_reduce)
                L = lines_fn(nn)
                sl = -(-L // 8)
                tag = f"{fmt}_W4_n{nn}"
                dec_bytes = wc["W"] * L * lsize + 4 * nn
                dsets = []
                for _ in range(sets_for(dec_bytes)):
                    fifos = rank_buffers(wc["W"], 8 * sl * lsize, torch.uint8)
                    for p, f in zip(payloads, fifos):
                        pack(p, f, sl)
                    dsets.append((fifos, torch.empty(nn, dtype=torch.float32, device=dev)))
                hfifos = None
                if orc:
                    hfifos = [np.zeros(8 * sl * lsize, np.uint8) for _ in host_payloads]
                    for hp, hf in zip(host_payloads, hfifos):
                        opack(hp, hf, sl)
                r = row(f"{tag}_decode", dec_bytes,
                        [lambda d=d, sl=sl: unpack(d[0], d[1], sl) for d in dsets],
                        steps=8 * len(dsets),
                        oracle_fn=orc and (lambda hf=hfifos, nn=nn, sl=sl: ounpack(hf, nn, sl)))
                # payload rate: W payloads in, one sum out, at 4 bytes a value
                r["payload_GBps"] = round((wc["W"] + 1) * 4 * nn / (r["us_per_call"] * 1e3), 1)
                if fmt == "ll128":
                    add_traffic(r, "ar::ll128_unpack_reduce_kernel<4>", 8 * L, 256, dec_bytes)
                else:
                    add_traffic(r, "ar::ll_unpack_reduce_kernel<4>", L, 128, dec_bytes)
                del dsets
                pack_bytes = 4 * nn + L * lsize
                # source offsets of 0, 4, 8 and 12 bytes ([NCCL14]'s alignment sweep)
                offsets = (0, 1, 2, 3) if nn == wc["n"] else (0,)
                for off in offsets:
                    psets = []
                    for _ in range(sets_for(pack_bytes)):
                        raw = torch.empty(nn + 4, dtype=torch.float32, device=dev)
                        src = raw[off:off + nn]
                        src.copy_(payloads[0])
                        psets.append((raw, src, torch.empty(8 * sl * lsize, dtype=torch.uint8,
                                                            device=dev)))
                    name = f"{fmt}_n{nn}_pack" + (f"_src_offset{4 * off}" if off else "")
                    rp = row(name, pack_bytes,
                        [lambda q=q, sl=sl: pack(q[1], q[2], sl) for q in psets],
                        steps=8 * len(psets),
                        oracle_fn=(orc and not off and
                                   (lambda hp=host_payloads[0], hf=hfifos[0], sl=sl:
                                    opack(hp, hf, sl))) or None)
                    if not off:
                        if fmt == "ll128":
                            add_traffic(rp, "ar::ll128_pack_kernel", 16 * ((L + 1) // 2), 256,
                                        pack_bytes)
                        else:
                            add_traffic(rp, "ar::ll_pack_kernel", L, 256, pack_bytes)
                    del psets
                del hfifos
            del payloads
            torch.cuda.empty_cache()


    if args.rows in ("all", "stream"):
        wc = synth.WIRE
        # streaming through 8-step FIFOs (one launch of producer and consumer
        # workgroups per call): the 16 Mi fp32 wire payload at NCCL's default
        # step sizes, and a one-step 8 KiB message.  Each call starts from the
        # step the previous call stored in the counters, so graph replays run
        # fresh ring steps; the cold src/out sets rotate while the rings stay.
        def ring_written(proto, n_msg, step):
            """Ring bytes the producers write for one call: whole steps, then
            the last step's payload-carrying lines (LL 8 -> 16 bytes, LL128
            120 -> 128 bytes, Simple raw)."""
            def wire_of(nb):
                if proto == ar.AR_PROTO_LL:
                    return -(-nb // 8) * 16
                if proto == ar.AR_PROTO_LL128:
                    return -(-nb // 120) * 128
                return nb
            T = -(-4 * n_msg // step)
            return (T - 1) * wire_of(step) + wire_of(4 * n_msg - (T - 1) * step)

        nn = wc["n"]
        host_src = synth.wire(nn)[0]
        dsrc = torch.from_numpy(host_src).to(dev)
        ss = []
        for k in range(sets_for(8 * nn)):
            ss.append((dsrc if k == 0 else dsrc.clone(),
                       torch.empty(nn, dtype=torch.float32, device=dev)))
        for fmt, proto, step in (("ll", ar.AR_PROTO_LL, 32768),
                                 ("ll128", ar.AR_PROTO_LL128, 576000),
                                 ("simple", ar.AR_PROTO_SIMPLE, 524288)):
            for ch, n_msg in ((32, nn), (128, nn), (1, 2048)):
                wire = ar.ar_fifo_step_wire_bytes(proto, step)
                fifo = torch.zeros(ch * 8 * wire, dtype=torch.uint8, device=dev)
                cnt = torch.zeros(ar.ar_fifo_counter_words(ch), dtype=torch.int64, device=dev)
                errs = torch.zeros(1, dtype=torch.int32, device=dev)
                ring_bytes = ring_written(proto, n_msg, step)
                calls = [(lambda q=q, proto=proto, step=step, ch=ch, fifo=fifo, cnt=cnt,
                          errs=errs, n_msg=n_msg:
                          ar.ar_fifo_stream(proto, q[0], q[1], fifo, cnt, ch, step,
                                            ar.AR_FIFO_CONTINUE, errors=errs, n=n_msg))
                         for q in ss]
                # bytes the launch moves: payload read, ring written and read,
                # output written
                r = row(f"stream_{fmt}_n{n_msg}_step{step}_c{ch}", 8 * n_msg + 2 * ring_bytes,
                        calls,
                        steps=8 * len(ss) if n_msg == nn else 200,
                        oracle_fn=orc and n_msg == nn and ch == 32 and
                        (lambda proto=proto, step=step: orc.fifo_stream(proto, host_src, 32, step))
                        or None)
                t_s = r["us_per_call"] * 1e-6
                torch.cuda.synchronize()
                lanes, pairs, bsteps = ar.ar_fifo_plan(proto, n_msg, ch, step)
                r.update({"channels": ch,
                          "step_bytes": step, "payload_GBps": round(4 * n_msg / t_s / 1e9, 1),
                          "ring_bytes_written": ring_bytes,
                          "plan": {"lanes": lanes, "pairs_per_channel": pairs,
                                   "steps_per_batch": bsteps},
                          "failed_waits": int(errs.item())})
                del fifo, cnt, calls
        # message-size sweep at 32 channels: where LL, LL128 and Simple cross.
        # The step is NCCL's default, cut down to the message's share per
        # channel (rounded up to the protocol's unit) so that a mid-size
        # message spreads over all channels rather than filling one step.
        xo = {}
        for size in (1 << 13, 1 << 16, 1 << 19, 1 << 22, 1 << 25):
            n_msg = size // 4
            xo[str(size)] = {}
            for fmt, proto, default_step, unit in (("ll", ar.AR_PROTO_LL, 32768, 8),
                                                   ("ll128", ar.AR_PROTO_LL128, 576000, 120),
                                                   ("simple", ar.AR_PROTO_SIMPLE, 524288, 16)):
                ch = 32
                share = -(-(-(-size // ch)) // unit) * unit
                step = min(default_step, share)
                wire = ar.ar_fifo_step_wire_bytes(proto, step)
                fifo = torch.zeros(ch * 8 * wire, dtype=torch.uint8, device=dev)
                cnt = torch.zeros(ar.ar_fifo_counter_words(ch), dtype=torch.int64, device=dev)
                errs = torch.zeros(1, dtype=torch.int32, device=dev)
                calls = [(lambda q=q, proto=proto, step=step, fifo=fifo, cnt=cnt, errs=errs,
                          n_msg=n_msg:
                          ar.ar_fifo_stream(proto, q[0], q[1], fifo, cnt, 32, step,
                                            ar.AR_FIFO_CONTINUE, errors=errs, n=n_msg))
                         for q in ss]
                k = 8 * len(ss) if size >= (1 << 22) else 40 * len(ss)
                t = graph_time(calls, k, args.warmup)
                torch.cuda.synchronize()
                xo[str(size)][fmt] = round(t * 1e3, 3)
                xo[str(size)][fmt + "_step"] = step
                if int(errs.item()) != 0:
                    xo[str(size)][fmt + "_failed_waits"] = int(errs.item())
                del fifo, cnt, calls
            log(f"stream sweep {size} B at 32 channels: {xo[str(size)]} us")
        rows["stream_sizes_c32_us_per_call"] = xo
        del ss, dsrc
        torch.cuda.empty_cache()

    if args.rows != "none" or rows:
        result["rows"] = rows

    if args.calib_copy:
        # counter calibration: three plain 256 MiB copies with the library's
        # copy kernel (262,144 KiB read + 262,144 KiB written each)
        a = torch.ones(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            ar.ar_copy(a, b)
        torch.cuda.synchronize()

    # ------------------------------------------------------------------
    # CPU baseline: the oracle on the same per-rank two-stage work
    # ------------------------------------------------------------------
    if not args.no_cpu:
        log("CPU oracle baseline (~10 s)")
        tmps = [orc.reduce_scatter(xs, s) for s in range(W)]
        reps, t0 = 0, time.perf_counter()
        while True:
            own = orc.reduce_scatter(xs, 0)
            orc.all_gather([own] + tmps[1:], n)
            reps += 1
            el = time.perf_counter() - t0
            if el >= 10.0:
                break
        single = {"value": round(bytes_2stage * reps / el / 1e9, 3),
                  "ms_per_step": round(el / reps * 1e3, 3), "repetitions": reps,
                  "seconds": round(el, 2)}
        # the same oracle calls on every host core of this GPU's share at once
        # (one Python thread each; ctypes releases the GIL inside the C code),
        # each thread doing whole steps on its own outputs: aggregate throughput
        import concurrent.futures
        threads = max(1, min(16, len(os.sched_getaffinity(0))))
        log(f"CPU oracle baseline on {threads} threads (~3 s)")

        def worker(deadline):
            k = 0
            while time.perf_counter() < deadline:
                own = orc.reduce_scatter(xs, 0)
                orc.all_gather([own] + tmps[1:], n)
                k += 1
            return k

        t0 = time.perf_counter()
        with concurrent.futures.ThreadPoolExecutor(threads) as pool:
            counts = list(pool.map(worker, [t0 + 3.0] * threads))
        el_all = time.perf_counter() - t0
        reps_all = sum(counts)
        result["cpu_baseline"] = {
            "value": round(bytes_2stage * reps_all / el_all / 1e9, 3),
            "unit": "GB/s",
            "cores": threads,
            "kind": "oracle",
            "sample": f"the full per-rank two-stage work of the headline workload "
                      f"(reduce-scatter of shard 0 + all-gather of the 8 shards, "
                      f"8 x 4,194,304 bf16): {reps_all} steps in {el_all:.1f} s on "
                      f"{threads} threads at once (plain C, {cpu_model()}); the same "
                      f"work single-threaded: {reps} steps in {el:.1f} s",
            "ms_per_step": round(el_all / reps_all * 1e3, 3),
            "single_core": single,
        }

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
