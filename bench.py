#!/usr/bin/env python3
"""Throughput of the head-scale KV-pruning hot path on one MI355X.

A step is one generation pass of the whole hot path over one batch: for every
scale t = 0..K-1 and every layer, block-causal attention over the kept cache
segments plus the current scale, with the scale's kept segments compacted into
the ragged cache in the same launch (hk_attend_append; the final scale is only
attended).  The same pass with separate hk_attend / hk_append_scale calls is
timed beside it.  Inputs are synthetic and already resident in HBM when the
timed region starts.

Default workload: one Infinity-2B-shaped layer at full cache (16 heads,
head_dim 128, batch 1, 13 scales with sides 1..64, 10,521 tokens), bf16.
``value`` is attention TFLOP/s over the whole pass (algorithmic flops
4*d*n_q*n_k summed over all attention launches, divided by the pass time).

Also reported: the 256-query attention kernel's roofline (MFMA bf16), the
32-layer batch-8 10%-budget workload's scales/s per image, standalone
compaction GB/s (HBM roofline) on the 32-layer batch-4 full-cache workload,
and the fp64 CPU oracle timed on the same full-cache pass on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("attend TFLOP/s + % bf16 MFMA peak; compact GB/s; scales/sec per image at 10% budget")
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
ATTEND_SOURCES = ["kv_cache_compression_attend_amd/csrc/attend_bf16.hip",
                  "kv_cache_compression_attend_amd/csrc/attend.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attend_q256_infinity2b_layer_traffic.json")
ROOFLINE_KERNEL = "attend_q256_kernel<false, false, false, true>"


def attend_sources_sha() -> str:
    h = hashlib.sha256()
    for p in ATTEND_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # One step of the default workload takes ~0.7 ms.  After the seconds of
    # host-side set-up the GPU clock needs ~100 ms of work to ramp up: 5
    # warmup passes left the timed average 4% slower than steady state.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-pruned", action="store_true",
                    help="skip the 32-layer 10%%-budget scales/s measurement")
    ap.add_argument("--pruned-steps", type=int, default=5)
    ap.add_argument("--sections", default="all",
                    help="comma-separated workload sections after the main line (pruned, "
                         "progressive, window, int4, compact, infinity8b_4pct, "
                         "infinity8b_full_cache, calibration) or 'all'")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run three 1 GiB device-to-device copies (calibrates HBM byte counters)")
    ap.add_argument("--summarize-pass", metavar="KERNEL_TRACE_CSV",
                    help="print the per-launch durations of one fused pass of the main line from a "
                         "rocprofv3 kernel trace, then exit")
    ap.add_argument("--summarize-trace", metavar="KERNEL_TRACE_CSV",
                    help="print the average duration of the final-scale attend launch (the "
                         "largest-grid dispatches of the roofline kernel) from a rocprofv3 "
                         "kernel-trace CSV of this benchmark, then exit")
    ap.add_argument("--data-sensitivity", action="store_true",
                    help="time the final-scale attend launch of the main workload on its random "
                         "inputs, with V zeroed, and with K and V zeroed (same instructions, less "
                         "operand toggling), then exit")
    ap.add_argument("--cpu-passes", type=int, default=1,
                    help="passes of the oracle over the main workload (the whole layer takes ~4 s)")
    ap.add_argument("--cpu-heads", type=int, default=16,
                    help="heads of the full-cache layer the CPU oracle runs (all 13 scales)")
    ap.add_argument("--sections-only", action="store_true",
                    help="run only the sections named by --sections (no main line, no CPU "
                         "baseline) and print their JSON")
    ap.add_argument("--summarize-compact-counters", nargs=4,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="print the HBM traffic of the compaction kernels per pass of the compact "
                         "section (--sections-only --sections compact) from rocprofv3 counter CSVs, "
                         "then exit")
    ap.add_argument("--summarize-counters", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV",
                                                              "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="print the HBM traffic profile of the final-scale attend launch from "
                         "rocprofv3 counter CSVs of this benchmark and of --copy-probe, then exit")
    return ap.parse_args()


def summarize_trace(path):
    """Average duration of the final-scale launches of the roofline kernel in
    a rocprofv3 kernel trace (the kernel also serves smaller scales, whose
    dispatches have smaller grids)."""
    import csv
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if ROOFLINE_KERNEL in r["Kernel_Name"]:
                grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
                rows.append((grid, int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    if not rows:
        raise SystemExit(f"no {ROOFLINE_KERNEL} dispatch in {path}")
    top = max(g for g, _ in rows)
    durs = [d for g, d in rows if g == top]
    return {"kernel": ROOFLINE_KERNEL, "grid_threads": top, "dispatches": len(durs),
            "avg_ns": round(sum(durs) / len(durs), 1), "min_ns": min(durs), "max_ns": max(durs),
            "other_dispatches_of_kernel": len(rows) - len(durs)}


def summarize_pass(path):
    """Per-launch durations of one fused generation pass of the default
    workload, from a rocprofv3 kernel trace of the main line: the dispatches
    between consecutive final-scale launches (the roofline kernel's largest
    grid) that contain no compaction kernel (those belong to the unfused
    pass), median over the passes with the commonest launch sequence."""
    import csv
    import re
    import statistics
    seq = []
    with open(path) as f:
        for r in csv.DictReader(f):
            grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            m = re.search(r"(\w+_kernel(?:<[\w, ]+>)?)", r["Kernel_Name"])
            name = m.group(1) if m else r["Kernel_Name"]
            seq.append((int(r["Start_Timestamp"]), name, grid,
                        int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    seq.sort()
    top = max((g for _, n, g, _ in seq if n == ROOFLINE_KERNEL), default=None)
    if top is None:
        raise SystemExit(f"no {ROOFLINE_KERNEL} dispatch in {path}")
    ends = [i for i, (_, n, g, _) in enumerate(seq) if n == ROOFLINE_KERNEL and g == top]
    passes = []
    for a, b in zip(ends, ends[1:]):
        part = seq[a + 1: b + 1]
        if any("compact" in n for _, n, _, _ in part):
            continue
        passes.append(part)
    if not passes:
        raise SystemExit(f"no fused pass in {path}")
    shapes = [tuple((n, g) for _, n, g, _ in p) for p in passes]
    shape = max(set(shapes), key=shapes.count)
    same = [p for p, s in zip(passes, shapes) if s == shape]
    launches = [{"kernel": n, "grid_threads": g,
                 "median_us": round(statistics.median(p[i][3] for p in same) / 1e3, 2)}
                for i, (n, g) in enumerate(shape)]
    return {"passes": len(same), "launches": launches,
            "sum_median_us": round(sum(x["median_us"] for x in launches), 1)}


def summarize_counters(paths):
    """Traffic profile (bytes per launch) of the final-scale attend launch of
    the default workload: FETCH_SIZE and WRITE_SIZE averaged over its
    dispatches and scaled by what the same counters read for the 1 GiB
    copies of --copy-probe."""
    import csv

    def per_dispatch(path, match):
        vals, grid = {}, {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if match(r["Kernel_Name"]):
                    vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
                    grid[r["Dispatch_Id"]] = int(r["Grid_Size"])
        if not vals:
            raise SystemExit(f"no matching dispatch in {path}")
        # The kernel also serves smaller scales: keep the final-scale
        # dispatches, those with the largest grid.
        top = max(grid.values())
        keep = [d for d in vals if grid[d] == top]
        return sum(vals[d] for d in keep) / len(keep), len(keep)

    def is_kernel(name):
        return ROOFLINE_KERNEL in name

    def is_copy(name):
        return "copyBuffer" in name

    fetch, nf = per_dispatch(paths[0], is_kernel)
    write, nw = per_dispatch(paths[1], is_kernel)
    copy_fetch, _ = per_dispatch(paths[2], is_copy)
    copy_write, _ = per_dispatch(paths[3], is_copy)
    gib_kib = float(1 << 20)
    fs, ws = gib_kib / copy_fetch, gib_kib / copy_write
    # Compulsory bytes of the launch: Q, cached K and V, current K and V, out.
    B, H, D, n, cached = 1, 16, 128, 4096, 6425
    algo = (4 * n + 2 * cached) * B * H * D * 2
    total = (fetch * fs + write * ws) * 1024
    return {"kernel": ROOFLINE_KERNEL,
            "workload": "infinity2b-layer-full-b1, final scale (4,096 queries x 10,521 keys x 16 heads), one launch",
            "kernel_sha256": attend_sources_sha(), "kernel_sources": ATTEND_SOURCES,
            "fetch_size_kib_per_launch_raw": round(fetch, 2), "write_size_kib_per_launch_raw": round(write, 2),
            "dispatches": [nf, nw], "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
            "scale_source": "1 GiB device-to-device copies of bench.py --copy-probe: FETCH_SIZE "
                            f"{copy_fetch:,.1f} KiB, WRITE_SIZE {copy_write:,.1f} KiB per copy",
            "bytes_per_launch": int(round(total)), "algorithmic_bytes_per_launch": algo,
            "ratio_to_algorithmic": round(total / algo, 4),
            "commands": [
                "cd /tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d <f> -o run -- python3 <repo>/bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-pruned",
                "cd /tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv -d <w> -o run -- python3 <repo>/bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-pruned",
                "cd /tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d <cf> -o run -- python3 <repo>/bench.py --copy-probe",
                "cd /tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv -d <cw> -o run -- python3 <repo>/bench.py --copy-probe",
                "python3 <repo>/bench.py --summarize-counters <f>/run_counter_collection.csv "
                "<w>/run_counter_collection.csv <cf>/run_counter_collection.csv <cw>/run_counter_collection.csv"]}


def summarize_compact_counters(paths):
    """HBM traffic of the compaction kernels over the compact section's
    passes (all-layer appends of the 32-layer batch-4 full-cache workload,
    13.47 GB algorithmic per pass), scaled by the copy-probe counters."""
    import csv

    def totals(path, match):
        vals, grid = {}, {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if match(r["Kernel_Name"]):
                    key = r["Dispatch_Id"]
                    vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
                    grid[key] = (r["Kernel_Name"], int(r["Grid_Size"]))
        return vals, grid

    def is_compact(name):
        return "compact_rows_kernel" in name or "compact_kernel" in name

    def copy_kib(path):
        vals, _ = totals(path, lambda n: "copyBuffer" in n)
        if not vals:
            raise SystemExit(f"no copy dispatch in {path}")
        return sum(vals.values()) / len(vals)

    fv, fg = totals(paths[0], is_compact)
    wv, wg = totals(paths[1], is_compact)
    if not fv or not wv:
        raise SystemExit("no compaction dispatch")
    # passes: dispatches of the largest grid (one per pass, the largest scale)
    top = max(g for _, g in fg.values())
    passes = sum(1 for _, g in fg.values() if g == top)
    fs, ws = float(1 << 20) / copy_kib(paths[2]), float(1 << 20) / copy_kib(paths[3])
    fetch = sum(fv.values()) * fs * 1024 / passes
    write = sum(wv.values()) * ws * 1024 / passes
    per_kernel = {}
    for d, (n, _) in fg.items():
        short = "compact_rows_kernel" if "compact_rows_kernel" in n else "compact_kernel"
        per_kernel.setdefault(short, [0, 0.0, 0.0])
        per_kernel[short][0] += 1
        per_kernel[short][1] += fv[d] * fs * 1024 / passes
        per_kernel[short][2] += wv.get(d, 0.0) * ws * 1024 / passes
    algo = 13.47e9
    return {"workload": "infinity2b-l32-b4 full cache: one all-layer append per completed scale",
            "passes": passes, "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
            "read_bytes_per_pass": int(fetch), "write_bytes_per_pass": int(write),
            "bytes_per_pass": int(fetch + write), "algorithmic_bytes_per_pass": algo,
            "ratio_to_algorithmic": round((fetch + write) / algo, 4),
            "per_kernel": {k: {"dispatches_per_pass": v[0] / passes, "read_bytes": int(v[1]),
                               "write_bytes": int(v[2])} for k, v in per_kernel.items()},
            "commands": [
                "cd /tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d <f> -o run -- python3 <repo>/bench.py --sections-only --sections compact",
                "cd /tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv -d <w> -o run -- python3 <repo>/bench.py --sections-only --sections compact",
                "cd /tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d <cf> -o run -- python3 <repo>/bench.py --copy-probe",
                "cd /tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv -d <cw> -o run -- python3 <repo>/bench.py --copy-probe",
                "python3 <repo>/bench.py --summarize-compact-counters <f>/run_counter_collection.csv "
                "<w>/run_counter_collection.csv <cf>/run_counter_collection.csv <cw>/run_counter_collection.csv"]}


def pass_flops(wl, keep, lenb_fn):
    """Algorithmic attention flops of each (layer, step) launch: sum over (b, h)
    of 4 * d * n_t * (cached keys + n_t)."""
    out = {}
    for l in range(wl.layers):
        for t in range(wl.n_scales):
            n = wl.scale_tokens[t]
            keys = lenb_fn(t)[l] + n          # [H]
            out[(l, t)] = 4.0 * wl.head_dim * n * float(keys.sum()) * wl.batch
    return out


def compact_bytes(wl, keep, t, layers):
    """Algorithmic bytes of one compaction launch: read + write of every kept segment."""
    kept = int(keep[layers, :, t].sum()) if t <= wl.n_scales - 2 else 0
    elem = 2 if wl.dtype == "bf16" else 4
    return 2.0 * 2.0 * kept * wl.batch * wl.scale_tokens[t] * wl.head_dim * elem


def lenb_table(keep, tokens):
    import numpy as np
    L, H, K = keep.shape

    def f(t):
        out = np.zeros((L, H), dtype=np.int64)
        for s in range(min(t, K - 1)):
            out += keep[:, :, s].astype(np.int64) * tokens[s]
        return out
    return f


def data_sensitivity(ctx, wl, qs, kall, vall, outs, stream, torch, reps=20):
    """Average duration of the final-scale attend launch (HIP events) when
    the cache and the current scale hold the workload's random values, zero
    values, or zero keys and values: the instruction stream is the same, only
    the operands the matrix cores see toggle less."""
    K, L = wl.n_scales, wl.layers
    res = {}
    for mode in ("random", "v_zero", "kv_zero", "random_again"):
        ks = [k.clone() for k in kall]
        vs = [v.clone() for v in vall]
        if mode in ("v_zero", "kv_zero"):
            for v in vs:
                v.zero_()
        if mode == "kv_zero":
            for k in ks:
                k.zero_()
        ctx.reset()
        for t in range(K - 1):
            for l in range(L):
                ctx.attend_append(l, t, qs[t][l], ks[t][l], vs[t][l], outs[t], wl.softmax_scale,
                                  stream=stream)
        last = lambda: ctx.attend(0, K - 1, qs[K - 1][0], ks[K - 1][0], vs[K - 1][0], outs[K - 1],  # noqa
                                  wl.softmax_scale, stream=stream)
        for _ in range(3):
            last()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            last()
        e1.record(stream)
        torch.cuda.synchronize()
        res[mode] = round(e0.elapsed_time(e1) / reps * 1e3, 1)
    return {"data_sensitivity": {"workload": wl.name, "launch": "final-scale attend, layer 0",
                                 "avg_us": res, "reps": reps}}


def main():
    args = parse()
    if args.summarize_counters:
        print(json.dumps(summarize_counters(args.summarize_counters), indent=1))
        return
    if args.summarize_compact_counters:
        print(json.dumps(summarize_compact_counters(args.summarize_compact_counters), indent=1))
        return
    if args.summarize_pass:
        print(json.dumps(summarize_pass(args.summarize_pass), indent=1))
        return
    if args.summarize_trace:
        print(json.dumps(summarize_trace(args.summarize_trace), indent=1))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only (the path has no multi-GPU mode); --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import kv_cache_compression_attend_amd as hk
    import workloads

    assert torch.cuda.is_available(), "bench needs a GPU"
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    if args.copy_probe:
        src = torch.ones(1 << 29, dtype=torch.int16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_each": src.numel() * 2, "copies": 3}), flush=True)
        return

    # ---------------- main workload: one full-cache Infinity-2B-shaped layer ----------------
    # Its inputs are drawn on the host before the other workloads run, so
    # that no host-side work idles the GPU between their passes (which bring
    # it to its sustained clock) and the main line's timed passes.
    if not args.sections_only:
        wl = workloads.get("c1")
        table = workloads.dirichlet_scas(wl)
        keep, _, _ = hk.build_schedule(table, wl.scale_tokens, wl.budget, wl.n_sink)
        ctx = hk.Context(wl.layers, wl.heads, wl.head_dim, wl.batch, wl.scale_tokens, keep,
                         torch.bfloat16)
        K, L = wl.n_scales, wl.layers
        qs, kall, vall, outs = [], [], [], []
        for t in range(K):
            ins = [workloads.step_inputs(wl, l, t) for l in range(L)]
            to = lambda a: torch.from_numpy(np.stack(a).view(np.int16)).to(dev).view(torch.bfloat16)  # noqa
            qs.append(to([x.q for x in ins]))
            kall.append(to([x.k for x in ins]))
            vall.append(to([x.v for x in ins]))
            outs.append(torch.empty_like(qs[-1][0]))
        flops = pass_flops(wl, keep, lenb_table(keep, wl.scale_tokens))
        total_flops = sum(flops.values())

    # ---------------- the other workloads ----------------
    # They run first: the GPU then reaches its sustained clock (it needs ~100
    # ms of work after the host-side set-up) before the main line's timed
    # passes, whatever the number of warmup passes.
    result = {}
    sections = {"pruned", "progressive", "window", "int4", "compact", "infinity8b_4pct",
                "infinity8b_full_cache", "calibration"}
    want = sections if args.sections == "all" else set(args.sections.split(","))
    unknown = want - sections
    if unknown:
        raise SystemExit(f"unknown sections {sorted(unknown)}")
    if args.no_pruned or args.data_sensitivity:
        want = set()
    # Each section runs in turn; a line on stderr reports each one as it ends.
    runners = [
        ("pruned", "pruned_10pct", lambda: pruned_rate(args, hk, workloads, torch, np, dev, stream)),
        ("progressive", "progressive_10pct",
         lambda: progressive_rate(args, hk, workloads, torch, np, dev, stream)),
        ("window", "scale_window", lambda: window_rate(args, hk, workloads, torch, np, dev, stream)),
        ("int4", "int4_10pct", lambda: int4_rate(args, hk, workloads, torch, np, dev, stream)),
        ("compact", "compact", lambda: compact_rate(args, hk, workloads, torch, np, dev, stream)),
        ("infinity8b_4pct", "infinity8b_4pct",
         lambda: infinity8b_rate(args, hk, workloads, torch, np, dev, stream, full_cache=False)),
        ("infinity8b_full_cache", "infinity8b_full_cache",
         lambda: infinity8b_rate(args, hk, workloads, torch, np, dev, stream, full_cache=True)),
        ("calibration", "calibration",
         lambda: calibration_rate(args, hk, workloads, torch, np, dev, stream)),
    ]
    for name, key, run in runners:
        if name in want:
            t0 = time.time()
            result[key] = run()
            print(f"[bench] section {name} done in {time.time() - t0:.1f} s", file=sys.stderr,
                  flush=True)

    if args.sections_only:
        print(json.dumps(result), flush=True)
        return

    if args.data_sensitivity:
        print(json.dumps(data_sensitivity(ctx, wl, qs, kall, vall, outs, stream, torch)), flush=True)
        return

    def one_pass(rec=None):
        """One generation pass: attention of every (layer, scale) with the
        scale's compaction fused into the same launch."""
        ctx.reset()
        for t in range(K):
            for l in range(L):
                if rec is not None:
                    rec[("a", l, t)][0].record(stream)
                ctx.attend_append(l, t, qs[t][l], kall[t][l], vall[t][l], outs[t], wl.softmax_scale,
                                  stream=stream)
                if rec is not None:
                    rec[("a", l, t)][1].record(stream)

    def unfused_pass():
        """The same pass with attention and compaction as separate calls."""
        ctx.reset()
        for t in range(K):
            for l in range(L):
                ctx.attend(l, t, qs[t][l], kall[t][l], vall[t][l], outs[t], wl.softmax_scale,
                           stream=stream)
            if t < K - 1:
                if L == 1:
                    ctx.append_scale(0, 1, t, kall[t][0], vall[t][0], stream=stream)
                else:
                    ctx.append_scale(0, L, t, kall[t], vall[t], stream=stream)

    for _ in range(args.warmup):
        one_pass()
    torch.cuda.synchronize()

    # timed passes (whole-pass clock), then the same number of passes with per-launch events
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(args.steps):
        one_pass()
    t1.record(stream)
    torch.cuda.synchronize()
    ms_pass = t0.elapsed_time(t1) / args.steps

    recs = []
    for _ in range(args.steps):
        rec = {}
        for t in range(K):
            for l in range(L):
                rec[("a", l, t)] = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        recs.append(rec)
    # A sleep kernel ahead of the passes lets the host queue launches and
    # events ahead of the GPU (it queues a pass in less time than the GPU
    # runs one), so the events time the launches and not the host's calls
    # between them; the passes then run back to back, as in the timed region.
    gpu_sleep(torch)
    for rec in recs:
        one_pass(rec)
    torch.cuda.synchronize()
    attend_ms = {key: np.mean([r[key][0].elapsed_time(r[key][1]) for r in recs])
                 for key in recs[0] if key[0] == "a"}

    for _ in range(2):
        unfused_pass()
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(args.steps):
        unfused_pass()
    t1.record(stream)
    torch.cuda.synchronize()
    ms_unfused = t0.elapsed_time(t1) / args.steps
    attend_total_ms = sum(attend_ms.values())
    attend_tflops = total_flops / (attend_total_ms * 1e-3) / 1e12
    n_launch = len(attend_ms)
    # The dominant launch: the final scale, served by the 256-query pipelined
    # kernel without a split.
    q256 = [("a", l, K - 1) for l in range(L)]
    assert all(ctx.attend_plan(K - 1) == (256, 1) for _ in q256), ctx.attend_plan(K - 1)
    q256_ms = sum(attend_ms[k] for k in q256)
    q256_flops = sum(flops[(k[1], k[2])] for k in q256)
    q256_tflops = q256_flops / (q256_ms * 1e-3) / 1e12 if q256 else 0.0
    per_step = {t: round(flops[(0, t)] / (attend_ms[("a", 0, t)] * 1e-3) / 1e12, 1) for t in range(K)}

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("kernel_sha256") == attend_sources_sha():
            traffic = tr.get("bytes_per_launch")

    value = total_flops / (ms_pass * 1e-3) / 1e12
    sections_out = result
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_pass, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) draws rounded to bf16; no model weights)",
        "config": {"workload": "infinity2b-layer-full-b1: 1 layer x 16 heads x head_dim 128, "
                               "batch 1, 13 scales (sides 1..64, 10,521 tokens), 100% budget; "
                               "13 attend_append calls per step (compaction fused)",
                   "global_batch": wl.batch, "seq_len": wl.total_tokens,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": ROOFLINE_KERNEL,
                     "achieved": round(q256_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(q256_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic,
                     "launches_per_step": len(q256),
                     "avg_launch_us": round(q256_ms / max(len(q256), 1) * 1e3, 2),
                     "flops_per_launch": q256_flops / max(len(q256), 1)},
        "roofline_all_attend": {"bound": "mfma", "kernels": "all attend launches incl. split merges",
                                "achieved": round(attend_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                                "unit": "TFLOP/s", "frac": round(attend_tflops / PEAK_BF16_TFLOPS, 4),
                                "avg_launch_us": round(attend_total_ms / n_launch * 1e3, 2)},
        "attend_plan_per_step": {t: list(ctx.attend_plan(t)) for t in range(K)},
        "attend_tflops_per_step": per_step,
        "unfused_ms_per_step": round(ms_unfused, 4),
        "unfused_value": round(total_flops / (ms_unfused * 1e-3) / 1e12, 2),
    }
    ctx.close()
    del qs, kall, vall, outs
    torch.cuda.empty_cache()
    result.update(sections_out)

    print(f"[bench] main line done: {result['value']} TFLOP/s", file=sys.stderr, flush=True)

    # ---------------- fp64 CPU oracle on a bounded sample ----------------
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, wl, keep)
        print("[bench] cpu baseline done", file=sys.stderr, flush=True)
    print(json.dumps(result), flush=True)


def gpu_sleep(torch, ms=3.0):
    """Keeps the GPU busy for about `ms` (a spin kernel) so that the host can
    queue a whole pass of launches and events behind it."""
    torch.cuda._sleep(int(ms * 2.4e6))


def step_profile(ctx, K, L, call, flops, stream, torch, passes=2):
    """Per-step time of a whole pass (HIP events at the step boundaries on the
    launch stream, mean over passes) and the step's attention TFLOP/s (its
    launches over all layers, compaction fused where the call fuses it)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    ms = [0.0] * K
    for _ in range(passes):
        ctx.reset()
        gpu_sleep(torch)
        for t in range(K):
            ev[t].record(stream)
            for l in range(L):
                call(l, t)
        ev[K].record(stream)
        torch.cuda.synchronize()
        for t in range(K):
            ms[t] += ev[t].elapsed_time(ev[t + 1]) / passes
    out = {}
    for t in range(K):
        f = sum(flops[(l, t)] for l in range(L))
        out[t] = {"ms": round(ms[t], 4), "tflops": round(f / (ms[t] * 1e-3) / 1e12, 1),
                  "plan": list(ctx.attend_plan(t))}
    return out


def pruned_rate(args, hk, workloads, torch, np, dev, stream):
    """Whole-pass rate of the 32-layer, batch-8, 10%-budget workload."""
    wl = workloads.get("c2")
    keep, ret, n_pruned = hk.build_schedule(workloads.dirichlet_scas(wl), wl.scale_tokens,
                                            wl.budget, wl.n_sink)
    ctx = hk.Context(wl.layers, wl.heads, wl.head_dim, wl.batch, wl.scale_tokens, keep,
                     torch.bfloat16)
    g = torch.Generator(device=dev)
    g.manual_seed(2)
    K, L = wl.n_scales, wl.layers
    qs, kall, vall, outs = [], [], [], []
    for t in range(K):
        shape = (L, wl.batch, wl.scale_tokens[t], wl.heads, wl.head_dim)
        qs.append((torch.randn(shape, generator=g, device=dev) * wl.qk_std).to(torch.bfloat16))
        kall.append((torch.randn(shape, generator=g, device=dev) * wl.qk_std).to(torch.bfloat16))
        vall.append(torch.randn(shape, generator=g, device=dev).to(torch.bfloat16))
        outs.append(torch.empty(shape[1:], dtype=torch.bfloat16, device=dev))
    flops = pass_flops(wl, keep, lenb_table(keep, wl.scale_tokens))

    def one_pass():
        ctx.reset()
        for t in range(K):
            for l in range(L):
                ctx.attend_append(l, t, qs[t][l], kall[t][l], vall[t][l], outs[t], wl.softmax_scale,
                                  stream=stream)

    one_pass()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.pruned_steps):
        one_pass()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.pruned_steps
    steps = step_profile(ctx, K, L, lambda l, t: ctx.attend_append(
        l, t, qs[t][l], kall[t][l], vall[t][l], outs[t], wl.softmax_scale, stream=stream),
        flops, stream, torch)
    ctx.close()
    return {"workload": "infinity2b-l32-b8-budget10: 32 layers x 16 heads x d128, batch 8, "
                        f"10% budget ({n_pruned} of 512 heads pruned per prunable scale)",
            "ms_per_pass": round(ms, 3),
            "scales_per_sec_per_image": round(K / (ms * 1e-3), 1),
            "image_scales_per_sec": round(K * wl.batch / (ms * 1e-3), 1),
            "attend_tflops_incl_compaction": round(sum(flops.values()) / (ms * 1e-3) / 1e12, 1),
            "passes": args.pruned_steps,
            "per_step": steps,
            "inputs": "torch.randn on the GPU (seeded), same distribution as the parity inputs"}


def infinity8b_rate(args, hk, workloads, torch, np, dev, stream, full_cache):
    """Whole-pass rate of the 40-layer, 28-head, batch-16 (Infinity-8B-shaped)
    workload: at its 4% budget, or the full-cache reference (every segment
    kept; 58.9 GB of cache).  One seeded draw of Q, K and V per scale serves
    all 40 layers (the per-layer draws would take 145 GB); the work per launch
    is the same as with distinct draws."""
    wl = workloads.get("c4")
    K, L = wl.n_scales, wl.layers
    if full_cache:
        keep = np.ones((L, wl.heads, K), dtype=np.uint8)
        keep[:, :, K - 1] = 0
        n_pruned = 0
    else:
        keep, _, n_pruned = hk.build_schedule(workloads.dirichlet_scas(wl), wl.scale_tokens,
                                              wl.budget, wl.n_sink)
    ctx = hk.Context(L, wl.heads, wl.head_dim, wl.batch, wl.scale_tokens, keep, torch.bfloat16)
    g = torch.Generator(device=dev)
    g.manual_seed(4)
    qs, ks, vs, outs = [], [], [], []
    for t in range(K):
        shape = (wl.batch, wl.scale_tokens[t], wl.heads, wl.head_dim)
        qs.append((torch.randn(shape, generator=g, device=dev) * wl.qk_std).to(torch.bfloat16))
        ks.append((torch.randn(shape, generator=g, device=dev) * wl.qk_std).to(torch.bfloat16))
        vs.append(torch.randn(shape, generator=g, device=dev).to(torch.bfloat16))
        outs.append(torch.empty(shape, dtype=torch.bfloat16, device=dev))
    flops = pass_flops(wl, keep, lenb_table(keep, wl.scale_tokens))
    copied = sum(compact_bytes(wl, keep, t, list(range(L))) for t in range(K - 1))

    def one_pass():
        ctx.reset()
        for t in range(K):
            for l in range(L):
                ctx.attend_append(l, t, qs[t], ks[t], vs[t], outs[t], wl.softmax_scale, stream=stream)

    one_pass()
    torch.cuda.synchronize()
    passes = 2 if full_cache else max(2, args.pruned_steps // 2)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(passes):
        one_pass()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / passes
    steps = step_profile(ctx, K, L, lambda l, t: ctx.attend_append(
        l, t, qs[t], ks[t], vs[t], outs[t], wl.softmax_scale, stream=stream),
        flops, stream, torch, passes=1)
    cache_gb = 2.0 * ctx.cache_elems * 2 / 1e9
    ctx.close()
    del qs, ks, vs, outs
    torch.cuda.empty_cache()
    budget = "full cache (every segment kept)" if full_cache else \
        f"4% budget ({n_pruned} of {L * wl.heads} heads pruned per prunable scale)"
    return {"workload": f"infinity8b-l40h28-b16: 40 layers x 28 heads x d128, batch 16, {budget}",
            "ms_per_pass": round(ms, 2),
            "scales_per_sec_per_image": round(K / (ms * 1e-3), 1),
            "image_scales_per_sec": round(K * wl.batch / (ms * 1e-3), 1),
            "attend_tflop_per_pass": round(sum(flops.values()) / 1e12, 2),
            "attend_tflops_incl_compaction": round(sum(flops.values()) / (ms * 1e-3) / 1e12, 1),
            "compaction_gb_per_pass": round(copied / 1e9, 2),
            "cache_GB": round(cache_gb, 2),
            "passes": passes,
            "per_step": steps,
            "inputs": "one seeded torch.randn draw of Q, K, V per scale, shared by the 40 layers"}


def held_table(expire, tokens):
    """Rows each (l, h) holds while step t is attended: held segments s < t."""
    import numpy as np
    L, H, K = expire.shape

    def f(t):
        out = np.zeros((L, H), dtype=np.int64)
        for s in range(min(t, K - 1)):
            out += (expire[:, :, s].astype(np.int64) >= t) * tokens[s]
        return out
    return f


def moved_rows(expire, tokens, t):
    """Rows per batch entry the gather of step t rewrites, summed over heads:
    the surviving held segments behind the first one that leaves."""
    L, H, K = expire.shape
    total = 0
    if t > K - 2:
        return 0
    for l in range(L):
        for h in range(H):
            e = expire[l, h]
            seen_drop = False
            for s in range(t):
                if e[s] < t:
                    continue
                if e[s] == t:
                    seen_drop = True
                elif seen_drop:
                    total += tokens[s]
    return total


def progressive_rate(args, hk, workloads, torch, np, dev, stream):
    """Whole-pass rate of the 32-layer, batch-8, 10%-budget workload under the
    progressive schedule (lazy prefix lengths, per-layer accounting): segments
    stay cached until the budget needs their room and then leave from the
    middle of the head's cache."""
    wl = workloads.get("c2")
    table = workloads.dirichlet_scas(wl)
    expire, prefix, live = hk.build_progressive_schedule(table, wl.scale_tokens, wl.budget,
                                                         wl.n_sink, True)
    keep, _, _ = hk.build_schedule(table, wl.scale_tokens, wl.budget, wl.n_sink)
    K = wl.n_scales
    flops = pass_flops(wl, None, held_table(expire, wl.scale_tokens))
    static_flops = pass_flops(wl, keep, lenb_table(keep, wl.scale_tokens))
    ms, cache_bytes = expiry_pass(args, hk, wl, expire, torch, dev, stream, 3)
    ms_pool, pool_bytes = expiry_pass(args, hk, wl, expire, torch, dev, stream, 3, pooled=True)
    appends = progressive_appends(args, hk, wl, expire, torch, np, dev, stream)
    row_bytes = wl.head_dim * 2
    gather_bytes = sum(moved_rows(expire, wl.scale_tokens, t) for t in range(K)) * wl.batch \
        * row_bytes * 2 * 2
    slot_bytes = wl.batch * row_bytes * 2          # one token slot of K and V, whole batch
    budget_slots = int(np.floor(wl.budget * wl.layers * wl.heads * sum(wl.scale_tokens[: K - 1])))
    return {"workload": "infinity2b-l32-b8-budget10-progressive: 32 layers x 16 heads x d128, "
                        "batch 8, 10% budget, lazy prefix lengths with per-layer accounting",
            "prefix_per_step": [int(x) for x in prefix],
            "ms_per_pass": round(ms_pool, 3),
            "scales_per_sec_per_image": round(K / (ms_pool * 1e-3), 1),
            "attend_tflops_incl_compaction": round(sum(flops.values()) / (ms_pool * 1e-3) / 1e12, 1),
            "attend_flops_vs_static": round(sum(flops.values()) / sum(static_flops.values()), 3),
            "gather_bytes_per_pass_per_head_regions": float(gather_bytes),
            "live_peak_token_slots": int(live.max()),
            "budget_token_slots": budget_slots,
            "live_peak_GB": round(int(live.max()) * slot_bytes / 1e9, 3),
            "budget_GB": round(budget_slots * slot_bytes / 1e9, 3),
            "allocated_cache_GB": round(pool_bytes / 1e9, 3),
            "allocation": "one pool shared by every head (rows of dropped segments reused, "
                          "nothing moved)",
            "per_head_regions": {"allocated_cache_GB": round(cache_bytes / 1e9, 3),
                                 "ms_per_pass": round(ms, 3),
                                 "note": "each head sized to its own peak; dropped segments "
                                         "removed by an in-place gather",
                                 "appends": appends},
            "static_allocated_cache_GB": round(hk.layout(wl.scale_tokens, keep, wl.batch,
                                                         wl.head_dim)[0] * 2 * 2 / 1e9, 3),
            "passes": args.pruned_steps}


def progressive_appends(args, hk, wl, expire, torch, np, dev, stream):
    """The appends of the progressive schedule on per-head regions, one
    all-layer hk_append_scale per completed scale, issued once every layer has
    attended the scale (the order the gather needs): the in-place gather of
    the segments that leave, then the compaction of the new scale.  GB/s of
    read + write bytes from events around each append."""
    K, L = wl.n_scales, wl.layers
    ctx = hk.Context(wl.layers, wl.heads, wl.head_dim, wl.batch, wl.scale_tokens, None,
                     torch.bfloat16, expire=expire)
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    qs, kall, vall, outs = [], [], [], []
    for t in range(K - 1):
        shape = (L, wl.batch, wl.scale_tokens[t], wl.heads, wl.head_dim)
        qs.append((torch.randn(shape[1:], generator=g, device=dev) * wl.qk_std).to(torch.bfloat16))
        kall.append((torch.randn(shape, generator=g, device=dev) * wl.qk_std).to(torch.bfloat16))
        vall.append(torch.randn(shape, generator=g, device=dev).to(torch.bfloat16))
        outs.append(torch.empty_like(qs[-1]))
    row_bytes = wl.head_dim * 2
    nbytes, gbytes = {}, {}
    for t in range(K - 1):
        stored = int((expire[:, :, t] > t).sum())
        gbytes[t] = moved_rows(expire, wl.scale_tokens, t) * wl.batch * row_bytes * 2 * 2
        nbytes[t] = gbytes[t] + stored * wl.batch * wl.scale_tokens[t] * row_bytes * 2 * 2
    ev = {t: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for t in range(K - 1)}
    times = {t: [] for t in range(K - 1)}
    for rep in range(4):
        ctx.reset()
        gpu_sleep(torch)
        for t in range(K - 1):
            for l in range(L):
                ctx.attend(l, t, qs[t], kall[t][l], vall[t][l], outs[t], wl.softmax_scale,
                           stream=stream)
            ev[t][0].record(stream)
            ctx.append_scale(0, L, t, kall[t], vall[t], stream=stream)
            ev[t][1].record(stream)
        torch.cuda.synchronize()
        if rep:
            for t in range(K - 1):
                times[t].append(ev[t][0].elapsed_time(ev[t][1]))
    ctx.close()
    ms = {t: float(np.mean(times[t])) for t in times}
    moving = [t for t in ms if gbytes[t] > 0]
    total = sum(nbytes.values())
    gbps = total / (sum(ms.values()) * 1e-3) / 1e9
    return {"what": "one all-layer append per completed scale (in-place gather, then compaction), "
                    "events around each append",
            "bytes_per_pass": float(total), "gather_bytes_per_pass": float(sum(gbytes.values())),
            "ms_per_pass": round(sum(ms.values()), 4),
            "GBps": round(gbps, 1), "frac_hbm": round(gbps / PEAK_HBM_GBPS, 4),
            "steps_with_moves_GBps": round(sum(nbytes[t] for t in moving) /
                                           (sum(ms[t] for t in moving) * 1e-3) / 1e9, 1),
            "per_step_GBps": {t: round(nbytes[t] / (ms[t] * 1e-3) / 1e9, 1) for t in ms}}


def expiry_pass(args, hk, wl, expire, torch, dev, stream, seed, keep=None, sub_blocks=None,
                pooled=False):
    """Mean time of whole passes (every layer and scale, attend_append) under
    an expiry schedule (per-head regions, or one pool shared by every head),
    or a keep-mask with 4-bit storage, on seeded GPU inputs of the workload's
    shapes.  Returns (ms, bytes of the K and V caches)."""
    if sub_blocks is None:
        ctx = hk.Context(wl.layers, wl.heads, wl.head_dim, wl.batch, wl.scale_tokens, None,
                         torch.bfloat16, expire=expire, pooled=pooled)
        cache_bytes = ctx.cache_elems * 2 * 2
    else:
        ctx = hk.Context(wl.layers, wl.heads, wl.head_dim, wl.batch, wl.scale_tokens, keep,
                         torch.bfloat16, sub_blocks=sub_blocks)
        cache_bytes = ctx.store_bytes * 2
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    K, L = wl.n_scales, wl.layers
    qs, kall, vall, outs = [], [], [], []
    for t in range(K):
        shape = (L, wl.batch, wl.scale_tokens[t], wl.heads, wl.head_dim)
        qs.append((torch.randn(shape, generator=g, device=dev) * wl.qk_std).to(torch.bfloat16))
        kall.append((torch.randn(shape, generator=g, device=dev) * wl.qk_std).to(torch.bfloat16))
        vall.append(torch.randn(shape, generator=g, device=dev).to(torch.bfloat16))
        outs.append(torch.empty(shape[1:], dtype=torch.bfloat16, device=dev))

    def one_pass():
        ctx.reset()
        for t in range(K):
            for l in range(L):
                ctx.attend_append(l, t, qs[t][l], kall[t][l], vall[t][l], outs[t], wl.softmax_scale,
                                  stream=stream)

    one_pass()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.pruned_steps):
        one_pass()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.pruned_steps
    ctx.close()
    return ms, cache_bytes


def int4_rate(args, hk, workloads, torch, np, dev, stream):
    """The 32-layer, batch-8, 10%-budget workload with its retained cache
    stored in 4 bits (one group per (scale, channel)): pass rate and cache
    bytes against the bf16 cache of the same schedule."""
    wl = workloads.get("c2")
    keep, _, _ = hk.build_schedule(workloads.dirichlet_scas(wl), wl.scale_tokens, wl.budget,
                                   wl.n_sink)
    K = wl.n_scales
    out = {"workload": "infinity2b-l32-b8-budget10-int4: the 10%-budget schedule, retained "
                       "segments stored as 4-bit codes per (scale sub-block, channel) group"}
    bf16_bytes = hk.layout(wl.scale_tokens, keep, wl.batch, wl.head_dim)[0] * 2 * 2
    for m in (1, 8):
        ms, store = expiry_pass(args, hk, wl, None, torch, dev, stream, 6, keep=keep, sub_blocks=m)
        out[f"sub_blocks_{m}"] = {"ms_per_pass": round(ms, 3),
                                  "scales_per_sec_per_image": round(K / (ms * 1e-3), 1),
                                  "cache_GB": round(store / 1e9, 3),
                                  "cache_vs_bf16": round(store / bf16_bytes, 4)}
    out["bf16_cache_GB"] = round(bf16_bytes / 1e9, 3)
    out["passes"] = args.pruned_steps
    return out


def window_rate(args, hk, workloads, torch, np, dev, stream):
    """The 32-layer, batch-8 workload under the condensed + local scale-window
    schedule: two condensed scales, a window of two local scales, and the four
    layers with the lowest (seeded, synthetic) similarity score keep every
    scale."""
    wl = workloads.get("c2")
    K, L = wl.n_scales, wl.layers
    sim = np.random.default_rng(5).random(L).astype(np.float32)
    expire = hk.build_scale_window_schedule(L, wl.heads, wl.scale_tokens, 2, 2, K, sim, 4)
    ms, cache_bytes = expiry_pass(args, hk, wl, expire, torch, dev, stream, 4)
    full = L * wl.heads * sum(wl.scale_tokens[: K - 1])
    peak = max(hk.cache_size_after_layer(wl.scale_tokens, expire, k, l)
               for k in range(K) for l in range(L))
    flops = pass_flops(wl, None, held_table(expire, wl.scale_tokens))
    return {"workload": "infinity2b-l32-b8-scale-window: 32 layers x 16 heads x d128, batch 8; "
                        "2 condensed scales, 2 local scales, 4 cache-demanding layers keep all",
            "ms_per_pass": round(ms, 3),
            "scales_per_sec_per_image": round(K / (ms * 1e-3), 1),
            "attend_tflops_incl_compaction": round(sum(flops.values()) / (ms * 1e-3) / 1e12, 1),
            "live_peak_fraction_of_full_cache": round(peak / full, 4),
            "allocated_cache_GB": round(cache_bytes / 1e9, 3),
            "passes": args.pruned_steps}


def calibration_rate(args, hk, workloads, torch, np, dev, stream):
    """Calibration workload (32 layers x 16 heads, batch 4, full cache, key
    offsets per (head, source scale)): one pass with streamed S-CAS against the
    same pass without, and the ranking stability between two calibration
    subsets (two passes on different draws)."""
    wl = workloads.get("c3")
    keep = workloads.full_keep(wl)
    K, L = wl.n_scales, wl.layers
    mu = torch.from_numpy(workloads.key_offsets(wl)).to(dev)          # [H][K]
    ctx = hk.Context(L, wl.heads, wl.head_dim, wl.batch, wl.scale_tokens, keep, torch.bfloat16)
    outs = [torch.empty((wl.batch, wl.scale_tokens[t], wl.heads, wl.head_dim), dtype=torch.bfloat16,
                        device=dev) for t in range(K)]

    def draw(seed):
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        qs, ks, vs = [], [], []
        for t in range(K):
            shape = (L, wl.batch, wl.scale_tokens[t], wl.heads, wl.head_dim)
            qs.append((torch.randn(shape, generator=g, device=dev) * wl.qk_std).to(torch.bfloat16))
            z = torch.randn(shape, generator=g, device=dev) + mu[None, None, None, :, t, None]
            ks.append((z * wl.qk_std).to(torch.bfloat16))
            vs.append(torch.randn(shape, generator=g, device=dev).to(torch.bfloat16))
        return qs, ks, vs

    def run(data, table, rec=None):
        qs, ks, vs = data
        ctx.reset()
        for t in range(K):
            for l in range(L):
                if rec is not None and t == K - 1:
                    rec[l][0].record(stream)
                if table is None:
                    ctx.attend(l, t, qs[t][l], ks[t][l], vs[t][l], outs[t], 1.0, stream=stream)
                else:
                    ctx.attend_with_scas_sum(l, t, qs[t][l], ks[t][l], vs[t][l], outs[t], 1.0, table,
                                             stream=stream)
                if rec is not None and t == K - 1:
                    rec[l][1].record(stream)
            if t < K - 1:
                ctx.append_scale(0, L, t, ks[t], vs[t], stream=stream)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    data = draw(11)
    scratch = torch.zeros((L, wl.heads, K, K), dtype=torch.float64, device=dev)
    ms_plain = timed(lambda: run(data, None), 2)
    ms_scas = timed(lambda: run(data, scratch), 2)
    # The final-scale attention launches of the plain pass (batch 4, 4,096
    # queries x 10,521 keys per head), each timed with events on the launch
    # stream, the pass queued behind a spin kernel; median over 3 passes.
    final = []
    for _ in range(3):
        rec = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(L)]
        gpu_sleep(torch)
        run(data, None, rec)
        torch.cuda.synchronize()
        final += [r[0].elapsed_time(r[1]) for r in rec]
    final_flops = 4.0 * wl.head_dim * wl.scale_tokens[-1] * sum(wl.scale_tokens) * wl.heads * wl.batch
    final_us = float(np.median(final)) * 1e3
    final_tflops = final_flops / (final_us * 1e-6) / 1e12
    final_plan = list(ctx.attend_plan(K - 1))
    tables = []
    for seed in (21, 22):
        tab = torch.zeros((L, wl.heads, K, K), dtype=torch.float64, device=dev)
        run(draw(seed), tab)
        torch.cuda.synchronize()
        tables.append(hk.scas_mean(tab.cpu().numpy(), wl.batch))
    rho, jac = hk.ranking_stability(tables[0], tables[1], wl.scale_tokens, 0.10, 2)
    ctx.close()
    return {"workload": "infinity2b-l32-b4-calibration: 32 layers x 16 heads, batch 4, full cache",
            "ms_per_pass_attend": round(ms_plain, 3), "ms_per_pass_with_scas": round(ms_scas, 3),
            "scas_overhead_ratio": round(ms_scas / ms_plain, 3),
            "final_scale_attend": {"what": "final-scale attend launch without S-CAS (batch 4), median "
                                           "of per-launch events over 3 passes x 32 layers",
                                   "plan": final_plan,
                                   "median_us": round(final_us, 2),
                                   "flops_per_launch": final_flops,
                                   "achieved_tflops": round(final_tflops, 2),
                                   "frac": round(final_tflops / PEAK_BF16_TFLOPS, 4)},
            "ranking_stability": {"subsets": "two batches of 4 images (different draws)",
                                  "spearman_rho_per_source_scale": {s: round(float(r), 4) for s, r in enumerate(rho)
                                                                    if not np.isnan(r)},
                                  "jaccard_pruned_at_10pct": round(jac, 4)}}


def compact_rate(args, hk, workloads, torch, np, dev, stream):
    """Standalone compaction (hk_append_scale over all 32 layers per completed
    scale) of the batch-4 full-cache workload: 13.5 GB moved per pass."""
    wl = workloads.get("c3")
    keep = workloads.full_keep(wl)
    ctx = hk.Context(wl.layers, wl.heads, wl.head_dim, wl.batch, wl.scale_tokens, keep,
                     torch.bfloat16)
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    K, L = wl.n_scales, wl.layers
    kall, vall = [], []
    for t in range(K - 1):
        shape = (L, wl.batch, wl.scale_tokens[t], wl.heads, wl.head_dim)
        kall.append(torch.randn(shape, generator=g, device=dev).to(torch.bfloat16))
        vall.append(torch.randn(shape, generator=g, device=dev).to(torch.bfloat16))
    nbytes = {t: compact_bytes(wl, keep, t, slice(0, L)) for t in range(K - 1)}
    ev = {t: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for t in range(K - 1)}
    times = {t: [] for t in range(K - 1)}
    for rep in range(4):
        ctx.reset()
        # The spin kernel holds the GPU while the host queues the pass, so the
        # events time the launches, not the host's calls between them (the
        # early scales move a few MB and would otherwise wait on the host).
        gpu_sleep(torch)
        for t in range(K - 1):
            ev[t][0].record(stream)
            ctx.append_scale(0, L, t, kall[t], vall[t], stream=stream)
            ev[t][1].record(stream)
        torch.cuda.synchronize()
        if rep:
            for t in range(K - 1):
                times[t].append(ev[t][0].elapsed_time(ev[t][1]))
    # The whole pass: one event pair around the 12 appends (the per-step
    # events above each add a few microseconds between launches).
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    whole = []
    for rep in range(4):
        ctx.reset()
        gpu_sleep(torch)
        e0.record(stream)
        for t in range(K - 1):
            ctx.append_scale(0, L, t, kall[t], vall[t], stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        if rep:
            whole.append(e0.elapsed_time(e1))
    whole_gbps = sum(nbytes.values()) / (float(np.mean(whole)) * 1e-3) / 1e9
    ms = {t: float(np.mean(times[t])) for t in times}
    big = max(nbytes, key=lambda t: nbytes[t])
    total = sum(nbytes.values()) / (sum(ms.values()) * 1e-3) / 1e9
    bigr = nbytes[big] / (ms[big] * 1e-3) / 1e9
    ctx.close()
    return {"workload": "infinity2b-l32-b4 full cache: one all-layer append per completed scale",
            "bound": "hbm", "GBps": round(total, 1), "frac_hbm": round(total / PEAK_HBM_GBPS, 4),
            "timing": "GBps: bytes of the pass over the sum of per-append event times; "
                      "whole_pass: one event pair around the pass's appends",
            "whole_pass_GBps": round(whole_gbps, 1),
            "whole_pass_frac_hbm": round(whole_gbps / PEAK_HBM_GBPS, 4),
            "largest_step": big, "largest_step_bytes": nbytes[big],
            "largest_step_GBps": round(bigr, 1), "largest_step_frac_hbm": round(bigr / PEAK_HBM_GBPS, 4),
            "per_step_GBps": {t: round(nbytes[t] / (ms[t] * 1e-3) / 1e9, 1) for t in ms}}


def _oracle_sample(wl, keep, layer, batches, heads, passes=1, with_scas=False):
    """Runs the fp64 oracle over every scale of the given (batch entry, head)
    units of one layer; returns (algorithmic flops, seconds)."""
    import workloads
    from oracle import attention as oatt
    from oracle.numerics import to_f64

    steps = [workloads.step_inputs(wl, layer, t, batch=max(batches) + 1) for t in range(wl.n_scales)]
    flops = 0.0
    start = time.perf_counter()
    for _ in range(passes):
        for t in range(wl.n_scales):
            for b in batches:
                for h in heads:
                    kj, vj, src, lens = oatt.gather_keys([s.k for s in steps[: t + 1]],
                                                         [s.v for s in steps[: t + 1]], keep[layer, h],
                                                         t, b, h)
                    q = to_f64(steps[t].q[b, :, h, :], wl.dtype)
                    _, prob = oatt.softmax_attention(q, to_f64(kj, wl.dtype), to_f64(vj, wl.dtype),
                                                     wl.softmax_scale)
                    if with_scas:
                        oatt.segment_mass(prob, src, lens, t)
                    flops += 4.0 * wl.head_dim * q.shape[0] * kj.shape[0]
    return flops, time.perf_counter() - start


def _oracle_keep(wl):
    """The workload's keep-mask, built by the oracle's own schedule."""
    import workloads
    from oracle import schedule as osch
    if wl.schedule == "random_drop2":
        return workloads.random_drop2_keep(wl)
    if wl.schedule == "full":
        return workloads.full_keep(wl)
    return osch.build_schedule(workloads.dirichlet_scas(wl), wl.scale_tokens, wl.budget, wl.n_sink)[0]


def cpu_baseline(args, wl, keep):
    """The fp64 oracle, as it stands, on the host cores: the main workload's
    whole pass, and a bounded sample of every other workload, whose time for
    the whole workload is extrapolated by algorithmic flops (labelled)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import workloads

    blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    host = len(os.sched_getaffinity(0))
    heads = list(range(min(args.cpu_heads, wl.heads)))
    passes = max(1, args.cpu_passes)
    flops, secs = _oracle_sample(wl, keep, 0, [0], heads, passes=passes)
    out = {"value": round(flops / secs / 1e12, 5), "unit": "TFLOP/s", "cores": host,
           "blas_threads": int(blas), "kind": "oracle", "seconds": round(secs, 2),
           "sample": f"full-cache layer, batch 1, all 13 scales of heads {heads[0]}..{heads[-1]} "
                     f"({len(heads)} of {wl.heads}), fp64 NumPy, {passes} pass(es)"}
    per = {}
    # (workload, layer, batch entries, heads, S-CAS) of each sample
    plan = [("c0", 0, [0], None, True), ("c2", 0, [0], 8, False), ("c3", 0, [0], None, True),
            ("c4", 0, [0], 8, False)]
    for key, layer, batches, nh, scas in plan:
        w = workloads.get(key)
        kp = _oracle_keep(w)
        hs = list(range(w.heads)) if nh is None else [int(x) for x in
                                                     np.linspace(0, w.heads - 1, nh).round()]
        f, sec = _oracle_sample(w, kp, layer, batches, hs, with_scas=scas)
        full = sum(pass_flops(w, kp, lenb_table(kp, w.scale_tokens)).values())
        whole = len(batches) * len(hs) == w.batch * w.heads and w.layers == 1
        per[key] = {"workload": w.name, "sample": f"layer {layer}, batch entries {batches}, heads "
                                                  f"{hs[0]}..{hs[-1]} ({len(hs)} of {w.heads}), all "
                                                  f"{w.n_scales} scales" + (", S-CAS" if scas else ""),
                    "sample_seconds": round(sec, 3), "sample_tflop": round(f / 1e12, 5),
                    "TFLOP_per_s": round(f / sec / 1e12, 5),
                    "seconds_per_pass": round(sec * full / f, 2),
                    "seconds_per_pass_is": "measured" if whole else
                    "extrapolated by algorithmic flops from the sample",
                    "pass_tflop": round(full / 1e12, 3)}
    out["per_workload"] = per
    return out


if __name__ == "__main__":
    main()
