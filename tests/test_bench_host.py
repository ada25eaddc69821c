"""Host logic of bench.py, on the CPU: the one-GPU refusal, the algorithmic
work it divides by, and the selection and scaling of the rocprofv3 summaries
that the committed profiles come from (synthetic CSVs)."""
import csv
import importlib.util
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def full_keep(wl):
    keep = np.ones((wl.layers, wl.heads, wl.n_scales), dtype=np.uint8)
    keep[:, :, -1] = 0
    return keep


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"] and msg["n_gpus"] == 2


def test_attention_flops_of_the_full_cache_layer(bench):
    """4 d n_t (held + n_t) per (b, h): 0.561 TFLOP over the 13 scales of the
    16-head full-cache layer, 0.353 TFLOP at the final scale."""
    wl = workloads.get("c1")
    keep = full_keep(wl)
    flops = bench.pass_flops(wl, keep, bench.lenb_table(keep, wl.scale_tokens))
    st = wl.scale_tokens
    by_hand = [4.0 * 128 * st[t] * sum(st[: t + 1]) * 16 for t in range(wl.n_scales)]
    assert [flops[(0, t)] for t in range(wl.n_scales)] == pytest.approx(by_hand, rel=0, abs=0)
    assert sum(by_hand) / 1e12 == pytest.approx(0.561, abs=5e-4)
    assert by_hand[-1] / 1e12 == pytest.approx(0.353, abs=5e-4)


def test_attention_flops_skip_dropped_segments(bench):
    wl = workloads.get("c1")
    keep = full_keep(wl)
    keep[0, 3, 5] = 0       # head 3 drops scale 5: later scales read n_5 fewer keys
    flops = bench.pass_flops(wl, keep, bench.lenb_table(keep, wl.scale_tokens))
    full = bench.pass_flops(wl, full_keep(wl), bench.lenb_table(full_keep(wl), wl.scale_tokens))
    st = wl.scale_tokens
    for t in range(wl.n_scales):
        missing = 4.0 * 128 * st[t] * st[5] if t > 5 else 0.0
        assert full[(0, t)] - flops[(0, t)] == missing


@pytest.mark.parametrize("key,total_gb", [("c2", 2.65), ("c3", 13.47), ("c4", 4.61)])
def test_compaction_bytes(bench, key, total_gb):
    """2 (read + write) x 2 (K, V) x kept (l, h) x B x n_t x d x 2 bytes, summed
    over the appended scales 0..K-2."""
    wl = workloads.get(key)
    if wl.schedule == "dirichlet":
        from oracle import schedule as osch
        keep = osch.build_schedule(workloads.dirichlet_scas(wl), wl.scale_tokens, wl.budget, wl.n_sink)[0]
    else:
        keep = full_keep(wl)
    total = sum(bench.compact_bytes(wl, keep, t, list(range(wl.layers))) for t in range(wl.n_scales - 1))
    assert total / 1e9 == pytest.approx(total_gb, abs=0.005)
    assert bench.compact_bytes(wl, keep, wl.n_scales - 1, list(range(wl.layers))) == 0.0


def _write_csv(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_trace_summary_takes_the_final_scale_launches(bench, tmp_path):
    """Of the roofline kernel's dispatches, only those with the largest grid
    (the final scale) are averaged; the split instantiation and other kernels
    are ignored."""
    hdr = ["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp",
           "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]
    k = "void hk::(anonymous namespace)::" + bench.ROOFLINE_KERNEL + "(hk::AttendArgs)"
    split = "void hk::(anonymous namespace)::attend_q256_kernel<false, true, false, true>(hk::AttendArgs)"
    rows = [["KERNEL_DISPATCH", 1, k, 0, 9000, 8192, 1, 1],         # a small scale
            ["KERNEL_DISPATCH", 2, split, 0, 500000, 221184, 1, 1],  # a split launch, larger grid
            ["KERNEL_DISPATCH", 3, k, 100, 330100, 131072, 1, 1],
            ["KERNEL_DISPATCH", 4, k, 200, 332200, 131072, 1, 1],
            ["KERNEL_DISPATCH", 5, "attend_combine_kernel", 0, 7000, 4096, 1, 1]]
    path = tmp_path / "trace.csv"
    _write_csv(path, hdr, rows)
    s = bench.summarize_trace(str(path))
    assert s["grid_threads"] == 131072 and s["dispatches"] == 2
    assert s["avg_ns"] == pytest.approx(331000.0)
    assert s["other_dispatches_of_kernel"] == 1


def test_counter_summary_scales_by_the_copy_probe(bench, tmp_path):
    """Per-dispatch FETCH_SIZE and WRITE_SIZE (summed over the rows of a
    dispatch) of the final-scale launches, scaled so that the probe's 1 GiB
    copies read 1 GiB: FETCH x 2 when the probe's FETCH reads half."""
    hdr = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    k = bench.ROOFLINE_KERNEL
    gib_kib = float(1 << 20)
    fetch = [[1, k, 8192, "FETCH_SIZE", 10.0],                     # a small scale: ignored
             [2, k, 131072, "FETCH_SIZE", 30000.0], [2, k, 131072, "FETCH_SIZE", 20000.0],
             [3, k, 131072, "FETCH_SIZE", 50000.0]]
    write = [[2, k, 131072, "WRITE_SIZE", 16000.0], [3, k, 131072, "WRITE_SIZE", 16000.0]]
    cfetch = [[1, "__amd_rocclr_copyBuffer", 512, "FETCH_SIZE", gib_kib / 2]]
    cwrite = [[1, "__amd_rocclr_copyBuffer", 512, "WRITE_SIZE", gib_kib]]
    paths = []
    for name, rows in (("f", fetch), ("w", write), ("cf", cfetch), ("cw", cwrite)):
        p = tmp_path / f"{name}.csv"
        _write_csv(p, hdr, rows)
        paths.append(str(p))
    s = bench.summarize_counters(paths)
    assert s["dispatches"] == [2, 2]
    assert s["fetch_scale"] == pytest.approx(2.0) and s["write_scale"] == pytest.approx(1.0)
    assert s["bytes_per_launch"] == round((50000.0 * 2 + 16000.0) * 1024)
    assert s["kernel_sha256"] == bench.attend_sources_sha()


def test_pass_summary_takes_the_fused_passes(bench, tmp_path):
    """Launches between consecutive final-scale dispatches form one pass; a
    pass that holds a compaction kernel (the unfused pass) is left out, and
    each launch's duration is the median over the passes."""
    hdr = ["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp",
           "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]
    k = "void hk::(anonymous namespace)::" + bench.ROOFLINE_KERNEL + "(hk::AttendArgs)"
    small = "void hk::(anonymous namespace)::attend_q128_kernel<false, false>(hk::AttendArgs)"
    rows, t, did = [], 0, 0

    def add(name, dur, grid):
        nonlocal t, did
        did += 1
        rows.append(["KERNEL_DISPATCH", did, name, t, t + dur, grid, 1, 1])
        t += dur + 100

    add(k, 300000, 131072)
    for small_ns, final_ns in ((5000, 320000), (7000, 330000), (6000, 340000)):
        add(small, small_ns, 4096)
        add(k, final_ns, 131072)
    add("void hk::compact_rows_kernel(hk::RowsArgs)", 4000, 8192)   # an unfused pass
    add(small, 90000, 4096)
    add(k, 900000, 131072)
    path = tmp_path / "trace.csv"
    _write_csv(path, hdr, rows)
    s = bench.summarize_pass(str(path))
    assert s["passes"] == 3
    assert [x["kernel"] for x in s["launches"]] == ["attend_q128_kernel<false, false>", bench.ROOFLINE_KERNEL]
    assert [x["median_us"] for x in s["launches"]] == [6.0, 330.0]
    assert s["sum_median_us"] == 336.0
