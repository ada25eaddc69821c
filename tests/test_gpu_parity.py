"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Tolerances: bf16 attention output max-abs <= 1e-2 and mean-abs <= 1e-3;
fp32 attention output max-abs <= 1e-5; S-CAS <= 1e-4 absolute; keep-masks
and compacted caches bit-exact.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import schedule as osch
from oracle.numerics import to_f64

import kv_cache_compression_attend_amd as hk
from _gpu import (check_cache, generate, gpu_rows, note, oracle_rows, sample_rows, to_device,
                  torch_dtype)

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN, F32_MAX, SCAS_TOL = 1e-2, 1e-3, 1e-5, 1e-4


def _tol(wl):
    return (BF16_MAX, BF16_MEAN) if wl.dtype == "bf16" else (F32_MAX, F32_MAX)


def _compare_outputs(run, layers, rows_per_unit=96, bh=None, seed=0, own_rounding=False):
    """Outputs against the oracle on sampled rows: max-abs <= tmax and
    mean-abs <= tmean per (layer, scale).  own_rounding adds, element by
    element, half an ulp of bf16 at the oracle's value (2^-8 |want|), the
    error the bf16 output itself carries, for inputs whose outputs reach
    magnitudes where that half-ulp is not small against tmax."""
    wl = run.wl
    tmax, tmean = _tol(wl)
    worst = 0.0
    for l in layers:
        for t in range(wl.n_scales):
            n = wl.scale_tokens[t]
            rows = sample_rows(n, rows_per_unit, seed + 31 * t + l)
            pairs = bh if bh is not None else [(b, h) for b in range(wl.batch) for h in range(wl.heads)]
            err_sum, err_cnt = 0.0, 0
            for b, h in pairs:
                want, _ = oracle_rows(run, l, t, b, h, rows)
                got = gpu_rows(run, l, t, b, h, rows)
                assert np.isfinite(got).all(), (l, t, b, h)
                e = np.abs(got - want)
                worst = max(worst, float(e.max()))
                bound = tmax + (np.abs(want) * 2.0 ** -8 if own_rounding else 0.0)
                assert (e <= bound).all(), (l, t, b, h, float(e.max()), float(np.max(e - bound)))
                err_sum += float(e.sum())
                err_cnt += e.size
            assert err_sum / err_cnt <= tmean, (l, t, err_sum / err_cnt)
    return worst


def _compare_scas(run, l, steps=None, heads=None, tol=SCAS_TOL):
    wl = run.wl
    steps = range(wl.n_scales) if steps is None else steps
    heads = range(wl.heads) if heads is None else heads
    for t in steps:
        rows = np.arange(wl.scale_tokens[t])
        for h in heads:
            mass = np.zeros(t + 1)
            for b in range(wl.batch):
                _, m = oracle_rows(run, l, t, b, h, rows)
                mass += m
            mass /= wl.batch
            got = run.scas[l, h, t, : t + 1].astype(np.float64)
            np.testing.assert_allclose(got, mass, atol=tol, rtol=0, err_msg=f"l{l} h{h} t{t}")
            for s in range(t):
                if not run.keep[l, h, s]:
                    assert run.scas[l, h, t, s] == 0.0
            assert (run.scas[l, h, t, t + 1:] == 0).all()


def _schedule(wl):
    if wl.schedule == "random_drop2":
        return workloads.random_drop2_keep(wl)
    if wl.schedule == "full":
        keep, _, n = hk.build_schedule(workloads.dirichlet_scas(wl), wl.scale_tokens, 1.0, wl.n_sink)
        assert n == 0
        return keep
    table = workloads.dirichlet_scas(wl)
    keep, ret, n = hk.build_schedule(table, wl.scale_tokens, wl.budget, wl.n_sink)
    want = osch.build_schedule(table, wl.scale_tokens, wl.budget, wl.n_sink)
    np.testing.assert_array_equal(keep, want[0])
    return keep


def _custom(index, name, sides, heads, head_dim, batch, dtype, layers=1, alpha=None):
    return workloads.Workload(
        index=index, name=name, layers=layers, heads=heads, head_dim=head_dim, batch=batch,
        sides=tuple(sides), dtype=dtype, budget=1.0, n_sink=1,
        softmax_scale=alpha if alpha is not None else (1.0 if dtype == "bf16" else head_dim ** -0.5),
        qk_std=head_dim ** -0.25 if dtype == "bf16" else 1.0, schedule="custom")


def _random_keep(wl, seed, p=0.5):
    g = np.random.default_rng(seed)
    keep = (g.random((wl.layers, wl.heads, wl.n_scales)) < p).astype(np.uint8)
    keep[:, :, 0] = 1
    keep[:, :, -1] = 0
    keep[0, 0, 1:] = 0  # one head keeps only the sink
    return keep


def test_tiny_f32_workload():
    wl = workloads.get("c0")
    keep = _schedule(wl)
    run = generate(wl, keep, [0], scas=True)
    _compare_outputs(run, [0])
    _compare_scas(run, 0, tol=1e-5)
    check_cache(run, [0])
    run.ctx.close()


def test_infinity2b_layer_full_cache():
    """Every output row of every head and scale against the oracle."""
    wl = workloads.get("c1")
    keep = _schedule(wl)
    run = generate(wl, keep, [0])
    worst = _compare_outputs(run, [0], rows_per_unit=max(wl.scale_tokens))
    note(f"c1 worst max-abs {worst:.3e}")
    check_cache(run, [0])
    run.ctx.close()


@pytest.mark.parametrize("D", [16, 32, 64, 128])
def test_f32_head_dims_ragged(D):
    wl = _custom(20 + D, f"ragged-f32-d{D}", (1, 3, 5, 7, 9), heads=3, head_dim=D, batch=2,
                 dtype="f32", layers=2)
    keep = _random_keep(wl, D)
    run = generate(wl, keep, [0, 1], scas=True, multi_layer_append=True)
    _compare_outputs(run, [0, 1])
    for l in (0, 1):
        _compare_scas(run, l, tol=1e-5)
    check_cache(run, [0, 1])
    run.ctx.close()


@pytest.mark.parametrize("scas", [True, False])
@pytest.mark.parametrize("seed", [0, 1])
def test_bf16_ragged_tiles_and_junctions(seed, scas):
    """Scale sizes that are not multiples of the 128-query / 64-key tiles, cache
    lengths that end mid-tile, heads that keep nothing but the sink.  Without
    S-CAS the small launches split their key range (merged afterwards)."""
    wl = _custom(30 + seed, f"ragged-bf16-{seed}", (1, 3, 5, 7, 11, 13, 17, 19, 23), heads=5,
                 head_dim=128, batch=3, dtype="bf16", layers=3)
    keep = _random_keep(wl, 100 + seed)
    run = generate(wl, keep, [0, 1, 2], scas=scas, multi_layer_append=bool(seed))
    _compare_outputs(run, [0, 1, 2], rows_per_unit=400)
    if scas:
        for l in range(3):
            _compare_scas(run, l)
    check_cache(run, [0, 1, 2])
    run.ctx.close()


@pytest.mark.parametrize("seed", [0, 1])
def test_bf16_ragged_wide_launch(seed):
    """Enough (batch, head) pairs that the launch takes the 256-query,
    8-wave pipelined tiling: scale sizes off the 256-query and 64-key grids,
    junctions mid-tile, single-tile and many-tile heads, S-CAS on."""
    wl = _custom(60 + seed, f"ragged-wide-{seed}", (1, 3, 7, 13, 23), heads=16, head_dim=128,
                 batch=16, dtype="bf16", layers=1)
    keep = _random_keep(wl, 200 + seed)
    run = generate(wl, keep, [0], scas=True)
    pairs = [(b, h) for b in (0, 5, 15) for h in range(16)]
    _compare_outputs(run, [0], rows_per_unit=600, bh=pairs)
    _compare_scas(run, 0, steps=(3, 4), heads=(0, 1, 7, 15))
    check_cache(run, [0])
    run.ctx.close()


@pytest.mark.parametrize("heads", [28, 48, 100])
def test_token_block_compaction_head_counts(heads):
    """All-layer appends of scales that most heads store go through the token
    blocks: two tokens per workgroup at 28 heads (896 vectors, a partial
    fourth slot per lane), one token at 48 (768) and at 100 (1,600 vectors,
    two passes per workgroup).  One head drops a scale, so the blocks also
    skip a head.  Cache bit for bit, outputs against the oracle."""
    wl = _custom(100 + heads, f"token-blocks-h{heads}", (1, 3, 5, 8, 11), heads=heads, head_dim=128,
                 batch=2, dtype="bf16", layers=2)
    keep = np.ones((wl.layers, wl.heads, wl.n_scales), dtype=np.uint8)
    keep[:, :, -1] = 0
    keep[:, 1, 2] = 0
    run = generate(wl, keep, [0, 1], multi_layer_append=True)
    pairs = [(b, h) for b in range(wl.batch) for h in (0, 1, heads // 2, heads - 1)]
    _compare_outputs(run, [0, 1], rows_per_unit=32, bh=pairs)
    check_cache(run, [0, 1])
    run.ctx.close()


@pytest.mark.parametrize("case", ["full-b1", "pruned-b8", "ragged-f32", "ragged-bf16-scas", "wide-scas"])
def test_fused_attend_append(case):
    """attend_append (attention and this scale's append in one call) leaves the
    same cache as attend + append_scale and the same outputs, across both bf16
    tilings, split launches, junctions, pruned heads and the fp32 path."""
    if case == "full-b1":
        wl, layers, scas = workloads.get("c1"), [0], False
        keep = _schedule(wl)
    elif case == "pruned-b8":
        wl, layers, scas = workloads.get("c2"), [5], False
        keep = _schedule(wl)
    elif case == "ragged-f32":
        wl = _custom(70, "fused-f32", (1, 3, 5, 7, 9), heads=3, head_dim=16, batch=2, dtype="f32", layers=2)
        keep, layers, scas = _random_keep(wl, 70), [0, 1], True
    elif case == "ragged-bf16-scas":
        wl = _custom(71, "fused-bf16", (1, 3, 5, 7, 11, 13, 17, 19, 23), heads=5, head_dim=128,
                     batch=3, dtype="bf16", layers=2)
        keep, layers, scas = _random_keep(wl, 71), [0, 1], True
    else:
        wl = _custom(72, "fused-wide", (1, 3, 7, 13, 23), heads=16, head_dim=128, batch=16,
                     dtype="bf16", layers=1)
        keep, layers, scas = _random_keep(wl, 72), [0], True
    run = generate(wl, keep, layers, scas=scas, fused=True)
    pairs = None if wl.batch * wl.heads <= 16 else [(b, h) for b in (0, wl.batch - 1) for h in range(wl.heads)]
    _compare_outputs(run, layers, rows_per_unit=64, bh=pairs)
    if scas:
        for l in layers:
            _compare_scas(run, l, steps=range(min(wl.n_scales, 5)), heads=range(min(wl.heads, 4)),
                          tol=1e-5 if wl.dtype == "f32" else SCAS_TOL)
    check_cache(run, layers)
    run.ctx.close()


def test_fused_append_order_errors():
    wl = _custom(73, "fused-errors", (1, 2, 3), heads=2, head_dim=128, batch=1, dtype="bf16")
    keep = np.ones((1, 2, 3), dtype=np.uint8)
    ctx = hk.Context(1, 2, 128, 1, wl.scale_tokens, keep, torch.bfloat16)
    mk = lambda t: torch.zeros((1, wl.scale_tokens[t], 2, 128), dtype=torch.bfloat16, device="cuda")  # noqa
    ctx.attend_append(0, 0, mk(0), mk(0), mk(0), mk(0), 1.0)
    with pytest.raises(hk.HeatKVError) as e:          # scale 0 already appended
        ctx.append_scale(0, 1, 0, mk(0), mk(0))
    assert e.value.status == hk.HK_EORDER
    ctx.attend(0, 1, mk(1), mk(1), mk(1), mk(1), 1.0)  # allowed: scale 0 is cached
    ctx.append_scale(0, 1, 1, mk(1), mk(1))
    with pytest.raises(hk.HeatKVError) as e:          # scale 1 appended twice
        ctx.attend_append(0, 1, mk(1), mk(1), mk(1), mk(1), 1.0)
    assert e.value.status == hk.HK_EORDER
    ctx.attend_append(0, 2, mk(2), mk(2), mk(2), mk(2), 1.0)  # final scale: attention only
    assert ctx.retained_tokens(2) == 2 * (1 + 4)
    torch.cuda.synchronize()
    ctx.close()


def test_streaming_calibration_over_batches():
    """attend_with_scas_sum over three batches of calibration images, then the
    mean over all images, equals the oracle's per-image S-CAS averaged over
    every image of the three batches."""
    wl = _custom(80, "calib-stream", (1, 2, 3, 5, 8), heads=4, head_dim=128, batch=2,
                 dtype="bf16", layers=2)
    keep = _random_keep(wl, 80)
    K = wl.n_scales
    total = torch.zeros((2, 4, K, K), dtype=torch.float64, device="cuda")
    want = np.zeros((2, 4, K, K))
    n_img = 0
    for seed in (11, 12, 13):
        ctx = hk.Context(2, 4, 128, 2, wl.scale_tokens, keep, torch.bfloat16)
        ins = {l: [workloads.step_inputs(wl, l, t, seed) for t in range(K)] for l in range(2)}
        for t in range(K):
            for l in range(2):
                x = ins[l][t]
                q, k, v = to_device(x.q, wl), to_device(x.k, wl), to_device(x.v, wl)
                out = torch.empty_like(q)
                note(f"calib-stream seed {seed} layer {l} step {t}")
                ctx.attend_with_scas_sum(l, t, q, k, v, out, 1.0, total)
                if t < K - 1:
                    ctx.append_scale(l, l + 1, t, k, v)
        torch.cuda.synchronize()
        ctx.close()
        from oracle import attention as oatt
        for l in range(2):
            for t in range(K):
                for h in range(4):
                    for b in range(2):
                        kj, vj, src, lens = oatt.gather_keys([x.k for x in ins[l][: t + 1]],
                                                             [x.v for x in ins[l][: t + 1]], keep[l, h], t, b, h)
                        _, p = oatt.softmax_attention(to_f64(ins[l][t].q[b, :, h, :], "bf16"),
                                                      to_f64(kj, "bf16"), to_f64(vj, "bf16"), 1.0)
                        want[l, h, t, : t + 1] += oatt.segment_mass(p, src, lens, t)
        n_img += 2
    got = hk.scas_mean(total.cpu().numpy(), n_img)
    np.testing.assert_allclose(got, want / n_img, atol=SCAS_TOL, rtol=0)
    for l in range(2):
        for h in range(4):
            for t in range(K):
                np.testing.assert_allclose(got[l, h, t, : t + 1].sum(), 1.0, atol=1e-4)
                for s in range(t):
                    if not keep[l, h, s]:
                        assert got[l, h, t, s] == 0.0


def test_maximum_scale_count_with_scas():
    """HK_MAX_SCALES = 16 scales (every S-CAS accumulator in use), random
    pruning, fused attend_append with S-CAS; outputs, S-CAS and cache."""
    wl = _custom(84, "max-scales", tuple(range(1, 17)), heads=2, head_dim=128, batch=1, dtype="bf16")
    assert wl.n_scales == hk.HK_MAX_SCALES
    keep = _random_keep(wl, 84, p=0.7)
    run = generate(wl, keep, [0], scas=True, fused=True)
    _compare_outputs(run, [0], rows_per_unit=48)
    _compare_scas(run, 0)
    check_cache(run, [0])
    run.ctx.close()


def test_one_head_batch_one():
    wl = _custom(85, "one-head", (1, 2, 3, 5, 8, 13), heads=1, head_dim=128, batch=1, dtype="bf16")
    keep = np.ones((1, 1, wl.n_scales), dtype=np.uint8)
    keep[0, 0, -1] = 0
    keep[0, 0, 2] = 0
    run = generate(wl, keep, [0], scas=True)
    _compare_outputs(run, [0])
    _compare_scas(run, 0)
    check_cache(run, [0])
    run.ctx.close()


def test_graph_capture_replays_match_eager():
    """A whole pass (attend_append of every scale, with key-range splits and
    the fused append) captured into a HIP graph replays to the eager result,
    replay after replay, with eager passes in between: the per-scale calls
    allocate nothing and record no memset nodes."""
    wl = _custom(86, "graph", (1, 2, 4, 6, 8, 12, 16, 20, 24), heads=4, head_dim=128, batch=1,
                 dtype="bf16")
    keep = _random_keep(wl, 86, p=0.8)
    ctx = hk.Context(1, wl.heads, 128, 1, wl.scale_tokens, keep, torch.bfloat16)
    assert any(ctx.attend_plan(t)[1] > 1 for t in range(wl.n_scales)), "no split launch covered"
    xs = [workloads.step_inputs(wl, 0, t, 0) for t in range(wl.n_scales)]
    dev = [tuple(to_device(a, wl) for a in (x.q, x.k, x.v)) for x in xs]
    outs = [torch.empty_like(d[0]) for d in dev]

    def one_pass():
        ctx.reset()
        for t, (q, k, v) in enumerate(dev):
            ctx.attend_append(0, t, q, k, v, outs[t], wl.softmax_scale)

    one_pass()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        one_pass()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        one_pass()
    torch.cuda.synchronize()
    for rep in range(5):
        for o in outs:
            o.zero_()
        note(f"graph replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        for t, (a_, b_) in enumerate(zip(outs, ref)):
            assert torch.equal(a_, b_), (rep, t)
        one_pass()
        torch.cuda.synchronize()
    del graph
    ctx.close()


def test_single_scale_workload():
    wl = _custom(40, "single-scale", (9,), heads=2, head_dim=128, batch=2, dtype="bf16")
    keep = np.zeros((1, 2, 1), dtype=np.uint8)
    run = generate(wl, keep, [0], scas=True)
    _compare_outputs(run, [0])
    _compare_scas(run, 0)
    run.ctx.close()


def test_pruned_10pct_full_size_layers():
    """32 layers x 16 heads, batch 8, 10% budget; two layers run end to end."""
    wl = workloads.get("c2")
    keep = _schedule(wl)
    layers = [0, 13]
    run = generate(wl, keep, layers)
    pairs = [(b, h) for b in (0, 3, 7) for h in range(16)]
    _compare_outputs(run, layers, rows_per_unit=48, bh=pairs)
    check_cache(run, layers)
    run.ctx.close()


def test_calibration_full_size_scas():
    """32 x 16 heads, batch 4, full cache, S-CAS on; key offsets make rankings non-uniform."""
    wl = workloads.get("c3")
    keep = _schedule(wl)
    run = generate(wl, keep, [0], scas=True)
    pairs = [(b, h) for b in range(4) for h in (0, 5, 10, 15)]
    _compare_outputs(run, [0], rows_per_unit=48, bh=pairs)
    _compare_scas(run, 0, steps=range(wl.n_scales))
    table = run.scas[0]
    for t in range(wl.n_scales):
        np.testing.assert_allclose(table[:, t, : t + 1].sum(axis=1), 1.0, atol=1e-4)
    run.ctx.close()


# Batch entries that fall on each of the 8 dies when a launch runs its heads
# heaviest first (die x takes entries [2x, 2x + 2) at batch 16).
PER_DIE_16 = (0, 3, 4, 7, 8, 11, 12, 15)


def test_infinity8b_shape_4pct_layer():
    """40 layers x 28 heads, batch 16, 4% budget; one layer end to end, every
    head of one batch entry on each die."""
    wl = workloads.get("c4")
    keep = _schedule(wl)
    run = generate(wl, keep, [7])
    pairs = [(b, h) for b in PER_DIE_16 for h in range(28)]
    _compare_outputs(run, [7], rows_per_unit=32, bh=pairs)
    check_cache(run, [7])
    run.ctx.close()


def test_infinity8b_full_cache_reference_layer():
    """The 8B-shaped full-cache reference run: 40 layers x 28 heads, batch 16,
    every segment kept (58.9 GB of cache), driven with attend_append as the
    benchmark drives it.  The last layer (the highest cache offsets) runs
    end to end: every head of one batch entry per die on sampled rows, every
    row of two (batch entry, head) pairs at the final scale, and the layer's
    cache bit for bit."""
    wl = workloads.get("c4")
    keep = workloads.full_keep(wl)
    layer = wl.layers - 1
    run = generate(wl, keep, [layer], fused=True)
    pairs = [(b, h) for b in PER_DIE_16 for h in range(wl.heads)]
    worst = _compare_outputs(run, [layer], rows_per_unit=24, bh=pairs)
    t = wl.n_scales - 1
    rows = np.arange(wl.scale_tokens[t])
    for b, h in ((0, 0), (15, 27)):
        want, _ = oracle_rows(run, layer, t, b, h, rows)
        got = gpu_rows(run, layer, t, b, h, rows)
        e = np.abs(got - want)
        assert e.max() <= BF16_MAX and e.mean() <= BF16_MEAN, (b, h, float(e.max()), float(e.mean()))
        worst = max(worst, float(e.max()))
    note(f"c4 full-cache worst max-abs {worst:.3e}")
    check_cache(run, [layer])
    run.ctx.close()


def test_determinism_and_scas_repeat():
    wl = workloads.get("c1")
    keep = _schedule(wl)
    ctx = hk.Context(1, 16, 128, 1, wl.scale_tokens, keep, torch.bfloat16)
    table = torch.zeros((1, 16, 13, 13), dtype=torch.float32, device="cuda")
    outs = []
    for rep in range(2):
        ctx.reset()
        got = []
        for t in range(13):
            inp = workloads.step_inputs(wl, 0, t)
            q, k, v = to_device(inp.q, wl), to_device(inp.k, wl), to_device(inp.v, wl)
            out = torch.empty_like(q)
            out2 = torch.empty_like(q)
            note(f"determinism rep {rep} step {t}")
            ctx.attend_with_scas(0, t, q, k, v, out, 1.0, table)
            ctx.attend(0, t, q, k, v, out2, 1.0)
            got.append(out.view(torch.int16).cpu().numpy())
            got.append(out2.view(torch.int16).cpu().numpy())
            if t < 12:
                ctx.append_scale(0, 1, t, k, v)
        got.append(table.cpu().numpy().view(np.int32))
        outs.append(got)
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
    ctx.close()


def test_split_merge_is_deterministic():
    """A split launch's partials are merged in split order, whatever order its
    workgroups finish in: the largest split launch of the full-cache layer,
    repeated, gives identical output bits."""
    wl = workloads.get("c1")
    keep = _schedule(wl)
    ctx = hk.Context(1, 16, 128, 1, wl.scale_tokens, keep, torch.bfloat16)
    split_steps = [t for t in range(wl.n_scales) if ctx.attend_plan(t)[1] > 1]
    assert split_steps, "no split launch in this workload"
    last = split_steps[-1]
    for t in range(last):
        inp = workloads.step_inputs(wl, 0, t)
        k, v = to_device(inp.k, wl), to_device(inp.v, wl)
        ctx.append_scale(0, 1, t, k, v)
    inp = workloads.step_inputs(wl, 0, last)
    q, k, v = to_device(inp.q, wl), to_device(inp.k, wl), to_device(inp.v, wl)
    ref = None
    for rep in range(12):
        out = torch.full_like(q, float("nan"))
        note(f"split merge rep {rep} step {last} splits {ctx.attend_plan(last)[1]}")
        ctx.attend(0, last, q, k, v, out, 1.0)
        got = out.view(torch.int16).cpu().numpy()
        if ref is None:
            ref = got
            assert torch.isfinite(out).all()
        else:
            assert np.array_equal(ref, got), rep
    ctx.close()


def test_order_and_argument_errors():
    wl = _custom(50, "errors", (1, 2, 3), heads=2, head_dim=128, batch=1, dtype="bf16")
    keep = np.ones((1, 2, 3), dtype=np.uint8)
    ctx = hk.Context(1, 2, 128, 1, wl.scale_tokens, keep, torch.bfloat16)
    mk = lambda t: torch.zeros((1, wl.scale_tokens[t], 2, 128), dtype=torch.bfloat16, device="cuda")  # noqa
    with pytest.raises(hk.HeatKVError) as e:
        ctx.attend(0, 1, mk(1), mk(1), mk(1), mk(1), 1.0)
    assert e.value.status == hk.HK_EORDER
    with pytest.raises(hk.HeatKVError) as e:
        ctx.append_scale(0, 1, 1, mk(1), mk(1))
    assert e.value.status == hk.HK_EORDER
    with pytest.raises(hk.HeatKVError) as e:
        ctx.append_scale(0, 1, 2, mk(2), mk(2))
    assert e.value.status == hk.HK_EINVAL
    with pytest.raises(hk.HeatKVError) as e:
        ctx.attend(0, 0, mk(1), mk(0), mk(0), mk(0), 1.0)   # wrong shape
    assert e.value.status == hk.HK_EINVAL
    with pytest.raises(hk.HeatKVError) as e:
        ctx.attend(0, 0, mk(0), mk(0), mk(0), mk(0), -1.0)
    assert e.value.status == hk.HK_EINVAL
    # raw ABI: misaligned pointer is rejected before any launch
    base = mk(2)
    p = base.data_ptr() + 2
    import ctypes
    rc = hk._lib.hk_attend(ctx._h, 0, 0, ctypes.c_void_p(p), ctypes.c_void_p(p),
                           ctypes.c_void_p(p), ctypes.c_void_p(p), 1.0, None)
    assert rc == hk.HK_EINVAL
    ctx.attend(0, 0, mk(0), mk(0), mk(0), mk(0), 1.0)
    ctx.append_scale(0, 1, 0, mk(0), mk(0))
    assert ctx.retained_tokens(0) == 2 and ctx.retained_tokens(2) == 2 * (1 + 4)
    torch.cuda.synchronize()
    ctx.close()


def test_split_launch_with_empty_splits():
    """A 256-query launch whose keys are split over several workgroups, where
    one head holds so few keys that some of its splits are empty (their
    partials carry zero weight in the merge); every head against the oracle,
    plain and fused."""
    wl = _custom(91, "split-empty", (1, 2, 3, 4, 6, 8, 12, 16, 24), heads=3, head_dim=128, batch=1,
                 dtype="bf16")
    keep = np.ones((1, wl.heads, wl.n_scales), dtype=np.uint8)
    keep[:, :, -1] = 0
    keep[0, 2, 1:] = 0          # head 2 keeps the sink only
    keep[0, 1, 3:6] = 0         # head 1 drops a middle run
    for fused in (False, True):
        run = generate(wl, keep, [0], fused=fused)
        last = wl.n_scales - 1
        rows, splits = run.ctx.attend_plan(last)
        assert rows == 256 and splits > 1, (rows, splits)
        keys_short = 1 + wl.scale_tokens[last]
        tiles = -(-keys_short // 64)
        per = -(-tiles // splits)
        assert (splits - 1) * per >= tiles, "no empty split for the short head"
        _compare_outputs(run, [0], rows_per_unit=256)
        check_cache(run, [0])
        run.ctx.close()


def test_heads_heaviest_first_with_split_launch():
    """Batch 8 with heads that hold different numbers of keys: each die runs
    its batch entries' heads heaviest first (the per-step head order), also
    in split launches and with empty splits; every (batch entry, head)
    against the oracle, plain and fused."""
    wl = _custom(92, "ordered-split", (1, 2, 3, 4, 6, 8, 12, 16, 24), heads=3, head_dim=128, batch=8,
                 dtype="bf16")
    keep = np.ones((1, wl.heads, wl.n_scales), dtype=np.uint8)
    keep[:, :, -1] = 0
    keep[0, 0, 1:] = 0          # head 0 keeps the sink only: the lightest, ranked last
    keep[0, 1, 3:6] = 0         # head 1 drops a middle run
    for fused in (False, True):
        run = generate(wl, keep, [0], fused=fused)
        rows, splits = run.ctx.attend_plan(wl.n_scales - 1)
        assert rows == 256 and splits > 1, (rows, splits)
        pairs = [(b, h) for b in range(wl.batch) for h in range(wl.heads)]
        _compare_outputs(run, [0], rows_per_unit=64, bh=pairs)
        check_cache(run, [0])
        run.ctx.close()


@pytest.mark.parametrize("mode", ["plain", "fused", "scas"])
def test_rescale_on_peaked_scores(mode):
    """A softmax scale of 6 makes most queries' running max rise by more than
    2^8 after their first key block, so the lazy max rescales the output
    accumulators, the denominator (and the S-CAS sums) in the middle of a
    head's keys; both tilings and split launches take part.  The softmax is
    then so peaked that an output is close to a single V row (|out| up to
    ~4), so the max-abs bound also allows the bf16 output's own rounding."""
    wl = _custom(92, "peaked", (1, 2, 4, 8, 12, 16, 24, 32), heads=16, head_dim=128, batch=2,
                 dtype="bf16", alpha=6.0)
    keep = _random_keep(wl, 92, p=0.8)
    scas = mode == "scas"
    run = generate(wl, keep, [0], scas=scas, fused=mode == "fused")
    rows = {run.ctx.attend_plan(t, scas)[0] for t in range(wl.n_scales)}
    assert rows == {128, 256}, rows
    _compare_outputs(run, [0], rows_per_unit=128, bh=[(b, h) for b in range(2) for h in (0, 3, 9, 15)],
                     own_rounding=True)
    if scas:
        _compare_scas(run, 0, heads=(0, 3, 9, 15))
    check_cache(run, [0])
    run.ctx.close()
