"""GPU parity of the progressive schedule: segments leave the middle of a
head's cache when the pruning set grows, and the library moves the survivors
down in place.  Compared with the fp64 oracle after every scale: attention
outputs (bf16 max-abs <= 1e-2, mean-abs <= 1e-3; fp32 <= 1e-5), S-CAS rows
(<= 1e-4) and the cache contents of every (layer, head, batch entry), bit for
bit."""
import numpy as np
import pytest
import torch

import workloads
from oracle import attention as oatt
from oracle import policies as opol
from oracle import progressive as opr
from oracle.numerics import to_f64

import kv_cache_compression_attend_amd as hk
from _gpu import SENTINEL_BF16, SENTINEL_F32, note, sample_rows, to_device, to_host_bits, torch_dtype

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN, F32_MAX, SCAS_TOL = 1e-2, 1e-3, 1e-5, 1e-4


def _wl(index, sides, layers, heads, head_dim, batch, dtype):
    return workloads.Workload(
        index=index, name=f"progressive-{index}", layers=layers, heads=heads, head_dim=head_dim,
        batch=batch, sides=tuple(sides), dtype=dtype, budget=1.0, n_sink=1,
        softmax_scale=1.0 if dtype == "bf16" else head_dim ** -0.5,
        qk_std=head_dim ** -0.25 if dtype == "bf16" else 1.0, schedule="custom")


def _schedule(wl, beta, n_sink, seed, per_layer=True):
    table = workloads.random_scas_table(wl.layers, wl.heads, wl.n_scales, seed)
    exp, n, live = hk.build_progressive_schedule(table, wl.scale_tokens, beta, n_sink, per_layer)
    want = opr.progressive_schedule(table, wl.scale_tokens, beta, n_sink, per_layer)
    np.testing.assert_array_equal(exp, want[0])
    np.testing.assert_array_equal(live, want[2])
    return exp


def _mid_drops(exp):
    K = exp.shape[2]
    s = np.arange(K)[None, None, :]
    return int(((exp > s) & (exp < K - 1)).sum())


def _poison(ctx):
    for c in (ctx.k_cache, ctx.v_cache):
        if c.dtype == torch.bfloat16:
            c.view(torch.int16).fill_(SENTINEL_BF16)
        else:
            c.view(torch.int32).fill_(SENTINEL_F32)


def _check_cache_after(ctx, wl, exp, inputs, layers, t):
    """Rows [0, rows at the end of step t) of every driven (l, h, b) equal the
    oracle's surviving segments, bit for bit."""
    lo = int(ctx.base[min(layers), 0])
    hi = int(ctx.base[max(layers), -1]) + wl.batch * int(ctx.cap[max(layers), -1]) * wl.head_dim
    kb, vb = to_host_bits(ctx.k_cache[lo:hi]), to_host_bits(ctx.v_cache[lo:hi])
    for l in layers:
        for h in range(wl.heads):
            cap, base = int(ctx.cap[l, h]), int(ctx.base[l, h]) - lo
            rows = opr.rows_at_end(exp[l, h], wl.scale_tokens, t)
            for which, bits in (("k", kb), ("v", vb)):
                region = bits[base: base + wl.batch * cap * wl.head_dim].reshape(wl.batch, cap, wl.head_dim)
                for b in range(wl.batch):
                    want = opr.expected_rows([getattr(x, which) for x in inputs[l]], exp[l, h], t, b, h)
                    assert want.shape[0] == rows
                    assert np.array_equal(region[b, :rows], want), (which, l, h, b, t)


def _check_outputs(wl, exp, inputs, outs, layers, rows_per_unit=64, batches=None):
    tmax, tmean = (BF16_MAX, BF16_MEAN) if wl.dtype == "bf16" else (F32_MAX, F32_MAX)
    batches = range(wl.batch) if batches is None else batches
    for l in layers:
        for t in range(wl.n_scales):
            rows = sample_rows(wl.scale_tokens[t], rows_per_unit, 7 * t + l)
            err_sum, err_cnt = 0.0, 0
            for b in batches:
                for h in range(wl.heads):
                    vis = opr.visible(exp[l, h], t)
                    kj, vj, _, _ = oatt.gather_keys([x.k for x in inputs[l][: t + 1]],
                                                    [x.v for x in inputs[l][: t + 1]], vis, t, b, h)
                    q = to_f64(inputs[l][t].q[b, rows, h, :], wl.dtype)
                    want, _ = oatt.softmax_attention(q, to_f64(kj, wl.dtype), to_f64(vj, wl.dtype),
                                                     wl.softmax_scale)
                    got = to_f64(outs[(l, t)][b, rows, h, :], wl.dtype)
                    e = np.abs(got - want)
                    assert np.isfinite(got).all() and e.max() <= tmax, (l, t, b, h, float(e.max()))
                    err_sum += float(e.sum())
                    err_cnt += e.size
            assert err_sum / err_cnt <= tmean, (l, t)


def _check_scas(wl, exp, inputs, table, layers):
    for l in layers:
        for t in range(wl.n_scales):
            for h in range(wl.heads):
                vis = opr.visible(exp[l, h], t)
                mass = np.zeros(t + 1)
                for b in range(wl.batch):
                    kj, vj, src, lens = oatt.gather_keys([x.k for x in inputs[l][: t + 1]],
                                                         [x.v for x in inputs[l][: t + 1]], vis, t, b, h)
                    q = to_f64(inputs[l][t].q[b, :, h, :], wl.dtype)
                    _, p = oatt.softmax_attention(q, to_f64(kj, wl.dtype), to_f64(vj, wl.dtype),
                                                  wl.softmax_scale)
                    mass += oatt.segment_mass(p, src, lens, t)
                got = table[l, h, t, : t + 1].astype(np.float64)
                np.testing.assert_allclose(got, mass / wl.batch, atol=SCAS_TOL, rtol=0,
                                           err_msg=f"l{l} h{h} t{t}")
                for s in range(t):
                    if not vis[s]:
                        assert table[l, h, t, s] == 0.0


def _drive(wl, exp, mode, layers=None, scas=False, check_every_step=True, seed=0):
    """Run every scale through the library: 'split' = attend then append per
    layer, 'fused' = attend_append per layer, 'multi' = attend every layer then
    one append over all of them."""
    layers = list(range(wl.layers)) if layers is None else layers
    ctx = hk.Context(wl.layers, wl.heads, wl.head_dim, wl.batch, wl.scale_tokens, None,
                     torch_dtype(wl), expire=exp)
    _poison(ctx)
    table = torch.zeros((wl.layers, wl.heads, wl.n_scales, wl.n_scales), dtype=torch.float32,
                        device="cuda") if scas else None
    inputs = {l: [] for l in layers}
    outs = {}
    K = wl.n_scales
    for t in range(K):
        ks, vs = [], []
        for l in layers:
            x = workloads.step_inputs(wl, l, t, seed)
            inputs[l].append(x)
            q, k, v = to_device(x.q, wl), to_device(x.k, wl), to_device(x.v, wl)
            out = torch.empty_like(q)
            note(f"{wl.name} {mode} layer {l} step {t}")
            if mode == "fused":
                ctx.attend_append(l, t, q, k, v, out, wl.softmax_scale, table)
            else:
                if scas:
                    ctx.attend_with_scas(l, t, q, k, v, out, wl.softmax_scale, table)
                else:
                    ctx.attend(l, t, q, k, v, out, wl.softmax_scale)
                if mode == "split" and t < K - 1:
                    ctx.append_scale(l, l + 1, t, k, v)
            outs[(l, t)] = out
            ks.append(k)
            vs.append(v)
        if mode == "multi" and t < K - 1:
            assert layers == list(range(layers[0], layers[0] + len(layers)))
            note(f"{wl.name} multi-layer append step {t}")
            ctx.append_scale(layers[0], layers[-1] + 1, t, torch.stack(ks), torch.stack(vs))
        torch.cuda.synchronize()
        if check_every_step or t >= K - 2:
            _check_cache_after(ctx, wl, exp, inputs, layers, t)
    outs = {key: to_host_bits(o) for key, o in outs.items()}
    return ctx, inputs, outs, (table.cpu().numpy() if scas else None)


@pytest.mark.parametrize("mode", ["split", "fused"])
def test_handmade_expiry_moves_overlapping_chunks(mode):
    """Small drops under long survivors: moves of 116 to 273 rows shifted by
    1 to 16 rows, so source and destination overlap inside and across the
    gather's 256-row chunks of each 128-byte column part.  At step 5 the
    only change is a dropped tail segment (head 2): nothing moves, but the
    new segment goes where the dropped one was."""
    wl = _wl(90, (1, 2, 3, 4, 6, 8, 12, 16, 20), layers=1, heads=4, head_dim=128, batch=2,
             dtype="bf16")
    K = wl.n_scales
    exp = np.full((1, 4, K), K - 1, dtype=np.uint8)
    exp[0, :, :] = np.maximum(exp[0, :, :], np.arange(K))
    exp[0, 0, 1] = 7          # step 7: scales 2..6 (269 rows) move down by 4
    exp[0, 1, 2] = 6          # step 6: scales 3..5 (116 rows) move down by 9
    exp[0, 1, 3] = 7          # step 7: scales 4..6 (244 rows) move down by 16
    exp[0, 2, 1] = 3          # step 3: scale 2 moves down by 4
    exp[0, 2, 4] = 5          # step 5: the tail segment leaves, nothing moves
    exp[0, 2, 5] = 5          # never stored
    exp[0, 3, 0] = 7          # step 7: scales 1..6 (273 rows) move down by 1
    assert (exp[0, :, 5] == 5).sum() == 1 and (exp[0, :, :5] == 5).sum() == 1
    ctx, inputs, outs, _ = _drive(wl, exp, mode)
    _check_outputs(wl, exp, inputs, outs, [0])
    ctx.close()


@pytest.mark.parametrize("mode", ["split", "fused", "multi"])
def test_progressive_bf16(mode):
    wl = _wl(91, (1, 2, 3, 4, 6, 8, 12, 16), layers=2, heads=4, head_dim=128, batch=2, dtype="bf16")
    exp = _schedule(wl, 0.3, 2, seed=4)
    assert _mid_drops(exp) > 0
    ctx, inputs, outs, table = _drive(wl, exp, mode, scas=(mode == "fused"))
    _check_outputs(wl, exp, inputs, outs, [0, 1])
    if table is not None:
        _check_scas(wl, exp, inputs, table, [0, 1])
    ctx.close()


@pytest.mark.parametrize("head_dim", [16, 32, 64, 128])
def test_progressive_f32(head_dim):
    """fp32 rows of 64 to 512 bytes: the gather moves them as one column part
    (head_dim 16 and 32), two (64) or four 128-byte parts (128)."""
    wl = _wl(92 + head_dim, (1, 2, 3, 4, 6, 8), layers=2, heads=3, head_dim=head_dim, batch=2,
             dtype="f32")
    exp = _schedule(wl, 0.35, 1, seed=9)
    assert _mid_drops(exp) > 0
    ctx, inputs, outs, table = _drive(wl, exp, "split", scas=True)
    _check_outputs(wl, exp, inputs, outs, [0, 1])
    _check_scas(wl, exp, inputs, table, [0, 1])
    ctx.close()


def test_progressive_order_errors():
    wl = _wl(93, (1, 2, 3, 4, 6), layers=1, heads=2, head_dim=128, batch=1, dtype="bf16")
    K = wl.n_scales
    exp = np.full((1, 2, K), K - 1, dtype=np.uint8)
    exp[0, 0, 1] = 3          # layer 0 moves at step 3
    ctx = hk.Context(1, 2, 128, 1, wl.scale_tokens, None, torch.bfloat16, expire=exp)
    xs = [workloads.step_inputs(wl, 0, t, 0) for t in range(K)]
    dev = [tuple(to_device(a, wl) for a in (x.q, x.k, x.v)) for x in xs]
    for t in range(3):
        q, k, v = dev[t]
        ctx.attend_append(0, t, q, k, v, torch.empty_like(q), 1.0)
    q, k, v = dev[3]
    with pytest.raises(hk.HeatKVError) as e:
        ctx.append_scale(0, 1, 3, k, v)       # would move rows attend(0, 3) still reads
    assert e.value.status == hk.HK_EORDER
    ctx.attend(0, 3, q, k, v, torch.empty_like(q), 1.0)
    ctx.append_scale(0, 1, 3, k, v)
    with pytest.raises(hk.HeatKVError) as e:
        ctx.attend(0, 3, q, k, v, torch.empty_like(q), 1.0)   # layout of step 3 is gone
    assert e.value.status == hk.HK_EORDER
    q2, k2, v2 = dev[2]
    with pytest.raises(hk.HeatKVError) as e:
        # step 2 itself drops nothing, but the append of step 3 moved its rows
        ctx.attend(0, 2, q2, k2, v2, torch.empty_like(q2), 1.0)
    assert e.value.status == hk.HK_EORDER
    torch.cuda.synchronize()
    ctx.close()


def test_progressive_infinity2b_budget10_two_layers():
    """The 32-layer, batch-8, 10%-budget shape with its progressive schedule
    (per-layer accounting), driving layers 0 and 1 with the fused call;
    every other layer's region keeps its sentinel."""
    wl = workloads.get("c2")
    table = workloads.dirichlet_scas(wl)
    exp, n, live = hk.build_progressive_schedule(table, wl.scale_tokens, wl.budget, wl.n_sink, True)
    want = opr.progressive_schedule(table, wl.scale_tokens, wl.budget, wl.n_sink, True)
    np.testing.assert_array_equal(exp, want[0])
    layers = [0, 1]
    assert _mid_drops(exp[layers]) > 0
    ctx, inputs, outs, _ = _drive(wl, exp, "fused", layers=layers, check_every_step=False)
    _check_outputs(wl, exp, inputs, outs, layers, rows_per_unit=12, batches=(0, wl.batch - 1))
    for l in (2, wl.layers - 1):
        lo = int(ctx.base[l, 0])
        hi = int(ctx.base[l, -1]) + wl.batch * int(ctx.cap[l, -1]) * wl.head_dim
        for c in (ctx.k_cache, ctx.v_cache):
            assert (to_host_bits(c[lo:hi]) == SENTINEL_BF16).all(), l
    ctx.close()


@pytest.mark.parametrize("mode", ["fused", "multi"])
def test_scale_window_policy_bf16(mode):
    """Condensed + local scale-window schedule: two condensed scales, a window
    of two local scales, four in the least similar layer.  The oldest local
    segment leaves from the middle of the cache at every step."""
    wl = _wl(95, (1, 2, 3, 4, 6, 8, 12, 16, 20), layers=3, heads=2, head_dim=128, batch=2,
             dtype="bf16")
    sim = [0.5, 0.2, 0.9]
    exp = hk.build_scale_window_schedule(3, 2, wl.scale_tokens, 2, 2, 4, sim, 1)
    np.testing.assert_array_equal(exp, opol.scale_window_schedule(3, 2, wl.scale_tokens, 2, 2, 4,
                                                                  sim, 1))
    ctx, inputs, outs, table = _drive(wl, exp, mode, scas=(mode == "fused"))
    _check_outputs(wl, exp, inputs, outs, [0, 1, 2])
    if table is not None:
        _check_scas(wl, exp, inputs, table, [0, 1, 2])
    ctx.close()


def test_scale_window_policy_infinity2b_shape():
    """The window schedule at the shape the benchmark runs it: 32 layers x 16
    heads, batch 8, two condensed scales, a window of two local scales, the
    four least similar layers keeping every scale.  A cache-demanding layer
    and a windowed one are driven end to end with the fused call and checked
    against the oracle (outputs on sampled rows of three batch entries, the
    cache of every head after the last two scales); every other layer's
    region keeps its sentinel."""
    wl = workloads.get("c2")
    K, L = wl.n_scales, wl.layers
    sim = np.random.default_rng(5).random(L).astype(np.float32)
    exp = hk.build_scale_window_schedule(L, wl.heads, wl.scale_tokens, 2, 2, K, sim, 4)
    np.testing.assert_array_equal(exp, opol.scale_window_schedule(L, wl.heads, wl.scale_tokens, 2, 2,
                                                                  K, sim, 4))
    demanding = int(np.argsort(sim)[0])
    windowed = int(np.argsort(sim)[-1])
    assert (exp[demanding] == K - 1).sum() > (exp[windowed] == K - 1).sum()
    layers = sorted({demanding, windowed})
    assert _mid_drops(exp[windowed:windowed + 1]) > 0
    ctx, inputs, outs, _ = _drive(wl, exp, "fused", layers=layers, check_every_step=False)
    _check_outputs(wl, exp, inputs, outs, layers, rows_per_unit=12, batches=(0, 4, wl.batch - 1))
    other = [l for l in range(L) if l not in layers][:2]
    for l in other:
        lo = int(ctx.base[l, 0])
        hi = int(ctx.base[l, -1]) + wl.batch * int(ctx.cap[l, -1]) * wl.head_dim
        for c in (ctx.k_cache, ctx.v_cache):
            assert (to_host_bits(c[lo:hi]) == SENTINEL_BF16).all(), l
    ctx.close()
