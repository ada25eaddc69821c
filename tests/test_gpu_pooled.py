"""GPU parity of the pooled cache: every head's rows in one pool per batch
entry, rows of dropped segments reused by later segments, nothing ever moved.
Attention reads the held rows through the per-(step, layer, head) map.
Against the fp64 oracle: attention outputs (bf16 max-abs <= 1e-2, mean-abs
<= 1e-3), S-CAS rows (<= 1e-4), and the pool contents of every held segment
of every driven (layer, head, batch entry), bit for bit, read through the
library's row assignment (hk_layout_pooled)."""
import numpy as np
import pytest
import torch

import workloads
from oracle import policies as opol
from oracle import progressive as opr

import kv_cache_compression_attend_amd as hk
from _gpu import SENTINEL_BF16, note, to_device, to_host_bits
from test_gpu_progressive import _check_outputs, _check_scas, _mid_drops, _schedule, _wl

pytestmark = pytest.mark.gpu


def _check_pool(ctx, wl, exp, seg, inputs, layers, t):
    """The pool rows of every segment (l, h) holds at the end of step t hold
    that segment's input rows, for every driven layer and batch entry."""
    K = wl.n_scales
    off = np.concatenate([[0], np.cumsum(wl.scale_tokens[: K - 1])])
    kb = to_host_bits(ctx.k_cache).reshape(wl.batch, ctx.pool_rows, wl.head_dim)
    vb = to_host_bits(ctx.v_cache).reshape(wl.batch, ctx.pool_rows, wl.head_dim)
    kk = min(t, K - 2)
    for l in layers:
        for h in range(wl.heads):
            for s in range(kk + 1):
                if int(exp[l, h, s]) <= kk:
                    continue
                rows = seg[l, h, off[s]: off[s + 1]]
                assert (rows >= 0).all()
                for which, bits in (("k", kb), ("v", vb)):
                    src = getattr(inputs[l][s], which)
                    for b in range(wl.batch):
                        assert np.array_equal(bits[b, rows], src[b, :, h, :]), (which, l, h, s, b, t)


def _drive_pooled(wl, exp, mode, layers=None, scas=False, check_every_step=True, seed=0,
                  check_layers=None):
    """Every scale of every layer through a pooled context: 'split' = attend
    then append per layer, 'fused' = attend_append per layer, 'multi' = attend
    every layer then one append over all of them.  Layers outside `layers`
    get seeded torch.randn inputs (they share the pool, so a wrong row
    assignment shows in the checked layers)."""
    layers = list(range(wl.layers)) if layers is None else layers
    check_layers = layers if check_layers is None else check_layers
    ctx = hk.Context(wl.layers, wl.heads, wl.head_dim, wl.batch, wl.scale_tokens, None,
                     torch.bfloat16, expire=exp, pooled=True)
    _, rows, seg = hk.layout_pooled(wl.scale_tokens, exp, wl.batch, wl.head_dim, with_rows=True)
    assert rows == ctx.pool_rows
    for c in (ctx.k_cache, ctx.v_cache):
        c.view(torch.int16).fill_(SENTINEL_BF16)
    table = torch.zeros((wl.layers, wl.heads, wl.n_scales, wl.n_scales), dtype=torch.float32,
                        device="cuda") if scas else None
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 7)
    inputs = {l: [] for l in layers}
    outs = {}
    K = wl.n_scales
    for t in range(K):
        ks, vs = [], []
        for l in range(wl.layers):
            if l in layers:
                x = workloads.step_inputs(wl, l, t, seed)
                inputs[l].append(x)
                q, k, v = to_device(x.q, wl), to_device(x.k, wl), to_device(x.v, wl)
            else:
                shape = (wl.batch, wl.scale_tokens[t], wl.heads, wl.head_dim)
                q, k, v = (torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16)
                           for _ in range(3))
            out = torch.empty_like(q)
            if l in check_layers:
                note(f"{wl.name} pooled {mode} layer {l} step {t}")
            if mode == "fused":
                ctx.attend_append(l, t, q, k, v, out, wl.softmax_scale, table)
            else:
                if scas:
                    ctx.attend_with_scas(l, t, q, k, v, out, wl.softmax_scale, table)
                else:
                    ctx.attend(l, t, q, k, v, out, wl.softmax_scale)
                if mode == "split" and t < K - 1:
                    ctx.append_scale(l, l + 1, t, k, v)
            if l in layers:
                outs[(l, t)] = out
            ks.append(k)
            vs.append(v)
        if mode == "multi" and t < K - 1:
            ctx.append_scale(0, wl.layers, t, torch.stack(ks), torch.stack(vs))
        torch.cuda.synchronize()
        if check_every_step or t >= K - 2:
            _check_pool(ctx, wl, exp, seg, inputs, check_layers, t)
    outs = {key: to_host_bits(o) for key, o in outs.items()}
    return ctx, inputs, outs, (table.cpu().numpy() if scas else None)


@pytest.mark.parametrize("mode", ["split", "fused", "multi"])
def test_pooled_progressive_bf16(mode):
    wl = _wl(91, (1, 2, 3, 4, 6, 8, 12, 16), layers=2, heads=4, head_dim=128, batch=2, dtype="bf16")
    exp = _schedule(wl, 0.3, 2, seed=4)
    assert _mid_drops(exp) > 0
    ctx, inputs, outs, table = _drive_pooled(wl, exp, mode, scas=(mode == "fused"))
    per_head, _, _ = hk.layout_expiry(wl.scale_tokens, exp, wl.batch, wl.head_dim)
    assert ctx.cache_elems < per_head
    _check_outputs(wl, exp, inputs, outs, [0, 1])
    if table is not None:
        _check_scas(wl, exp, inputs, table, [0, 1])
    ctx.close()


def test_pooled_handmade_expiry_reuses_rows():
    """Segments that leave the middle of a head's cache give their rows to
    later segments of other heads; the tiles of a head then read rows from
    anywhere in the pool (junctions with the current scale included)."""
    wl = _wl(90, (1, 2, 3, 4, 6, 8, 12, 16, 20), layers=1, heads=4, head_dim=128, batch=2,
             dtype="bf16")
    K = wl.n_scales
    exp = np.full((1, 4, K), K - 1, dtype=np.uint8)
    exp[0, :, :] = np.maximum(exp[0, :, :], np.arange(K))
    exp[0, 0, 1] = 7
    exp[0, 1, 2] = 6
    exp[0, 1, 3] = 7
    exp[0, 2, 1] = 3
    exp[0, 2, 4] = 5
    exp[0, 2, 5] = 5
    exp[0, 3, 0] = 7
    _, rows, seg = hk.layout_pooled(wl.scale_tokens, exp, wl.batch, wl.head_dim, with_rows=True)
    off = np.concatenate([[0], np.cumsum(wl.scale_tokens[: K - 1])])
    # some segment stored after step 7 sits below a row of a segment stored earlier
    late = seg[0, :, off[7]: off[8]]
    assert late.min() < seg[0, :, off[6]: off[7]].max()
    ctx, inputs, outs, _ = _drive_pooled(wl, exp, "split")
    _check_outputs(wl, exp, inputs, outs, [0])
    ctx.close()


@pytest.mark.parametrize("mode", ["fused", "multi"])
def test_pooled_scale_window_policy(mode):
    wl = _wl(95, (1, 2, 3, 4, 6, 8, 12, 16, 20), layers=3, heads=2, head_dim=128, batch=2,
             dtype="bf16")
    sim = [0.5, 0.2, 0.9]
    exp = hk.build_scale_window_schedule(3, 2, wl.scale_tokens, 2, 2, 4, sim, 1)
    np.testing.assert_array_equal(exp, opol.scale_window_schedule(3, 2, wl.scale_tokens, 2, 2, 4,
                                                                  sim, 1))
    ctx, inputs, outs, table = _drive_pooled(wl, exp, mode, scas=(mode == "fused"))
    _check_outputs(wl, exp, inputs, outs, [0, 1, 2])
    if table is not None:
        _check_scas(wl, exp, inputs, table, [0, 1, 2])
    ctx.close()


def test_pooled_progressive_infinity2b_budget10():
    """The 32-layer, batch-8, 10%-budget shape with its progressive schedule:
    a pool of 328,656 rows per batch entry (the live peak, within the budget
    of 328,960) serves all 32 layers; layers 0 and 31 run on the workload's
    inputs and are checked, the other 30 share the pool with random inputs."""
    wl = workloads.get("c2")
    table = workloads.dirichlet_scas(wl)
    exp, n, live = hk.build_progressive_schedule(table, wl.scale_tokens, wl.budget, wl.n_sink, True)
    want = opr.progressive_schedule(table, wl.scale_tokens, wl.budget, wl.n_sink, True)
    np.testing.assert_array_equal(exp, want[0])
    layers = [0, wl.layers - 1]
    ctx, inputs, outs, _ = _drive_pooled(wl, exp, "fused", layers=layers, check_every_step=False)
    assert ctx.pool_rows == int(live.max())
    _check_outputs(wl, exp, inputs, outs, layers, rows_per_unit=12, batches=(0, 3, wl.batch - 1))
    ctx.close()


def test_pooled_order_errors():
    wl = _wl(93, (1, 2, 3, 4, 6), layers=2, heads=2, head_dim=128, batch=1, dtype="bf16")
    K = wl.n_scales
    exp = np.full((2, 2, K), K - 1, dtype=np.uint8)
    exp[:, :, :] = np.maximum(exp, np.arange(K))
    exp[0, 0, 1] = 2
    ctx = hk.Context(2, 2, 128, 1, wl.scale_tokens, None, torch.bfloat16, expire=exp, pooled=True)
    mk = lambda t: torch.zeros((1, wl.scale_tokens[t], 2, 128), dtype=torch.bfloat16, device="cuda")  # noqa
    for l in (0, 1):
        ctx.attend_append(l, 0, mk(0), mk(0), mk(0), mk(0), 1.0)
    ctx.attend(0, 1, mk(1), mk(1), mk(1), mk(1), 1.0)
    with pytest.raises(hk.HeatKVError) as e:      # layer 0 has not appended step 1
        ctx.append_scale(1, 2, 1, mk(1), mk(1))
    assert e.value.status == hk.HK_EORDER
    ctx.append_scale(0, 1, 1, mk(1), mk(1))
    with pytest.raises(hk.HeatKVError) as e:      # step 1 of layer 0 is appended
        ctx.attend(0, 1, mk(1), mk(1), mk(1), mk(1), 1.0)
    assert e.value.status == hk.HK_EORDER
    with pytest.raises(hk.HeatKVError) as e:      # layer 1 has not appended step 1
        ctx.attend_append(0, 2, mk(2), mk(2), mk(2), mk(2), 1.0)
    assert e.value.status == hk.HK_EORDER
    ctx.attend_append(1, 1, mk(1), mk(1), mk(1), mk(1), 1.0)
    ctx.attend_append(0, 2, mk(2), mk(2), mk(2), mk(2), 1.0)
    torch.cuda.synchronize()
    ctx.close()
