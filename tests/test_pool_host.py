"""Pooled cache layout (host, CPU): every head's rows in one pool per batch
entry, rows of dropped segments reused by later ones.  The library's row
assignment is checked against the schedule's own per-layer accounting
(oracle.progressive): the pool holds exactly the most token slots live after
any layer of any scale, no two segments live at the same time share a row,
and every stored segment has its n_s rows."""
import numpy as np
import pytest

import workloads
from oracle import progressive as opr

import kv_cache_compression_attend_amd as hk


def _live_segments(expire, k, l):
    """(layer, head, scale) segments held once layer l has finished scale k:
    layers 0..l at the end of scale k, the later ones at the end of k-1."""
    L, H, K = expire.shape
    out = []
    for ll in range(L):
        kk = k if ll <= l else k - 1
        if kk < 0:
            continue
        kk = min(kk, K - 2)
        for h in range(H):
            for s in range(kk + 1):
                if int(expire[ll, h, s]) > kk:
                    out.append((ll, h, s))
    return out


def _check_plan(expire, tokens):
    L, H, K = expire.shape
    B, D = 2, 128
    elems, rows, seg = hk.layout_pooled(tokens, expire, B, D, with_rows=True)
    assert elems == B * rows * D
    off = np.concatenate([[0], np.cumsum(tokens[: K - 1])])
    # every stored segment has its rows, every unstored one -1
    for l in range(L):
        for h in range(H):
            for s in range(K - 1):
                r = seg[l, h, off[s]: off[s + 1]]
                if int(expire[l, h, s]) > s:
                    assert (r >= 0).all() and (r < rows).all() and len(set(r.tolist())) == len(r)
                else:
                    assert (r == -1).all()
    peak = 0
    for k in range(K):
        for l in range(L):
            live = _live_segments(expire, k, l)
            n = sum(int(tokens[s]) for (_, _, s) in live)
            peak = max(peak, n)
            used = np.concatenate([seg[ll, h, off[s]: off[s + 1]] for (ll, h, s) in live]) \
                if live else np.zeros(0, np.int32)
            assert len(np.unique(used)) == len(used), (k, l)
    assert rows == peak
    return rows


@pytest.mark.parametrize("seed", range(12))
def test_pool_rows_disjoint_and_exactly_the_live_peak(seed):
    g = np.random.default_rng(seed)
    L, H, K = int(g.integers(1, 4)), int(g.integers(1, 5)), int(g.integers(2, 9))
    tokens = np.array(workloads.random_tokens(K, 500 + seed), dtype=np.int32)
    if seed % 2:
        expire = np.zeros((L, H, K), dtype=np.uint8)
        for s in range(K):
            expire[:, :, s] = g.integers(s, K, size=(L, H))
    else:
        table = workloads.random_scas_table(L, H, K, 600 + seed)
        try:
            expire = hk.build_progressive_schedule(table, tokens, float(g.uniform(0.3, 0.9)),
                                                   int(g.integers(0, K)), True)[0]
        except hk.HeatKVError:
            pytest.skip("budget below the sink scales")
    _check_plan(expire, tokens)


def test_pool_of_the_progressive_10pct_workload_is_its_live_peak():
    """32 layers x 16 heads, 10% budget, progressive schedule with per-layer
    accounting: the pool is the schedule's live peak, within the budget, against
    2.55 GB for regions sized to each head's own peak."""
    wl = workloads.get("c2")
    table = workloads.dirichlet_scas(wl)
    exp, n, live = hk.build_progressive_schedule(table, wl.scale_tokens, wl.budget, wl.n_sink, True)
    want = opr.progressive_schedule(table, wl.scale_tokens, wl.budget, wl.n_sink, True)
    np.testing.assert_array_equal(live, want[2])
    elems, rows = hk.layout_pooled(wl.scale_tokens, exp, wl.batch, wl.head_dim)
    F = wl.layers * wl.heads * sum(wl.scale_tokens[:-1])
    assert rows == int(live.max()) == 328656
    assert rows <= int(np.floor(wl.budget * F))
    per_head, _, _ = hk.layout_expiry(wl.scale_tokens, exp, wl.batch, wl.head_dim)
    assert elems < 0.53 * per_head


def test_pool_of_a_static_schedule_is_the_retained_cache():
    """A static keep-mask never frees rows: the pool is the retained size."""
    wl = workloads.get("c2")
    keep = hk.build_schedule(workloads.dirichlet_scas(wl), wl.scale_tokens, wl.budget, wl.n_sink)[0]
    exp = opr.expire_from_keep(keep)
    _, rows = hk.layout_pooled(wl.scale_tokens, exp, 1, 128)
    assert rows == int(opr.retained_per_step(exp, wl.scale_tokens)[-1]) == 323560


def test_pool_rejects_bad_schedules():
    tok = (1, 4, 9)
    exp = np.array([[[0, 3, 2]]], dtype=np.uint8)   # entry above K-1
    with pytest.raises(hk.HeatKVError):
        hk.layout_pooled(tok, exp, 1, 128)
    exp = np.array([[[0, 0, 2]]], dtype=np.uint8)   # entry below its scale
    with pytest.raises(hk.HeatKVError):
        hk.layout_pooled(tok, exp, 1, 128)
