"""Pins of the progressive-schedule oracle (``oracle.progressive``).

Nothing here compares the oracle with itself: the pins are closed forms of
the end-of-scale budget, an event-by-event simulation of the cache, an
exhaustive search over prefix-length sequences on tiny tables, and the
static schedule as the special case the pages describe."""
import itertools
import math

import numpy as np

import workloads
from oracle import progressive as opr
from oracle import schedule as osch


def _simulate(expire, tokens):
    """Replay the cache layer by layer: at scale k every layer drops its
    segments that expire at k and then stores segment k if it outlives k.
    Returns the total rows after each (k, layer) and the per-(l, h) segment
    lists at the end of every scale."""
    L, H, K = expire.shape
    held = {(l, h): [] for l in range(L) for h in range(H)}
    sizes = np.zeros((K, L), dtype=np.int64)
    lists = []
    for k in range(K):
        for l in range(L):
            if k <= K - 2:
                for h in range(H):
                    held[(l, h)] = [s for s in held[(l, h)] if expire[l, h, s] != k]
                    if expire[l, h, k] > k:
                        held[(l, h)].append(k)
            sizes[k, l] = sum(tokens[s] for lst in held.values() for s in lst)
        lists.append({key: list(v) for key, v in held.items()})
    return sizes, lists


def _ranks(scas):
    """rank[l, h, s]: position of head (l, h) in the ordering of scale s,
    computed with numpy's lexsort (not the oracle's sort)."""
    L, H, K, _ = scas.shape
    imp = np.zeros((L, H, K))
    for s in range(K):
        for t in range(s + 1, K):
            imp[:, :, s] += scas[:, :, t, s].astype(np.float64)
    rank = np.zeros((L, H, K), dtype=np.int64)
    flat_idx = np.arange(L * H)
    for s in range(K):
        order = np.lexsort((flat_idx, imp[:, :, s].reshape(-1)))
        rank.reshape(L * H, K)[order, s] = np.arange(L * H)
    return rank


def _tiny_cases(n):
    g = np.random.default_rng(5)
    for i in range(n):
        L, H, K = int(g.integers(1, 3)), int(g.integers(1, 4)), int(g.integers(2, 6))
        tokens = workloads.random_tokens(K, 100 + i, max_side=4)
        table = workloads.random_scas_table(L, H, K, 100 + i)
        if i % 5 == 0:
            table = np.round(table * 3) / 3  # exact ties
        beta = float(g.choice([g.uniform(0.05, 1.0), 0.3, 0.6, 1.0]))
        n_sink = int(g.integers(0, K))
        yield table.astype(np.float32), tokens, beta, n_sink


def test_full_budget_prunes_nothing():
    wl = workloads.get("c2")
    table = workloads.dirichlet_scas(wl)
    exp, n, live = opr.progressive_schedule(table, wl.scale_tokens, 1.0, 2)
    assert (n == 0).all()
    K = wl.n_scales
    assert (exp[:, :, : K - 1] == K - 1).all() and (exp[:, :, K - 1] == K - 1).all()
    F = osch.full_cache_slots(wl.layers, wl.heads, wl.scale_tokens)
    assert live[K - 2, -1] == F


def test_end_of_scale_prefix_closed_form():
    """With end-of-scale accounting, the size after scale k with prefix N is
    S_sink(k) + (L*H - N) * T_P(k), so N_k has a closed form."""
    for table, tokens, beta, n_sink in _tiny_cases(300):
        L, H, K, _ = table.shape
        heads = L * H
        bud = math.floor(beta * heads * sum(tokens[: K - 1]))
        try:
            exp, n, live = opr.progressive_schedule(table, tokens, beta, n_sink, per_layer=False)
        except osch.ScheduleError as e:
            assert e.code == "ebudget"
            assert bud < heads * sum(tokens[:n_sink])
            continue
        prev = 0
        for k in range(K - 1):
            s_sink = heads * sum(tokens[s] for s in range(min(n_sink, k + 1)))
            t_p = sum(tokens[s] for s in range(n_sink, min(k, K - 2) + 1))
            want = prev if t_p == 0 else max(prev, heads - min(heads, (bud - s_sink) // t_p))
            assert n[k] == want, (k, n, want)
            prev = want


def test_accounting_matches_event_simulation():
    """live[k][l] (Algorithm 2's size after layer l of scale k) equals a
    layer-by-layer replay of drops and appends; the cache of every head at the
    end of a scale is the segments the expiry steps say, in scale order."""
    for table, tokens, beta, n_sink in _tiny_cases(200):
        L, H, K, _ = table.shape
        for per_layer in (True, False):
            try:
                exp, n, live = opr.progressive_schedule(table, tokens, beta, n_sink, per_layer)
            except osch.ScheduleError:
                continue
            sizes, lists = _simulate(exp, tokens)
            np.testing.assert_array_equal(live, sizes)
            for k in range(K):
                for (l, h), segs in lists[k].items():
                    assert opr.rows_at_end(exp[l, h], tokens, k) == sum(tokens[s] for s in segs)
            np.testing.assert_array_equal(opr.retained_per_step(exp, tokens), sizes[:, -1])


def test_budget_holds_and_prefix_is_minimal_by_exhaustive_search():
    """The prefix lengths are the lexicographically smallest non-decreasing
    sequence whose simulated cache fits the budget after every layer (or
    every scale); found by trying every sequence on tiny tables."""
    checked = 0
    for table, tokens, beta, n_sink in _tiny_cases(120):
        L, H, K, _ = table.shape
        heads = L * H
        bud = math.floor(beta * heads * sum(tokens[: K - 1]))
        rank = _ranks(table)
        for per_layer in (True, False):
            try:
                exp, n, live = opr.progressive_schedule(table, tokens, beta, n_sink, per_layer)
            except osch.ScheduleError as err:
                assert err.code == "ebudget" and bud < heads * sum(tokens[:n_sink])
                continue
            best = None
            for seq in itertools.product(range(heads + 1), repeat=K - 1):
                if any(seq[i] > seq[i + 1] for i in range(K - 2)):
                    continue
                e = np.full((L, H, K), K - 1, dtype=np.int64)
                for k in range(K - 2, -1, -1):
                    for s in range(n_sink, min(k, K - 2) + 1):
                        e[:, :, s] = np.where(rank[:, :, s] < seq[k], k, e[:, :, s])
                sizes, _ = _simulate(e, tokens)
                worst = sizes[: K - 1].max() if per_layer else sizes[: K - 1, -1].max()
                if worst <= bud:
                    best = (seq, e)
                    break
            assert best is not None
            assert tuple(int(x) for x in n[: K - 1]) == best[0]
            np.testing.assert_array_equal(exp.astype(np.int64), best[1])
            assert live.max() <= bud if per_layer else live[:, -1].max() <= bud
            checked += 1
    assert checked > 100


def test_static_schedule_is_the_final_prefix():
    """End-of-scale accounting ends at the static schedule's N, and what the
    final scale reads is the static keep-mask; every earlier scale keeps at
    least as much as the static schedule (pruning is lazy)."""
    for key in ("c2", "c4"):
        wl = workloads.get(key)
        table = workloads.dirichlet_scas(wl)
        keep, r_static, n_static = osch.build_schedule(table, wl.scale_tokens, wl.budget, wl.n_sink)
        exp, n, live = opr.progressive_schedule(table, wl.scale_tokens, wl.budget, wl.n_sink,
                                                per_layer=False)
        K = wl.n_scales
        assert n[K - 2] == n_static
        assert (np.diff(n) >= 0).all()
        for l in range(wl.layers):
            for h in range(wl.heads):
                assert opr.visible(exp[l, h], K - 1)[: K - 1] == list(keep[l, h, : K - 1])
        r = opr.retained_per_step(exp, wl.scale_tokens)
        assert (r >= r_static).all() and r[K - 2] == r_static[K - 2]
        assert r.max() <= math.floor(wl.budget * osch.full_cache_slots(wl.layers, wl.heads, wl.scale_tokens))


def test_per_layer_accounting_is_never_looser():
    wl = workloads.get("c2")
    table = workloads.dirichlet_scas(wl)
    e1, n1, live1 = opr.progressive_schedule(table, wl.scale_tokens, wl.budget, wl.n_sink, True)
    e0, n0, live0 = opr.progressive_schedule(table, wl.scale_tokens, wl.budget, wl.n_sink, False)
    assert (n1 >= n0).all()
    bud = math.floor(wl.budget * osch.full_cache_slots(wl.layers, wl.heads, wl.scale_tokens))
    assert live1.max() <= bud
    assert live0.max() > bud  # end-of-scale accounting overshoots inside a scale


def test_expire_from_keep_round_trip():
    wl = workloads.get("c0")
    keep = workloads.random_drop2_keep(wl)
    exp = opr.expire_from_keep(keep)
    K = wl.n_scales
    for t in range(K):
        for h in range(wl.heads):
            vis = opr.visible(exp[0, h], t)
            assert vis == [int(keep[0, h, s]) if s < t else 0 for s in range(K)]
    np.testing.assert_array_equal(opr.capacity(exp, wl.scale_tokens),
                                  __import__("oracle").cache.capacity(keep, wl.scale_tokens))


def test_expected_rows_concatenates_survivors():
    g = np.random.default_rng(1)
    tokens = (1, 2, 3, 4, 5)
    ks = [g.integers(0, 1000, size=(2, n, 3, 4)) for n in tokens]
    exp = np.array([4, 2, 4, 3, 4])  # segment 1 leaves after scale 2, 3 is dropped at once
    for k, want in ((0, [0]), (1, [0, 1]), (2, [0, 2]), (3, [0, 2]), (4, [0, 2])):
        rows = opr.expected_rows(ks, exp, k, 1, 2)
        np.testing.assert_array_equal(rows, np.concatenate([ks[s][1, :, 2, :] for s in want]))
        assert opr.rows_at_end(exp, tokens, k) == sum(tokens[s] for s in want)
