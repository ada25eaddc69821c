"""Pins for the oracle's keep-mask schedule and cache accounting (CPU only)."""
import json
import math
import os

import numpy as np
import pytest

import workloads
from oracle import cache as ocache
from oracle import schedule as osch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_worked_schedules():
    g = json.load(open(os.path.join(GOLDEN, "schedule_hand.json")))
    for case in g["cases"]:
        table = np.array(case["scas"], dtype=np.float32)
        for bud in case["budgets"]:
            if "error" in bud:
                with pytest.raises(osch.ScheduleError) as e:
                    osch.build_schedule(table, case["tokens"], bud["beta"], case["n_sink"])
                assert e.value.code == bud["error"]
                continue
            keep, ret, n = osch.build_schedule(table, case["tokens"], bud["beta"], case["n_sink"])
            assert n == bud["N"], case["name"]
            np.testing.assert_array_equal(keep, np.array(bud["keep"], dtype=np.uint8))
            np.testing.assert_array_equal(ret, bud["retained"])


def _scalar_importance(table, l, h, s):
    acc = 0.0
    for t in range(s + 1, table.shape[2]):
        acc += float(table[l, h, t, s])
    return acc


def _feasible_with_prefix(table, tokens, beta, n_sink, N):
    """Brute force: build the mask for prefix N directly and test the budget."""
    L, H, K, _ = table.shape
    keep = np.ones((L, H, K), dtype=np.uint8)
    keep[:, :, K - 1] = 0
    for s in range(n_sink, K - 1):
        ranked = sorted(((_scalar_importance(table, l, h, s), l * H + h)
                         for l in range(L) for h in range(H)))
        for _, f in ranked[:N]:
            keep[f // H, f % H, s] = 0
    F = L * H * sum(tokens[:K - 1])
    bud = math.floor(beta * F)
    for k in range(K):
        r = sum(int(keep[l, h, s]) * tokens[s] for l in range(L) for h in range(H)
                for s in range(min(k, K - 2) + 1))
        if r > bud:
            return False, keep
    return True, keep


@pytest.mark.parametrize("seed", range(40))
def test_minimal_prefix_by_brute_force(seed):
    g = np.random.default_rng(seed)
    L, H = int(g.integers(1, 3)), int(g.integers(1, 4))
    K = int(g.integers(2, 6))
    tokens = workloads.random_tokens(K, seed)
    n_sink = int(g.integers(0, K))
    table = workloads.random_scas_table(L, H, K, seed)
    beta = float(g.uniform(0.05, 1.0))
    feas = [_feasible_with_prefix(table, tokens, beta, n_sink, N) for N in range(L * H + 1)]
    ok = [N for N in range(L * H + 1) if feas[N][0]]
    if not ok:
        with pytest.raises(osch.ScheduleError) as e:
            osch.build_schedule(table, tokens, beta, n_sink)
        assert e.value.code == "ebudget"
        return
    keep, ret, n = osch.build_schedule(table, tokens, beta, n_sink)
    assert n == min(ok)
    np.testing.assert_array_equal(keep, feas[n][1])


@pytest.mark.parametrize("seed", range(20))
def test_invariants(seed):
    g = np.random.default_rng(1000 + seed)
    L, H, K = int(g.integers(1, 5)), int(g.integers(1, 6)), int(g.integers(3, 9))
    tokens = workloads.random_tokens(K, seed, max_side=6)
    n_sink = int(g.integers(0, 3))
    table = workloads.random_scas_table(L, H, K, 500 + seed)
    F = osch.full_cache_slots(L, H, tokens)
    prev = None
    for beta in sorted(g.uniform(0.01, 1.0, size=6)) + [1.0]:
        try:
            keep, ret, n = osch.build_schedule(table, tokens, beta, n_sink)
        except osch.ScheduleError as e:
            assert e.code == "ebudget"
            assert math.floor(beta * F) < L * H * sum(tokens[:n_sink])
            continue
        assert keep[:, :, :n_sink].all(), "sink scales must be kept"
        assert not keep[:, :, K - 1].any(), "final scale is never cached"
        assert (ret <= math.floor(beta * F)).all(), "budget holds after every scale"
        # every pruned pair ranks below every kept pair of the same scale
        for s in range(n_sink, K - 1):
            imp = [(_scalar_importance(table, l, h, s), l * H + h)
                   for l in range(L) for h in range(H)]
            pruned = [x for x in imp if not keep[x[1] // H, x[1] % H, s]]
            kept = [x for x in imp if keep[x[1] // H, x[1] % H, s]]
            if pruned and kept:
                assert max(pruned) < min(kept)
            assert len(pruned) == n
        if prev is not None:
            assert (keep >= prev).all(), "keep sets are nested as the budget grows"
        prev = keep
        if beta == 1.0:
            assert n == 0


def test_error_codes():
    t = workloads.random_scas_table(1, 2, 4, 3)
    tok = (1, 4, 9, 16)
    for args in [(t, tok, 0.0, 1), (t, tok, 1.5, 1), (t, tok, 0.5, 4), (t, tok, 0.5, -1),
                 (t, tok[:3], 0.5, 1), (t[:, :, :3, :3], tok, 0.5, 1), (t, (1, 0, 9, 16), 0.5, 1)]:
        with pytest.raises(osch.ScheduleError) as e:
            osch.build_schedule(*args)
        assert e.value.code == "einval"


def test_workload_schedules():
    """Counts at the two pruned workloads follow the closed form keep_count =
    floor((floor(beta F) - sink cost) / prunable cost)."""
    for key, n_want, r_want in (("c2", 462, 323_560), ("c4", 1_077, 281_660)):
        wl = workloads.get(key)
        keep, ret, n = osch.build_schedule(workloads.dirichlet_scas(wl), wl.scale_tokens,
                                           wl.budget, wl.n_sink)
        assert n == n_want
        assert ret[-1] == r_want
        F = osch.full_cache_slots(wl.layers, wl.heads, wl.scale_tokens)
        assert (ret <= math.floor(wl.budget * F)).all()
        assert keep[:, :, :2].all()
    for key in ("c1", "c3"):
        wl = workloads.get(key)
        keep, ret, n = osch.build_schedule(workloads.dirichlet_scas(wl), wl.scale_tokens, 1.0, 2)
        assert n == 0 and keep[:, :, :-1].all()


def test_full_cache_accounting_pin():
    """The pages' full-cache size for Infinity-2B factors exactly with the final scale excluded."""
    g = json.load(open(os.path.join(GOLDEN, "infinity2b_full_cache.json")))
    tokens = [s * s for s in g["sides"]]
    got = ocache.full_cache_bytes(g["sequences"], g["layers"], g["hidden"], tokens, g["elem_bytes"])
    assert got == g["expected_bytes"]
    assert got == g["printed_MB"] * 2 ** 20
    # counting the final scale as well gives no whole number of sequences
    per_seq_all = 2 * g["layers"] * g["hidden"] * sum(tokens) * g["elem_bytes"]
    assert (g["printed_MB"] * 2 ** 20) % per_seq_all != 0


def test_cache_layout_and_expected_rows():
    wl = workloads.get("c0")
    keep = workloads.random_drop2_keep(wl)
    tok = wl.scale_tokens
    cap = ocache.capacity(keep, tok)
    for h in range(wl.heads):
        assert cap[0, h] == sum(tok[s] for s in range(wl.n_scales - 1) if keep[0, h, s])
    np.testing.assert_array_equal(ocache.len_before(keep, tok, wl.n_scales - 1), cap)
    base = ocache.bases(cap, wl.batch, wl.head_dim)
    assert base[0, 0] == 0 and base[0, 1] == cap[0, 0] * wl.batch * wl.head_dim
    ks = [workloads.step_inputs(wl, 0, t).k for t in range(wl.n_scales)]
    for h in range(wl.heads):
        rows = ocache.expected_rows(ks, keep[0, h], wl.n_scales - 1, 0, h)
        assert rows.shape[0] == cap[0, h]
        at = 0
        for s in range(wl.n_scales - 1):
            if keep[0, h, s]:
                np.testing.assert_array_equal(rows[at:at + tok[s]], ks[s][0, :, h, :])
                at += tok[s]
