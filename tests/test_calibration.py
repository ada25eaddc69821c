"""Streaming calibration and ranking stability: oracle pins and the C ABI (CPU)."""
import math

import numpy as np
import pytest
from scipy import stats

import workloads
from oracle import calibration as ocal
from oracle import schedule as osch

import kv_cache_compression_attend_amd as hk


def test_streamed_mean_is_mean_over_images():
    g = np.random.default_rng(0)
    per_image = g.random((7, 2, 3, 4, 4))
    sizes = [2, 4, 1]
    tables, at = [], 0
    for b in sizes:
        tables.append(per_image[at:at + b].mean(axis=0))
        at += b
    np.testing.assert_allclose(ocal.streamed_mean(tables, sizes), per_image.mean(axis=0),
                               rtol=0, atol=1e-15)


@pytest.mark.parametrize("seed", range(5))
def test_spearman_matches_library(seed):
    g = np.random.default_rng(seed)
    n = int(g.integers(2, 40))
    pa, pb = g.permutation(n), g.permutation(n)
    assert abs(ocal.spearman_positions(pa, pb) - stats.spearmanr(pa, pb).statistic) < 1e-12


def test_stability_closed_forms():
    t = workloads.random_scas_table(2, 3, 5, 1)
    tok = (1, 4, 9, 16, 25)
    rho, jac = ocal.ranking_stability(t, t, tok, 0.5, 1)
    assert math.isnan(rho[0]) and math.isnan(rho[4])
    assert np.all(rho[1:4] == 1.0) and jac == 1.0
    # reversing every importance reverses every ordering (no ties): rho = -1
    rev = np.zeros_like(t)
    K = 5
    for s in range(K):
        for tt in range(s + 1, K):
            rev[:, :, tt, s] = 1.0 - t[:, :, tt, s]
    imp_t = osch.importance(t)
    imp_r = osch.importance(rev)
    ok = all(len(set(np.round(imp_t[:, :, s].ravel(), 9))) == 6 for s in range(1, 4))
    assert ok
    rho_r, _ = ocal.ranking_stability(t, rev, tok, 0.5, 1)
    np.testing.assert_allclose(rho_r[1:4], -1.0, atol=1e-12)
    assert np.allclose(imp_r[:, :, 1:4] + imp_t[:, :, 1:4], [[[3, 2, 1]]])


def test_library_matches_oracle():
    g = np.random.default_rng(3)
    for i in range(200):
        L, H, K = int(g.integers(1, 4)), int(g.integers(1, 6)), int(g.integers(2, 8))
        tok = workloads.random_tokens(K, i)
        a = workloads.random_scas_table(L, H, K, i)
        b = workloads.random_scas_table(L, H, K, 1000 + i)
        if i % 5 == 0:
            b = a.copy()
        beta = float(g.uniform(0.2, 1.0))
        n_sink = int(g.integers(0, K))
        try:
            want = ocal.ranking_stability(a, b, tok, beta, n_sink)
        except osch.ScheduleError:
            with pytest.raises(hk.HeatKVError):
                hk.ranking_stability(a, b, tok, beta, n_sink)
            continue
        rho, jac = hk.ranking_stability(a, b, tok, beta, n_sink)
        np.testing.assert_array_equal(np.isnan(rho), np.isnan(want[0]))
        np.testing.assert_allclose(rho[~np.isnan(rho)], want[0][~np.isnan(want[0])], rtol=0, atol=1e-12)
        assert abs(jac - want[1]) < 1e-15


def test_scas_mean_host():
    g = np.random.default_rng(4)
    s = g.random((2, 3, 4, 4))
    np.testing.assert_array_equal(hk.scas_mean(s, 7.0), (s / 7.0).astype(np.float32))
    with pytest.raises(hk.HeatKVError):
        hk.scas_mean(s, 0.0)


def _stability_cases():
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "stability_hand.json")) as f:
        doc = json.load(f)
    return doc, doc["cases"]


def _pruned_set(keep):
    L, H, K = keep.shape
    return {(l, h, s) for l in range(L) for h in range(H) for s in range(K - 1) if not keep[l, h, s]}


@pytest.mark.parametrize("case", range(3))
def test_stability_hand_worked(case):
    """Hand-worked pruned sets, Jaccard indices and rank correlations of two
    different tables (tests/golden/stability_hand.json): the oracle and the
    library both reproduce them."""
    doc, cases = _stability_cases()
    c = cases[case]
    a = np.asarray(c["a"], dtype=np.float32)
    b = np.asarray(c["b"], dtype=np.float32)
    tok, beta, n_sink = doc["tokens"], doc["beta"], doc["n_sink"]
    for tab, key in ((a, "pruned_a"), (b, "pruned_b")):
        keep = osch.build_schedule(tab, tok, beta, n_sink)[0]
        assert _pruned_set(keep) == {tuple(p) for p in c[key]}, (c["name"], key)
        lib_keep = hk.build_schedule(tab, tok, beta, n_sink)[0]
        assert _pruned_set(lib_keep) == {tuple(p) for p in c[key]}, (c["name"], key)
    want_rho = np.array([math.nan if r is None else r for r in c["rho"]])
    for rho, jac in (ocal.ranking_stability(a, b, tok, beta, n_sink),
                     hk.ranking_stability(a, b, tok, beta, n_sink)):
        assert abs(jac - c["jaccard"]) < 1e-12, (c["name"], jac)
        np.testing.assert_array_equal(np.isnan(rho), np.isnan(want_rho))
        np.testing.assert_allclose(rho[~np.isnan(rho)], want_rho[~np.isnan(want_rho)], rtol=0, atol=1e-12)


def test_stability_jaccard_catches_planted_mistakes():
    """The hand-worked Jaccard values separate the plausible slips: dividing
    by |G_a| instead of the union, or counting the final scale's unstored
    pairs as pruned."""
    doc, cases = _stability_cases()
    for c in cases:
        ga = {tuple(p) for p in c["pruned_a"]}
        gb = {tuple(p) for p in c["pruned_b"]}
        fin = {(0, h, 3) for h in range(doc["H"])}
        right = len(ga & gb) / len(ga | gb)
        assert abs(right - c["jaccard"]) < 1e-12
        if ga & gb and ga & gb != ga:
            assert abs(len(ga & gb) / len(ga) - c["jaccard"]) > 0.1
        wrong = len((ga | fin) & (gb | fin)) / len(ga | gb | fin)
        assert abs(wrong - c["jaccard"]) > 0.1
