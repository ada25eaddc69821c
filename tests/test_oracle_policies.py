"""Pins of the condensed + local scale-window policy (``oracle.policies``):
what each scale reads, checked by brute force from the policy's wording, and
closed forms of the cache it keeps."""
import numpy as np

import workloads
from oracle import policies as opol
from oracle import progressive as opr
from oracle import schedule as osch


def test_each_scale_reads_condensed_and_local_scales():
    tokens = workloads.get("c1").scale_tokens
    K = len(tokens)
    for c in range(0, 4):
        for w in range(0, K + 1):
            exp = opol.scale_window_schedule(1, 2, tokens, c, w, w)
            for t in range(K):
                want = [1 if (s < t and (s < c or s >= t - w)) else 0 for s in range(K)]
                assert opr.visible(exp[0, 0], t) == want, (c, w, t)


def test_demanding_layers_get_the_wide_window():
    sim = [0.9, 0.1, 0.5, 0.1, 0.7]
    assert opol.demanding_layers(sim, 2) == [1, 3]     # ties: lower index first
    assert opol.demanding_layers(sim, 3) == [1, 2, 3]
    tokens = (1, 4, 9, 16, 25)
    exp = opol.scale_window_schedule(5, 1, tokens, 1, 1, 4, sim, 2)
    for l in range(5):
        wide = l in (1, 3)
        assert opr.visible(exp[l, 0], 4) == ([1, 1, 1, 1, 0] if wide else [1, 0, 0, 1, 0])


def test_full_window_is_the_full_cache_and_zero_window_keeps_condensed_only():
    wl = workloads.get("c2")
    K = wl.n_scales
    full = opol.scale_window_schedule(wl.layers, wl.heads, wl.scale_tokens, 0, K, K)
    keep = np.ones((wl.layers, wl.heads, K), dtype=np.uint8)
    np.testing.assert_array_equal(full, opr.expire_from_keep(keep))
    none = opol.scale_window_schedule(wl.layers, wl.heads, wl.scale_tokens, 2, 0, 0)
    r = opr.retained_per_step(none, wl.scale_tokens)
    heads = wl.layers * wl.heads
    for k in range(K):
        assert r[k] == heads * sum(wl.scale_tokens[s] for s in range(min(k + 1, 2)))


def test_retained_closed_form():
    """End of scale k: condensed scales <= k plus the local scales
    max(c, k-w+1) .. k (those that a later scale still reads)."""
    tokens = workloads.get("c1").scale_tokens
    K = len(tokens)
    for c in (0, 1, 2, 3):
        for w in (1, 2, 3, 5):
            exp = opol.scale_window_schedule(2, 3, tokens, c, w, w)
            r = opr.retained_per_step(exp, tokens)
            for k in range(K):
                kk = min(k, K - 2)
                segs = set(range(min(c, kk + 1))) | set(range(max(c, kk - w + 1), kk + 1))
                assert r[k] == 6 * sum(tokens[s] for s in segs), (c, w, k)


def test_invalid_arguments():
    for args in (dict(n_condensed=-1), dict(window=-1), dict(n_demanding=1)):
        kw = dict(n_condensed=1, window=1, window_demanding=1)
        kw.update(args)
        try:
            opol.scale_window_schedule(2, 1, (1, 4, 9), **kw)
        except osch.ScheduleError as e:
            assert e.code == "einval"
        else:
            raise AssertionError(args)
