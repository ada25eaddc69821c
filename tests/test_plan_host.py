"""The launch-plan model on the host (no GPU): the plans the default workload
runs with, and the model's invariants over a grid of launch shapes."""
import itertools

import pytest

import kv_cache_compression_attend_amd as hk
import workloads


def full_cache_max_keys(tokens, t):
    return sum(tokens[: t + 1])


def test_plans_of_the_full_cache_layer_at_batch_1():
    """The plans of the 16-head full-cache layer, batch 1, scale by scale: the
    choices the cost model makes there, each checked on the MI355X against
    every alternative (128-query tiles for the tiny scales, single-tile splits
    at scale 5, splits for 6-11, one unsplit 256-query launch at the end)."""
    wl = workloads.get("c1")
    tokens = wl.scale_tokens
    got = [hk.plan_attend_bf16(1, wl.heads, tokens[t], full_cache_max_keys(tokens, t))
           for t in range(wl.n_scales)]
    want = [(128, 1)] * 4 + [(256, 1), (256, 5), (256, 3), (256, 5), (256, 4), (256, 4),
                             (256, 2), (256, 3), (256, 1)]
    assert got == want


@pytest.mark.parametrize("key", ["c1", "c2", "c3", "c4"])
def test_final_scale_is_one_unsplit_256_query_launch(key):
    """The final scale (4,096 queries per head) fills the chip with 256-query
    tiles at every workload's batch: the launch the roofline figure times."""
    wl = workloads.get(key)
    tokens = wl.scale_tokens
    t = wl.n_scales - 1
    assert hk.plan_attend_bf16(wl.batch, wl.heads, tokens[t], full_cache_max_keys(tokens, t)) == (256, 1)


def test_model_invariants_over_launch_shapes():
    for B, H, n, keys in itertools.product((1, 2, 3, 8, 16), (1, 3, 16, 28), (1, 16, 100, 256, 1024, 4096),
                                           (1, 63, 64, 65, 500, 4000, 12000)):
        keys = max(keys, n)
        tiles = -(-keys // 64)
        rows, splits = hk.plan_attend_bf16(B, H, n, keys)
        assert rows in (128, 256)
        assert 1 <= splits <= 16 and splits <= tiles
        assert splits == 1 or rows == 256
        # S-CAS launches never split; the tiling may differ
        r2, s2 = hk.plan_attend_bf16(B, H, n, keys, allow_split=False)
        assert s2 == 1 and r2 in (128, 256)


def test_invalid_sizes_are_rejected():
    for args in ((0, 1, 1, 1), (1, 0, 1, 1), (1, 1, 0, 1), (1, 1, 1, 0)):
        with pytest.raises(hk.HeatKVError) as e:
            hk.plan_attend_bf16(*args)
        assert e.value.status == hk.HK_EINVAL
