"""Pins of the 4-bit cache quantizer (``oracle.quant``): hand-worked values,
an independent pure-Python float32 brute force, the rounding error bound,
packing, sub-block partitions, and attention over exactly representable
groups equal to plain attention."""
import json
import os
import struct

import numpy as np

import workloads
from oracle import attention as oatt
from oracle import quant as oq

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quant_hand.json")


def _f32(v):
    """Round a Python float to the nearest float32 (ties to even)."""
    return struct.unpack("f", struct.pack("f", v))[0]


def test_hand_worked_groups_and_packing():
    g = json.load(open(GOLDEN))
    for case in g["groups"]:
        codes, step, lo = oq.quantize_group(np.array(case["x"], dtype=np.float32))
        assert codes.tolist() == case["codes"], case
        assert lo == np.float32(case["lo"]) and step == np.float32(case["step"])
    pk = g["packing"]
    packed = oq.pack(np.array([pk["codes"]], dtype=np.uint8))
    assert packed[0].tolist() == pk["bytes"]
    assert oq.unpack(packed)[0].tolist() == pk["codes"]


def test_float32_arithmetic_matches_python_brute_force():
    rng = np.random.default_rng(0)
    for trial in range(300):
        n = int(rng.integers(1, 40))
        x = (rng.standard_normal(n) * rng.choice([0.01, 0.3, 5.0])).astype(np.float32)
        if trial % 10 == 0:
            x[: n // 2] = x[0]                      # repeated values
        codes, step, lo = oq.quantize_group(x)
        xs = [float(v) for v in x]
        lo_b = min(xs)
        hi_b = max(xs)
        step_b = _f32(_f32(hi_b - lo_b) / 15.0)
        assert float(lo) == lo_b and float(step) == step_b
        for v, c in zip(xs, codes.tolist()):
            if step_b == 0.0:
                want = 0
            else:
                r = _f32(_f32(v - lo_b) / step_b)
                want = min(15, max(0, int(round(r))))   # Python rounds half to even
            assert c == want, (v, lo_b, step_b)


def test_rounding_error_bound():
    rng = np.random.default_rng(1)
    for _ in range(200):
        n = int(rng.integers(1, 300))
        seg = (rng.standard_normal((n, 8)) * 0.3).astype(np.float32)
        for m in (1, 2, 3, 8):
            codes, step, lo = oq.quantize_segment(seg, m)
            deq = oq.dequantize_segment(codes, step, lo, m)
            for j, (a, b) in enumerate(oq.sub_block_bounds(n, m)):
                bound = step[j].astype(np.float64) * (0.5 + 1e-5) + 1e-12
                assert (np.abs(deq[a:b] - seg[a:b]) <= bound).all()
                if b > a:   # the extremes come back exactly
                    np.testing.assert_array_equal(deq[a:b].min(axis=0), seg[a:b].min(axis=0))


def test_sub_block_partition():
    for n in range(1, 70):
        for m in range(1, 10):
            bounds = oq.sub_block_bounds(n, m)
            assert bounds[0][0] == 0 and bounds[-1][1] == n
            assert all(bounds[j][1] == bounds[j + 1][0] for j in range(m - 1))
            sizes = [b - a for a, b in bounds]
            assert max(sizes) - min(sizes) <= 1
    assert oq.sub_block_bounds(5, 1) == [(0, 5)]
    assert oq.sub_block_bounds(1, 2) == [(0, 0), (0, 1)]


def test_pack_unpack_round_trip():
    rng = np.random.default_rng(2)
    codes = rng.integers(0, 16, size=(37, 128)).astype(np.uint8)
    packed = oq.pack(codes)
    assert packed.shape == (37, 64)
    for i in (0, 5, 36):
        for c in (0, 1, 126, 127):
            byte = int(packed[i, c // 2])
            assert ((byte >> (4 * (c % 2))) & 15) == codes[i, c]
    np.testing.assert_array_equal(oq.unpack(packed), codes)


def test_attention_over_exact_groups_is_plain_attention():
    """Values on a 4-bit grid with a power-of-two step survive quantization
    exactly, so attention over the stored segments equals the oracle's plain
    attention over the same values."""
    wl = workloads.get("c0")
    rng = np.random.default_rng(3)
    tokens = wl.scale_tokens
    B, H, D = 1, 2, 16

    def grid(n):
        x = rng.integers(0, 16, size=(B, n, H, D)).astype(np.float32) * 0.25 - 1.0
        x[:, 0] = -1.0      # every group spans the full grid: lo = -1, step = 0.25
        x[:, -1] = 2.75
        return x
    ks = [grid(n) for n in tokens]
    vs = [grid(n) for n in tokens]
    q = rng.standard_normal((B, tokens[-1], H, D))
    keep = np.array([1, 0, 1, 0], dtype=np.uint8)
    t = len(tokens) - 1
    for h in range(H):
        want, _ = oatt.softmax_attention(q[0, :, h, :], *oatt.gather_keys(ks, vs, keep, t, 0, h)[:2],
                                         wl.softmax_scale)
        got = oq.attend_rows(q, ks, vs, keep, t, 0, h, 1, wl.softmax_scale)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
        # a wrong grouping (two sub-blocks) does not reproduce the values exactly
        assert np.abs(oq.attend_rows(q, ks, vs, keep, t, 0, h, 4, wl.softmax_scale) - want).max() > 1e-9
