"""Pins for the oracle's attention and S-CAS (CPU only).

Each check ties the oracle to something other than itself: a hand-worked
example, brute force in scalar Python, closed forms, and a textbook library
routine (PyTorch's masked scaled-dot-product attention in float64).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads
from oracle import attention as oatt
from oracle.numerics import to_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _random_case(seed, B=2, H=3, D=5, sides=(1, 2, 3), p_keep=0.5):
    g = np.random.default_rng(seed)
    K = len(sides)
    ks = [g.standard_normal((B, s * s, H, D)) for s in sides]
    vs = [g.standard_normal((B, s * s, H, D)) for s in sides]
    qs = [g.standard_normal((B, s * s, H, D)) for s in sides]
    keep = (g.random((H, K)) < p_keep).astype(np.uint8)
    keep[:, K - 1] = 0
    return qs, ks, vs, keep


def _brute(q_row, ks, vs, keep_h, t, b, h, alpha):
    """Scalar Python: walk scales and tokens, score, softmax, weighted sum."""
    keys, vals, owner = [], [], []
    for s in range(t + 1):
        if s < t and not keep_h[s]:
            continue
        for i in range(ks[s].shape[1]):
            keys.append([float(x) for x in ks[s][b, i, h, :]])
            vals.append([float(x) for x in vs[s][b, i, h, :]])
            owner.append(s)
    scores = [alpha * math.fsum(a * c for a, c in zip(q_row, kk)) for kk in keys]
    m = max(scores)
    e = [math.exp(x - m) for x in scores]
    z = math.fsum(e)
    w = [x / z for x in e]
    out = [math.fsum(w[j] * vals[j][d] for j in range(len(w))) for d in range(len(vals[0]))]
    mass = [math.fsum(w[j] for j in range(len(w)) if owner[j] == s) for s in range(t + 1)]
    return out, mass


def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "attention_hand.json")))
    kk = np.array(g["keys"])
    vv = np.array(g["values"])
    q = np.array(g["query"])
    ks = [kk[s].reshape(1, 1, 1, 2) for s in range(3)]
    vs = [vv[s].reshape(1, 1, 1, 2) for s in range(3)]
    for case in g["cases"]:
        t = case["t"]
        keep = np.array([case["keep"]], dtype=np.uint8)
        out, mass = oatt.attend_step(q.reshape(1, 1, 1, 2), ks[: t + 1], vs[: t + 1], keep, t, 1.0)
        np.testing.assert_allclose(out[0, 0, 0], case["out"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(oatt.scas_row(mass)[0], case["scas"], rtol=0, atol=1e-14)


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_random(seed):
    qs, ks, vs, keep = _random_case(seed)
    alpha = 0.7
    for t in range(len(ks)):
        out, mass = oatt.attend_step(qs[t], ks[: t + 1], vs[: t + 1], keep, t, alpha)
        B, n, H, D = qs[t].shape
        for b in range(B):
            for h in range(H):
                mass_sum = np.zeros(t + 1)
                for i in range(n):
                    o, m = _brute(qs[t][b, i, h], ks, vs, keep[h], t, b, h, alpha)
                    np.testing.assert_allclose(out[b, i, h], o, atol=1e-12, rtol=0)
                    mass_sum += np.array(m)
                np.testing.assert_allclose(mass[b, h], mass_sum / n, atol=1e-12, rtol=0)


def test_brute_force_tiny_workload():
    """All four steps of the tiny fp32 workload, with its random keep-mask."""
    wl = workloads.get("c0")
    keep = workloads.random_drop2_keep(wl)[0]
    assert keep[:, 0].all() and not keep[:, -1].any()
    assert int((keep[:, 1:3] == 0).sum()) == 2
    steps = [workloads.step_inputs(wl, 0, t) for t in range(wl.n_scales)]
    qs = [to_f64(s.q, "f32") for s in steps]
    ks = [to_f64(s.k, "f32") for s in steps]
    vs = [to_f64(s.v, "f32") for s in steps]
    for t in range(wl.n_scales):
        out, mass = oatt.attend_step(qs[t], ks[: t + 1], vs[: t + 1], keep, t, wl.softmax_scale)
        for h in range(wl.heads):
            acc = np.zeros(t + 1)
            for i in range(qs[t].shape[1]):
                o, m = _brute(qs[t][0, i, h], ks, vs, keep[h], t, 0, h, wl.softmax_scale)
                np.testing.assert_allclose(out[0, i, h], o, atol=1e-12, rtol=0)
                acc += np.array(m)
            np.testing.assert_allclose(mass[0, h], acc / qs[t].shape[1], atol=1e-12, rtol=0)


def test_first_scale_returns_its_value():
    """t = 0 with one token: the single key gets weight 1, so out = V_0."""
    qs, ks, vs, keep = _random_case(11, sides=(1, 2))
    out, mass = oatt.attend_step(qs[0], ks[:1], vs[:1], keep, 0, 1.3)
    np.testing.assert_array_equal(out, vs[0])
    np.testing.assert_array_equal(mass, np.ones_like(mass))


def test_zero_query_gives_uniform_weights():
    """q = 0: every key scores 0, weights are 1/|J|, out = mean(V_J), S-CAS = n_s/|J|."""
    qs, ks, vs, keep = _random_case(12, sides=(1, 2, 3, 2))
    t = 3
    q0 = np.zeros_like(qs[t])
    out, mass = oatt.attend_step(q0, ks[: t + 1], vs[: t + 1], keep, t, 1.0)
    B, n, H, D = q0.shape
    for b in range(B):
        for h in range(H):
            src = [s for s in range(t) if keep[h, s]] + [t]
            total = sum(ks[s].shape[1] for s in src)
            mean_v = sum(vs[s][b, :, h, :].sum(axis=0) for s in src) / total
            for i in range(n):
                np.testing.assert_allclose(out[b, i, h], mean_v, atol=1e-13, rtol=0)
            for s in range(t + 1):
                want = ks[s].shape[1] / total if s in src else 0.0
                assert abs(mass[b, h, s] - want) < 1e-14


def test_constant_values():
    """V = c everywhere: the output is c whatever the weights."""
    qs, ks, vs, keep = _random_case(13)
    vc = [np.full_like(v, -2.5) for v in vs]
    for t in range(3):
        out, _ = oatt.attend_step(qs[t], ks[: t + 1], vc[: t + 1], keep, t, 0.9)
        np.testing.assert_allclose(out, -2.5, atol=1e-13, rtol=0)


@pytest.mark.parametrize("seed", range(4))
def test_dropped_pair_equals_masking(seed):
    qs, ks, vs, keep = _random_case(100 + seed, sides=(1, 2, 3, 4))
    for t in range(4):
        a, _ = oatt.attend_step(qs[t], ks[: t + 1], vs[: t + 1], keep, t, 0.6)
        b = oatt.attend_step_masked(qs[t], ks[: t + 1], vs[: t + 1], keep, t, 0.6)
        np.testing.assert_allclose(a, b, atol=1e-13, rtol=0)


def test_full_budget_equals_textbook_block_causal_attention():
    """At 100% budget, stepping scale by scale equals one full-sequence
    softmax attention with a block-causal mask (PyTorch's
    scaled_dot_product_attention in float64 on the CPU)."""
    sides = (1, 2, 3, 4)
    qs, ks, vs, _ = _random_case(21, B=2, H=2, D=8, sides=sides)
    K = len(sides)
    keep = np.ones((2, K), dtype=np.uint8)
    keep[:, K - 1] = 0
    alpha = 0.4
    Q = np.concatenate(qs, axis=1)
    Kf = np.concatenate(ks, axis=1)
    Vf = np.concatenate(vs, axis=1)
    scale_of = np.concatenate([np.full(s * s, i) for i, s in enumerate(sides)])
    allowed = scale_of[None, :] <= scale_of[:, None]
    tq = torch.from_numpy(Q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(Kf).permute(0, 2, 1, 3)
    tv = torch.from_numpy(Vf).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=torch.from_numpy(allowed), scale=alpha).permute(0, 2, 1, 3).numpy()
    off = 0
    for t in range(K):
        out, _ = oatt.attend_step(qs[t], ks[: t + 1], vs[: t + 1], keep, t, alpha)
        n = qs[t].shape[1]
        np.testing.assert_allclose(out, ref[:, off:off + n], atol=1e-12, rtol=0)
        off += n


@pytest.mark.parametrize("seed", range(3))
def test_scas_rows_sum_to_one_and_dropped_sources_are_zero(seed):
    qs, ks, vs, keep = _random_case(300 + seed, sides=(1, 2, 3, 4), p_keep=0.5)
    for t in range(4):
        _, mass = oatt.attend_step(qs[t], ks[: t + 1], vs[: t + 1], keep, t, 1.0)
        row = oatt.scas_row(mass)
        np.testing.assert_allclose(row.sum(axis=1), 1.0, atol=1e-13, rtol=0)
        for h in range(keep.shape[0]):
            for s in range(t):
                if not keep[h, s]:
                    assert row[h, s] == 0.0


def test_sampled_rows_match_full():
    qs, ks, vs, keep = _random_case(41, sides=(1, 3, 4))
    t = 2
    full, _ = oatt.attend_step(qs[t], ks, vs, keep, t, 0.5)
    rows = [0, 5, 15]
    part, _ = oatt.attend_step(qs[t], ks, vs, keep, t, 0.5, q_rows=rows)
    np.testing.assert_array_equal(part, full[:, rows])


def test_planted_mistake_is_caught(monkeypatch):
    """A plausible slip (reading dropped segments anyway) must fail brute force."""
    qs, ks, vs, keep = _random_case(5, p_keep=0.0)
    monkeypatch.setattr(oatt, "kept_sources", lambda keep_lh, t: list(range(t + 1)))
    t = 2
    out, _ = oatt.attend_step(qs[t], ks, vs, keep, t, 1.0)
    o, _ = _brute(qs[t][0, 0, 0], ks, vs, keep[0], t, 0, 0, 1.0)
    assert np.abs(out[0, 0, 0] - np.array(o)).max() > 1e-3
