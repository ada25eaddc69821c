"""Seeded input generators and the oracle's bf16 decode (CPU only)."""
import numpy as np

import workloads
from oracle.numerics import bf16_bits_to_f64


def test_bf16_round_to_nearest_even():
    f = np.array([0x3F800000, 0xC0000000, 0x3DCCCCCD, 0x3F808000, 0x3F818000,
                  0x3F80FFFF, 0x00000000, 0x80000000], dtype=np.uint32).view(np.float32)
    want = [0x3F80, 0xC000, 0x3DCD, 0x3F80, 0x3F82, 0x3F81, 0x0000, 0x8000]
    assert workloads.round_to_bf16_bits(f).tolist() == want


def test_bf16_decode_exact():
    bits = np.array([0x3F80, 0xC000, 0x3DCD, 0x7F7F, 0x0001], dtype=np.uint16)
    got = bf16_bits_to_f64(bits)
    assert got[0] == 1.0 and got[1] == -2.0
    assert got[2] == 0.10009765625
    assert got[3] == (2 - 2 ** -7) * 2.0 ** 127
    assert got[4] == 2.0 ** -133


def test_step_inputs_deterministic_and_independent():
    wl = workloads.get("c1")
    a = workloads.step_inputs(wl, 0, 3)
    b = workloads.step_inputs(wl, 0, 3)
    assert a.q.shape == (1, 36, 16, 128) and a.q.dtype == np.uint16
    np.testing.assert_array_equal(a.k, b.k)
    c = workloads.step_inputs(wl, 0, 4)
    assert not np.array_equal(a.q[:, :1], c.q[:, :1])
    # distribution: Q ~ N(0,1) * d^-1/4
    big = bf16_bits_to_f64(workloads.step_inputs(wl, 0, 12).q)
    assert abs(big.std() - 128 ** -0.25) < 0.01


def test_key_offsets_shift_keys():
    wl = workloads.get("c3")
    mu = workloads.key_offsets(wl)
    assert mu.shape == (16, 13)
    k = bf16_bits_to_f64(workloads.step_inputs(wl, 0, 12, batch=1).k)
    means = k.mean(axis=(0, 1, 3)) / wl.qk_std
    np.testing.assert_allclose(means, mu[:, 12], atol=0.05)


def test_dirichlet_table_rows():
    wl = workloads.get("c2")
    t = workloads.dirichlet_scas(wl)
    assert t.shape == (32, 16, 13, 13) and t.dtype == np.float32
    np.testing.assert_allclose(t.sum(axis=3), 1.0, atol=1e-5)
    assert np.all(np.triu(t[0, 0], 1) == 0)


def test_leading_batch_entries_are_a_prefix_of_the_full_draw():
    wl = workloads.get("c2")
    full = workloads.step_inputs(wl, 3, 5)
    for nb in (1, 3):
        part = workloads.step_inputs(wl, 3, 5, batch=nb)
        for a, b in ((part.q, full.q), (part.k, full.k), (part.v, full.v)):
            np.testing.assert_array_equal(a, b[:nb])
    wl3 = workloads.get("c3")
    np.testing.assert_array_equal(workloads.step_inputs(wl3, 0, 6, batch=2).k,
                                  workloads.step_inputs(wl3, 0, 6).k[:2])
