"""The C-ABI library on the host (no GPU work): exports, schedule, layout, errors."""
import ctypes
import os
import re

import numpy as np
import pytest

import workloads
from oracle import cache as ocache
from oracle import policies as opol
from oracle import progressive as opr
from oracle import schedule as osch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "heatkv.h")
LIB = os.path.join(ROOT, "kv_cache_compression_attend_amd", "libheatkv.so")

if not os.path.exists(LIB):  # build only when nothing is built
    import subprocess
    import sys
    subprocess.run([sys.executable, os.path.join(ROOT, "kv_cache_compression_attend_amd", "build.py")],
                   check=True)

import kv_cache_compression_attend_amd as hk  # noqa: E402


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hk_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert len(names) == 26, names
    lib = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(lib, n), n


def test_single_hip_runtime_loaded():
    maps = open("/proc/self/maps").read()
    paths = {l.split()[-1] for l in maps.splitlines() if "libamdhip64" in l}
    assert len(paths) == 1, paths


def _same_as_oracle(table, tokens, beta, n_sink):
    try:
        want = osch.build_schedule(table, tokens, beta, n_sink)
    except osch.ScheduleError as e:
        with pytest.raises(hk.HeatKVError) as got:
            hk.build_schedule(table, tokens, beta, n_sink)
        assert got.value.name == e.code.upper()
        return None
    keep, ret, n = hk.build_schedule(table, tokens, beta, n_sink)
    np.testing.assert_array_equal(keep, want[0])
    np.testing.assert_array_equal(ret, want[1])
    assert n == want[2]
    return keep


@pytest.mark.parametrize("key", ["c0", "c1", "c2", "c3", "c4"])
def test_schedule_bit_exact_on_workload_tables(key):
    wl = workloads.get(key)
    table = workloads.dirichlet_scas(wl)
    for beta in (wl.budget, 0.2, 0.1, 0.04, 1.0):
        _same_as_oracle(table, wl.scale_tokens, beta, wl.n_sink)


def test_schedule_bit_exact_random_tables():
    g = np.random.default_rng(7)
    for i in range(1000):
        L, H, K = int(g.integers(1, 4)), int(g.integers(1, 6)), int(g.integers(1, 9))
        tokens = workloads.random_tokens(K, i, max_side=5)
        table = workloads.random_scas_table(L, H, K, i)
        if i % 7 == 0:  # plant exact ties
            table[:, :, :, :] = np.round(table * 4) / 4
        beta = float(g.choice([g.uniform(0.01, 1.0), 1.0, 0.5]))
        n_sink = int(g.integers(0, K))
        _same_as_oracle(table, tokens, beta, n_sink)


def test_schedule_errors():
    t = workloads.random_scas_table(1, 2, 4, 3)
    tok = (1, 4, 9, 16)
    for beta, ns in ((0.0, 1), (1.5, 1), (0.5, 4), (0.5, -1), (float("nan"), 1)):
        with pytest.raises(hk.HeatKVError) as e:
            hk.build_schedule(t, tok, beta, ns)
        assert e.value.status == hk.HK_EINVAL
    with pytest.raises(hk.HeatKVError) as e:
        hk.build_schedule(t, (1, 0, 9, 16), 0.5, 1)
    assert e.value.status == hk.HK_EINVAL
    with pytest.raises(hk.HeatKVError) as e:
        hk.build_schedule(t, tok, 0.01, 1)
    assert e.value.status == hk.HK_EBUDGET
    assert "sink" in hk._lib.hk_last_error().decode()


@pytest.mark.parametrize("key", ["c0", "c2", "c4"])
def test_layout_matches_oracle(key):
    wl = workloads.get(key)
    if wl.schedule == "random_drop2":
        keep = workloads.random_drop2_keep(wl)
    else:
        keep = osch.build_schedule(workloads.dirichlet_scas(wl), wl.scale_tokens, wl.budget,
                                   wl.n_sink)[0]
    elems, cap, base = hk.layout(wl.scale_tokens, keep, wl.batch, wl.head_dim)
    ocap = ocache.capacity(keep, wl.scale_tokens)
    np.testing.assert_array_equal(cap, ocap)
    np.testing.assert_array_equal(base, ocache.bases(ocap, wl.batch, wl.head_dim))
    assert elems * (2 if wl.dtype == "bf16" else 4) == ocache.cache_bytes(
        keep, wl.scale_tokens, wl.batch, wl.head_dim, 2 if wl.dtype == "bf16" else 4)


def test_null_and_range_errors_without_gpu():
    lib = hk._lib
    assert lib.hk_attend(None, 0, 0, None, None, None, None, 1.0, None) == hk.HK_EINVAL
    assert lib.hk_append_scale(None, 0, 1, 0, None, None, 0, None) == hk.HK_EINVAL
    assert lib.hk_attend_append(None, 0, 0, None, None, None, None, 1.0, None, None) == hk.HK_EINVAL
    assert lib.hk_reset(None) == hk.HK_EINVAL
    r32 = ctypes.c_int32()
    assert lib.hk_attend_plan(None, 0, 0, ctypes.byref(r32), ctypes.byref(r32)) == hk.HK_EINVAL
    assert lib.hk_destroy(None) == hk.HK_OK
    out = ctypes.c_int64()
    assert lib.hk_retained_tokens(None, 0, ctypes.byref(out)) == hk.HK_EINVAL
    tok = np.array([1, 4], dtype=np.int32)
    keep = np.ones((1, 1, 2), dtype=np.uint8)
    h = ctypes.c_void_p()
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    assert lib.hk_create(ctypes.byref(h), 1, 1, 64, 1, 2, p(tok), p(keep), hk.HK_DTYPE_BF16,
                         None, None) == hk.HK_EUNSUPPORTED
    assert lib.hk_create(ctypes.byref(h), 1, 1, 128, 1, 17, p(np.ones(17, np.int32)),
                         p(np.ones(17, np.uint8)), hk.HK_DTYPE_BF16, None, None) == hk.HK_EUNSUPPORTED
    assert lib.hk_create(ctypes.byref(h), 1, 1, 24, 1, 2, p(tok), p(keep), hk.HK_DTYPE_F32,
                         None, None) == hk.HK_EUNSUPPORTED
    assert lib.hk_create(ctypes.byref(h), 0, 1, 16, 1, 2, p(tok), p(keep), hk.HK_DTYPE_F32,
                         None, None) == hk.HK_EINVAL
    assert lib.hk_create(ctypes.byref(h), 1, 1, 16, 1, 2, p(tok), p(keep), hk.HK_DTYPE_F32,
                         None, None) == hk.HK_EINVAL  # null cache with a non-empty layout


def _progressive_same(table, tokens, beta, n_sink, per_layer):
    try:
        want = opr.progressive_schedule(table, tokens, beta, n_sink, per_layer)
    except osch.ScheduleError as e:
        with pytest.raises(hk.HeatKVError) as got:
            hk.build_progressive_schedule(table, tokens, beta, n_sink, per_layer)
        assert got.value.name == e.code.upper()
        return None
    exp, n, live = hk.build_progressive_schedule(table, tokens, beta, n_sink, per_layer)
    np.testing.assert_array_equal(exp, want[0])
    np.testing.assert_array_equal(n, want[1])
    np.testing.assert_array_equal(live, want[2])
    return exp


def test_progressive_schedule_bit_exact_random_tables():
    g = np.random.default_rng(11)
    for i in range(400):
        L, H, K = int(g.integers(1, 4)), int(g.integers(1, 5)), int(g.integers(1, 8))
        tokens = workloads.random_tokens(K, 500 + i, max_side=5)
        table = workloads.random_scas_table(L, H, K, 500 + i)
        if i % 7 == 0:
            table[:, :, :, :] = np.round(table * 4) / 4
        beta = float(g.choice([g.uniform(0.01, 1.0), 1.0, 0.3]))
        n_sink = int(g.integers(0, K))
        exp = _progressive_same(table, tokens, beta, n_sink, bool(i % 2))
        if exp is None:
            continue
        L, H, K = exp.shape
        for k in range(K):
            for l in range(L):
                want = sum(opr.rows_at_end(exp[ll, h], tokens, k if ll <= l else k - 1)
                           for ll in range(L) for h in range(H) if ll <= l or k > 0)
                assert hk.cache_size_after_layer(tokens, exp, k, l) == want


@pytest.mark.parametrize("key", ["c2", "c4"])
def test_progressive_schedule_bit_exact_on_workload_tables(key):
    wl = workloads.get(key)
    table = workloads.dirichlet_scas(wl)
    exp = _progressive_same(table, wl.scale_tokens, wl.budget, wl.n_sink, True)
    elems, cap, base = hk.layout_expiry(wl.scale_tokens, exp, wl.batch, wl.head_dim)
    ocap = opr.capacity(exp, wl.scale_tokens)
    np.testing.assert_array_equal(cap, ocap)
    np.testing.assert_array_equal(base, ocache.bases(ocap, wl.batch, wl.head_dim))
    assert elems == int(ocap.sum()) * wl.batch * wl.head_dim


def test_layout_of_keep_equals_layout_of_its_expiry():
    wl = workloads.get("c2")
    keep = osch.build_schedule(workloads.dirichlet_scas(wl), wl.scale_tokens, wl.budget, wl.n_sink)[0]
    a = hk.layout(wl.scale_tokens, keep, wl.batch, wl.head_dim)
    b = hk.layout_expiry(wl.scale_tokens, opr.expire_from_keep(keep), wl.batch, wl.head_dim)
    assert a[0] == b[0]
    np.testing.assert_array_equal(a[1], b[1])
    np.testing.assert_array_equal(a[2], b[2])


def test_expiry_errors():
    tok = (1, 4, 9)
    bad = np.array([[[0, 2, 2]]], dtype=np.uint8)  # segment 0 leaves at step 0: fine
    assert hk.cache_size_after_layer(tok, bad, 1, 0) == 4
    for wrong in ([[[0, 0, 2]]], [[[3, 2, 2]]], [[[0, 1, 1]]]):
        e_ = np.array(wrong, dtype=np.uint8)
        with pytest.raises(hk.HeatKVError) as e:
            hk.layout_expiry(tok, e_, 1, 16)
        assert e.value.status == hk.HK_EINVAL
        with pytest.raises(hk.HeatKVError) as e:
            hk.cache_size_after_layer(tok, e_, 0, 0)
        assert e.value.status == hk.HK_EINVAL
    with pytest.raises(hk.HeatKVError) as e:
        hk.cache_size_after_layer(tok, bad, 3, 0)
    assert e.value.status == hk.HK_EINVAL
    lib = hk._lib
    h = ctypes.c_void_p()
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    wrong = np.array([[[0, 0, 2]]], dtype=np.uint8)
    assert lib.hk_create_expiry(ctypes.byref(h), 1, 1, 16, 1, 3, p(np.array(tok, np.int32)), p(wrong),
                                hk.HK_DTYPE_F32, None, None) == hk.HK_EINVAL
    t = workloads.random_scas_table(1, 2, 4, 3)
    with pytest.raises(hk.HeatKVError) as e:
        hk.build_progressive_schedule(t, (1, 4, 9, 16), 0.01, 1)
    assert e.value.status == hk.HK_EBUDGET


def test_scale_window_schedule_matches_oracle():
    g = np.random.default_rng(3)
    for i in range(300):
        L, H, K = int(g.integers(1, 6)), int(g.integers(1, 4)), int(g.integers(1, 14))
        tokens = workloads.random_tokens(K, 900 + i, max_side=6)
        c, w, wd = int(g.integers(0, K + 1)), int(g.integers(0, K + 2)), int(g.integers(0, K + 2))
        nd = int(g.integers(0, L + 1))
        sim = np.round(g.random(L) * 3).astype(np.float32)  # ties
        got = hk.build_scale_window_schedule(L, H, tokens, c, w, wd, sim, nd)
        want = opol.scale_window_schedule(L, H, tokens, c, w, wd, sim, nd)
        np.testing.assert_array_equal(got, want)
    with pytest.raises(hk.HeatKVError) as e:
        hk.build_scale_window_schedule(2, 1, (1, 4), 1, 1, 1, None, 1)
    assert e.value.status == hk.HK_EINVAL


def test_int4_layout_matches_its_definition():
    for key in ("c0", "c2", "c4"):
        wl = workloads.get(key)
        keep = workloads.random_drop2_keep(wl) if wl.schedule == "random_drop2" else \
            osch.build_schedule(workloads.dirichlet_scas(wl), wl.scale_tokens, wl.budget, wl.n_sink)[0]
        for m in (1, 2, 8):
            if wl.head_dim != 128:
                with pytest.raises(hk.HeatKVError) as e:
                    hk.layout_int4(wl.scale_tokens, keep, wl.batch, wl.head_dim, m)
                assert e.value.status == hk.HK_EUNSUPPORTED
                continue
            nbytes, poff = hk.layout_int4(wl.scale_tokens, keep, wl.batch, wl.head_dim, m)
            cap = ocache.capacity(keep, wl.scale_tokens)
            code = int(cap.sum()) * wl.batch * 64
            assert poff == (code + 255) // 256 * 256
            stored = int(keep[:, :, : wl.n_scales - 1].sum())
            assert nbytes == poff + stored * m * wl.batch * 128 * 8
    with pytest.raises(hk.HeatKVError) as e:
        hk.layout_int4((1, 4), np.ones((1, 1, 2), np.uint8), 1, 128, 0)
    assert e.value.status == hk.HK_EINVAL


def test_header_is_plain_c_and_links(tmp_path):
    """The boundary is a C ABI: the header compiles as C99 and a C program
    links against the library and calls a host entry point."""
    import shutil
    import subprocess
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    src = tmp_path / "probe.c"
    src.write_text(r'''
#include <stdio.h>
#include "heatkv.h"
int main(void) {
  int32_t tok[3] = {1, 4, 9};
  uint8_t keep[3] = {1, 1, 0};
  int64_t elems = 0;
  int rc = hk_layout(1, 1, 3, tok, keep, 2, 16, &elems, NULL, NULL);
  printf("%d %lld\n", rc, (long long)elems);
  rc = hk_layout(0, 1, 3, tok, keep, 2, 16, &elems, NULL, NULL);
  printf("%d %s\n", rc, hk_last_error());
  return 0;
}
''')
    exe = tmp_path / "probe"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe), LIB, "-Wl,-rpath," + os.path.dirname(LIB)],
                   check=True, capture_output=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    assert out[0] == "0 160"            # (1 + 4) rows x batch 2 x 16 dims
    assert out[1].startswith(str(hk.HK_EINVAL) + " ")
