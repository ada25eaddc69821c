"""The library's host code (schedules, layouts, ranking stability) under
AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

tests/host_sanitize.cpp is built with g++ against the host source directly
(no device code) and driven over random valid and invalid cases; it must
finish with no sanitizer report, and every status code and output must equal
the production library's for the same call.
"""
import ctypes
import os
import shutil
import struct
import subprocess

import numpy as np
import pytest

import workloads

import kv_cache_compression_attend_amd as hk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "tests", "host_sanitize.cpp"),
       os.path.join(ROOT, "kv_cache_compression_attend_amd", "csrc", "schedule.cpp")]


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    if not shutil.which("g++"):
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("san") / "host_sanitize")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include")] + SRC + ["-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        if "sanitize" in r.stderr and ("cannot find" in r.stderr or "unrecognized" in r.stderr):
            pytest.skip("sanitizer runtime not available: " + r.stderr[-300:])
        raise AssertionError(r.stderr)
    return exe


def _i32(*v):
    return struct.pack(f"<{len(v)}i", *v)


def _cases(seed=0, n=240):
    """(op, args dict, packed input bytes) for random valid and invalid calls."""
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        op = [1, 2, 3, 4, 5, 6, 7, 8, 9][i % 9]
        L, H, K = int(g.integers(1, 4)), int(g.integers(1, 6)), int(g.integers(1, 9))
        tok = np.array(workloads.random_tokens(K, 1000 + i), dtype=np.int32)
        if i % 23 == 0:
            tok[int(g.integers(0, K))] = 0                      # invalid: an empty scale
        a = dict(op=op, L=L, H=H, K=K, tok=tok)
        data = _i32(op, L, H, K)
        if op == 9:
            a["sum"] = g.random((L, H, K, K))
            a["images"] = float(g.choice([0.0, 3.0, 7.5])) if i % 5 == 0 else 4.0
            out.append((a, data + a["sum"].astype("<f8").tobytes() + struct.pack("<d", a["images"])))
            continue
        data += tok.astype("<i4").tobytes()
        if op in (1, 2, 7):
            a["scas"] = workloads.random_scas_table(L, H, K, 2000 + i)
            if i % 7 == 0:
                a["scas"][:, :, K - 1, :] = a["scas"][0, 0, K - 1, :]  # planted ties
            a["beta"] = float(g.choice([0.0, 0.05, 0.3, 0.7, 1.0, 1.5])) if i % 4 == 0 else \
                float(g.uniform(0.2, 1.0))
            a["n_sink"] = int(g.integers(-1, K + 1)) if i % 6 == 0 else int(g.integers(0, K))
            data += a["scas"].astype("<f4").tobytes()
            if op == 7:
                a["scas_b"] = workloads.random_scas_table(L, H, K, 3000 + i)
                data += a["scas_b"].astype("<f4").tobytes()
            data += struct.pack("<d", a["beta"]) + _i32(a["n_sink"])
            if op == 2:
                a["per_layer"] = int(i % 2)
                data += _i32(a["per_layer"])
        elif op in (3, 4, 6, 8):
            if op in (6, 8):
                sched = (g.random((L, H, K)) < 0.6).astype(np.uint8)
            else:
                sched = np.zeros((L, H, K), dtype=np.uint8)
                for s in range(K):
                    sched[:, :, s] = g.integers(s, K, size=(L, H))
                if i % 5 == 0:
                    sched[0, 0, K - 1] = K                        # invalid expiry step
            a["sched"] = sched
            data += sched.tobytes()
            if op == 4:
                a["step"], a["layer"] = int(g.integers(-1, K + 1)), int(g.integers(-1, L + 1))
                data += _i32(a["step"], a["layer"])
            else:
                a["B"], a["D"] = int(g.integers(1, 5)), int(g.choice([16, 64, 128]))
                data += _i32(a["B"], a["D"])
                if op == 6:
                    a["m"] = int(g.integers(0, 5))
                    data += _i32(a["m"])
        elif op == 5:
            a["nc"], a["w"], a["wd"] = int(g.integers(0, K + 1)), int(g.integers(-1, K + 1)), \
                int(g.integers(-1, K + 2))
            a["sim"] = g.random(L).astype(np.float32)
            a["nd"] = int(g.integers(-1, L + 2))
            data += _i32(a["nc"], a["w"], a["wd"]) + a["sim"].astype("<f4").tobytes() + _i32(a["nd"])
        out.append((a, data))
    return out


def _p(x):
    return x.ctypes.data_as(ctypes.c_void_p)


def _production(a):
    """(status, list of output arrays) of the same call on libheatkv.so."""
    lib = hk._lib
    op, L, H, K, tok = a["op"], a["L"], a["H"], a["K"], a["tok"]
    lh, lhk = L * H, L * H * K
    if op == 9:
        res = np.zeros(lhk * K, dtype=np.float32)
        return lib.hk_scas_mean(L, H, K, _p(np.ascontiguousarray(a["sum"])), a["images"], _p(res)), [res]
    if op == 1:
        keep, ret, npr = np.zeros(lhk, np.uint8), np.zeros(K, np.int64), np.zeros(1, np.int32)
        rc = lib.hk_build_schedule(L, H, K, _p(tok), _p(a["scas"]), a["beta"], a["n_sink"], _p(keep),
                                   _p(ret), _p(npr))
        return rc, [keep, ret, npr]
    if op == 2:
        e, pre, live = np.zeros(lhk, np.uint8), np.zeros(K, np.int32), np.zeros(K * L, np.int64)
        rc = lib.hk_build_progressive_schedule(L, H, K, _p(tok), _p(a["scas"]), a["beta"], a["n_sink"],
                                               a["per_layer"], _p(e), _p(pre), _p(live))
        return rc, [e, pre, live]
    if op in (3, 8):
        el, cap, base = np.zeros(1, np.int64), np.zeros(lh, np.int64), np.zeros(lh, np.int64)
        fn = lib.hk_layout_expiry if op == 3 else lib.hk_layout
        rc = fn(L, H, K, _p(tok), _p(a["sched"]), a["B"], a["D"], _p(el), _p(cap), _p(base))
        return rc, [el, cap, base]
    if op == 4:
        sz = np.zeros(1, np.int64)
        rc = lib.hk_cache_size_after_layer(L, H, K, _p(tok), _p(a["sched"]), a["step"], a["layer"], _p(sz))
        return rc, [sz]
    if op == 5:
        e = np.zeros(lhk, np.uint8)
        rc = lib.hk_build_scale_window_schedule(L, H, K, _p(tok), a["nc"], a["w"], a["wd"], _p(a["sim"]),
                                                a["nd"], _p(e))
        return rc, [e]
    if op == 6:
        st, po = np.zeros(1, np.int64), np.zeros(1, np.int64)
        rc = lib.hk_layout_int4(L, H, K, _p(tok), _p(a["sched"]), a["B"], a["D"], a["m"], _p(st), _p(po))
        return rc, [st, po]
    rho, jac = np.zeros(K, np.float64), np.zeros(1, np.float64)
    rc = lib.hk_ranking_stability(L, H, K, _p(tok), _p(a["scas"]), _p(a["scas_b"]), a["beta"],
                                  a["n_sink"], _p(rho), _p(jac))
    return rc, [rho, jac]


def test_host_entry_points_under_sanitizers(harness, tmp_path):
    cases = _cases()
    src = tmp_path / "in.bin"
    dst = tmp_path / "out.bin"
    src.write_bytes(b"".join(d for _, d in cases))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([harness, str(src), str(dst)], capture_output=True, text=True, env=env,
                       timeout=300)
    assert r.returncode == 0 and "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, \
        r.stderr[-3000:]
    blob = dst.read_bytes()
    at = 0
    n_ok = n_err = 0
    for a, _ in cases:
        (rc,) = struct.unpack_from("<i", blob, at)
        at += 4
        want_rc, outs = _production(a)
        assert rc == want_rc, (a["op"], rc, want_rc)
        if rc != 0:
            n_err += 1
            continue
        n_ok += 1
        for arr in outs:
            got = np.frombuffer(blob, dtype=arr.dtype, count=arr.size, offset=at)
            at += arr.nbytes
            np.testing.assert_array_equal(got, arr, err_msg=str(a["op"]))
    assert at == len(blob)
    assert n_ok > 100 and n_err > 20, (n_ok, n_err)
