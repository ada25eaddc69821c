"""Build libheatkv.so in-tree: host C++ with g++, HIP kernels with hipcc for gfx950.

Usage: python kv_cache_compression_attend_amd/build.py  (run by path: importing
the package would load the library being rebuilt).  Always recompiles every
source.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libheatkv.so")

HOST_SOURCES = ["schedule.cpp"]
HIP_SOURCES = ["context.hip", "attend_bf16.hip", "attend_f32.hip", "scas_finalize.hip",
               "compact.hip", "quant.hip", "noalloc.hip"]
ARCH = "gfx950"


def _rocm() -> str:
    return os.environ.get("ROCM_PATH", "/opt/rocm")


def _hipcc() -> str:
    p = shutil.which("hipcc") or os.path.join(_rocm(), "bin", "hipcc")
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return p


def hip_flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
            # packed fp32 arithmetic is kept out of generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include")]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    jobs = []
    for src in HOST_SOURCES:
        obj = os.path.join(OBJ, src + ".o")
        jobs.append(["g++", "-std=c++17", "-O2", "-fPIC", "-Wall", "-Wextra",
                     "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, src), "-o", obj])
    for src in HIP_SOURCES:
        obj = os.path.join(OBJ, src + ".o")
        jobs.append([_hipcc()] + hip_flags() + ["-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    objs = [os.path.join(OBJ, s + ".o") for s in HOST_SOURCES + HIP_SOURCES]
    tmp = LIB + ".tmp"
    _run([_hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs +
         ["-Wl,-rpath," + os.path.join(_rocm(), "lib")])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
