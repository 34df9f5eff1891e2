"""Compile the SeKV HIP library (libsekv.so) for gfx950, in-tree.

    python -m hierarchical_kv_cache_surprisal_amd.build_lib

Each source is compiled to an object in parallel, then linked into
hierarchical_kv_cache_surprisal_amd/libsekv.so.  hipcc cross-compiles, so no
GPU is needed.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libsekv.so")
BUILD = os.path.join(ROOT, "_build")

# (source, object name, extra defines): decode.hip builds once per route/attend
# kernel variant and once for the rest, so the variants compile in parallel
SOURCES = [("runtime.cpp", "runtime", []), ("plan.cpp", "plan", []), ("decode.hip", "decode", []), ("build.hip", "build", []),
           ("svd.hip", "svd", []), ("noalloc.hip", "noalloc", [])] + \
          [("decode.hip", f"decode_v{i}", [f"-DSEKV_DECODE_VARIANT={i}"]) for i in range(4)]

# the benchmark's streaming-read reference: a library of its own, outside the SeKV API
BENCH_SOURCES = [("bench_read.hip", "bench_read", [])]
BENCH_OUT = os.path.join(PKG, "libsekv_bench.so")

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = os.environ.get("SEKV_ARCH", "gfx950")

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", f"-I{INCLUDE}", f"-I{CSRC}",
          "-Wall", "-Wno-unused-function", "-Wno-unused-variable", "-Wno-unused-but-set-variable",
          # packed fp32 instructions disabled: the compiler still vectorises, without v_pk_*_f32
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


def _compile(job) -> str:
    src, name, defs = job
    obj = os.path.join(BUILD, name + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *COMMON, *defs, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if r.stderr.strip():
        warn = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
        if warn:
            sys.stderr.write("\n".join(warn) + "\n")
    return obj


def _link(objs, out, verbose):
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = SOURCES + BENCH_SOURCES
    with cf.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        objs = list(ex.map(_compile, jobs))
    _link(objs[:len(SOURCES)], OUT, verbose)
    _link(objs[len(SOURCES):], BENCH_OUT, verbose)
    return OUT


if __name__ == "__main__":
    build()
