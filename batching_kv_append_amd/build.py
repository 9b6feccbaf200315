"""Build libkvc.so (gfx950) in-tree with hipcc.

``python batching_kv_append_amd/build.py`` compiles every source under
``csrc/`` to an object in ``_build/`` and links ``libkvc.so`` next to this
file, plus ``libkvc_probe.so`` (streaming-read kernels the benchmark uses to
measure the practical HBM read ceiling; not part of the library's ABI).  All
HIP code is compiled with packed-fp32 instructions disabled (``-Xclang
-target-feature -Xclang -packed-fp32-ops``); the host pass warns that it does
not know that feature, which is harmless.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libkvc.so")
PROBE_LIB = os.path.join(HERE, "libkvc_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["status.cpp", "allocator.cpp", "scheduler.cpp", "api.hip", "noalloc.hip", "padded.hip",
           "cache_ops.hip", "decode.hip", "prefill.hip"]
PROBE_SOURCES = ["stream_probe.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-command-line-argument",
          f"-I{INCLUDE}", f"-I{CSRC}"]
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-munsafe-fp-atomics"]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    cmd = [HIPCC, *COMMON]
    if src.endswith(".hip"):
        cmd += ["-x", "hip", *HIP_FLAGS]
    cmd += ["-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{msgs}")
    if msgs and verbose:
        print(msgs, flush=True)
    return obj


def _link(objs, lib: str, verbose: bool):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile and link libkvc.so (and libkvc_probe.so); returns libkvc.so's path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES + PROBE_SOURCES))
    _link(objs[:len(SOURCES)], LIB, verbose)
    _link(objs[len(SOURCES):], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
