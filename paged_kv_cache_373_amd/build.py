"""Builds libpagedkv.so (HIP kernels + C ABI) for gfx950 with hipcc.

``python -m paged_kv_cache_373_amd.build``.  Each source is compiled to an
object on its own (in parallel), then the objects are linked; the library
lands next to this file, where the Python binding loads it from.

A second, separate library, libpkv_probe.so, holds the benchmark's
read-bandwidth probe.  It is a measurement tool, not part of the attention
path, and the product library does not contain it.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpagedkv.so")
PROBE_LIB = os.path.join(HERE, "libpkv_probe.so")
SOURCES = ["decode.hip", "decode_wg.hip", "cascade.hip", "prefill.hip", "cache_ops.hip",
           "check.hip", "noalloc.hip", "api.cpp"]
PROBE_SOURCES = ["probe.hip"]
ARCH = os.environ.get("PKV_OFFLOAD_ARCH", "gfx950")

# Packed fp32 instructions are kept out of every kernel (-packed-fp32-ops);
# the host pass warns that it does not know the feature, which is harmless.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
_NOISE = "'-packed-fp32-ops' is not a recognized feature for this target"


def _run(cmd, verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if _NOISE not in ln]
    if msgs and (verbose or res.returncode != 0):
        print("\n".join(msgs), file=sys.stderr, flush=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}")


def _link(hipcc: str, objs, lib: str, verbose: bool) -> str:
    tmp = lib + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-fPIC", "-shared", "-o", tmp, *objs], verbose)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJ, exist_ok=True)
    jobs = []
    for s in SOURCES + PROBE_SOURCES:
        obj = os.path.join(OBJ, os.path.splitext(s)[0] + ".o")
        jobs.append((s, obj, [hipcc, *HIPCC_FLAGS, "-c", "-o", obj, os.path.join(CSRC, s)]))
    workers = min(len(jobs), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(lambda j: _run(j[2], verbose), jobs))
    objs = {s: o for s, o, _ in jobs}
    _link(hipcc, [objs[s] for s in SOURCES], LIB, verbose)
    _link(hipcc, [objs[s] for s in PROBE_SOURCES], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
