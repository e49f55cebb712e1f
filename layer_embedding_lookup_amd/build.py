"""Builds libple.so (hand-written HIP kernels + C ABI) for gfx950 with hipcc, and
libple_bench.so (the benchmark's streaming-copy ceilings).

Usage: python -m layer_embedding_lookup_amd.build   (or call build()).
The library is built in-tree next to this file.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libple.so")
# the benchmark's streaming-copy ceilings (include/ple_bench.h), a library of their own
BENCH_LIB = os.path.join(HERE, "libple_bench.so")
BENCH_SOURCE = "ple_bench.hip"
SOURCES = ["ple_api.cpp", "ple_lookup.hip", "ple_kv_proj.hip", "ple_gate_conv.hip", "ple_dedup.hip", "ple_dp.hip",
           "ple_spec.hip", "ple_static.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libple)")


def common_flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            # packed fp32 instructions are kept out of every kernel (the compiler
            # still uses scalar fp32 ops); the host pass ignores the feature
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC]


def build(force: bool = True, verbose: bool = False, jobs: int = 4) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    deps = srcs + [os.path.join(CSRC, h) for h in os.listdir(CSRC) if h.endswith(".h")] + \
        [os.path.join(INCLUDE, "ple.h")]
    deps.append(os.path.join(CSRC, BENCH_SOURCE))
    if not force and all(os.path.exists(lb) and os.path.getmtime(lb) >= max(os.path.getmtime(d) for d in deps)
                         for lb in (LIB, BENCH_LIB)):
        return LIB
    cc = hipcc()
    objdir = os.path.join(ROOT, "_build", "libple")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src: str) -> str:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [cc, *common_flags(), "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, srcs))
    for lib, lib_objs in ((LIB, objs), (BENCH_LIB, [compile_one(os.path.join(CSRC, BENCH_SOURCE))])):
        tmp = lib + f".tmp{os.getpid()}"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *lib_objs]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc link failed:\n{res.stdout}\n{res.stderr}")
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(force=True, verbose="-v" in sys.argv))
