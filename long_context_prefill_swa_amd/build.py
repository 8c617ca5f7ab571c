"""Build liborthros.so (HIP, gfx950) in-tree.

Usage: python -m long_context_prefill_swa_amd.build   (or python build.py)
Objects go to _build/ beside this file; the library to
long_context_prefill_swa_amd/liborthros.so. The benchmark's shader-clock
probe is built beside it as libclock_probe.so (not part of the library).
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "liborthros.so")
PROBE_LIB = os.path.join(HERE, "libclock_probe.so")
PROBE_SRC = "clock_probe.hip"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["kv_append.hip", "rowwise.hip", "splitkv_mfma.hip", "splitkv_plan.cpp",
           "noalloc_scratch.hip",
           "band_mfma.hip", "band_roll.hip", "band_persist.hip",
           "band_bwd.hip", "orthros_api.cpp", "gemm.cpp", "layer.cpp"]

# Packed fp32 instructions stay off: hipcc is asked not to form them.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    err = "\n".join(x for x in r.stderr.splitlines()
                    if "packed-fp32-ops" not in x)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip() and verbose:
        print(err, flush=True)
    return obj


def _link(objs, out, libs, verbose):
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs,
           "-L/opt/rocm/lib", *libs, "-Wl,-rpath,/opt/rocm/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + [PROBE_SRC]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    _link(objs[:-1], LIB, ["-lhipblaslt"], verbose)
    _link(objs[-1:], PROBE_LIB, [], verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
