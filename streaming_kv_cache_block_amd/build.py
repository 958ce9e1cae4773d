"""Build the gfx950 HIP library (libllcache.so) and the host-only slot-math CLI.

    python -m streaming_kv_cache_block_amd.build

Compiles every HIP source with hipcc for gfx950 into objects under ``_build/`` and
links ``streaming_kv_cache_block_amd/libllcache.so``; also builds the seeded input
generator's device twin ``synth/libsynthfill.so`` (input preparation, not the product)
and ``libllceiling.so`` (the measured MFMA ceiling bench.py reports beside the roofline).  Packed-FP32 instruction
selection is switched off for device code.  ``slots_cli`` is built with g++ and
the host sanitizers (it has no device code).
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libllcache.so")
# debug library: the same kernels, the host side built with LL_DEBUG (NaN-poisoned slots,
# bounds checks of the slot arithmetic, a check that attention walks only written slots)
LIB_DEBUG = os.path.join(PKG, "libllcache_debug.so")
SLOTS_CLI = os.path.join(BUILD, "slots_cli")

HIP_SOURCES = ["attn.hip", "kvwrite.hip", "gemm.hip", "cache.cpp"]
ARCH = "gfx950"
# measured MFMA ceiling for the roofline (bench.py): a library of its own, not the product
CEILING_SRC = os.path.join(CSRC, "ceiling.hip")
CEILING_LIB = os.path.join(PKG, "libllceiling.so")
# seeded input generator's device twin (synth/): a library of its own, not the product
SYNTH_SRC = os.path.join(ROOT, "synth", "csrc", "fill.hip")
SYNTH_LIB = os.path.join(ROOT, "synth", "libsynthfill.so")


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    for cand in (os.path.join(rocm, "bin", "hipcc"), shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set ROCM_PATH)")


HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 target feature; that note is harmless
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    objs = []

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        out = _run([hipcc, "-x", "hip", *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and out.strip():
            print(out)
        return obj

    def synth_lib():
        tmp = SYNTH_LIB + ".tmp"
        _run([hipcc, "-x", "hip", *HIP_FLAGS, "-shared", SYNTH_SRC, "-o", tmp])
        os.replace(tmp, SYNTH_LIB)

    def ceiling_lib():
        tmp = CEILING_LIB + ".tmp"
        _run([hipcc, "-x", "hip", *HIP_FLAGS, "-shared", CEILING_SRC, "-o", tmp])
        os.replace(tmp, CEILING_LIB)

    def compile_debug_host():
        obj = os.path.join(BUILD, "cache_debug.o")
        _run([hipcc, "-x", "hip", *HIP_FLAGS, "-DLL_DEBUG", "-c", os.path.join(CSRC, "cache.cpp"), "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=min(6, len(HIP_SOURCES) + 2)) as ex:
        synth_job = ex.submit(synth_lib)
        ceiling_job = ex.submit(ceiling_lib)
        debug_job = ex.submit(compile_debug_host)
        objs = list(ex.map(compile_one, HIP_SOURCES))
        synth_job.result()
        ceiling_job.result()
        debug_obj = debug_job.result()
    for target, host in ((LIB, objs[-1]), (LIB_DEBUG, debug_obj)):
        tmp = target + ".tmp"
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs[:-1], host])
        os.replace(tmp, target)
    build_slots_cli()
    return LIB


def build_slots_cli() -> str:
    """Host-only build of the slot-math and split-plan driver (g++, address + UB
    sanitizers, LL_DEBUG bounds checks)."""
    os.makedirs(BUILD, exist_ok=True)
    _run(["g++", "-std=c++17", "-O1", "-g", "-DLL_DEBUG", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
          "-I", CSRC, os.path.join(CSRC, "slots_cli.cpp"), "-o", SLOTS_CLI])
    return SLOTS_CLI


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
