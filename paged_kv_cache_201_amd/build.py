"""Build libpkv.so for gfx950 in place (next to this file).

    python paged_kv_cache_201_amd/build.py [-v]

(run as a file: importing the package loads the library it builds)

Host-only C++ (the planner and page-table lowering) is compiled with g++;
the HIP sources with hipcc for gfx950.  Objects go to ``_build/`` at the
repository root; the shared library lands in this package directory, next
to libpkv_checked.so: the same objects with the entry points compiled with
PKV_CHECKED=1 (host-side checks of every step's index arrays before any
launch; see include/pkv.h).
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpkv.so")
CHECKED_LIB = os.path.join(PKG, "libpkv_checked.so")
CHECKED_SOURCE = "api.hip"  # the one source compiled again with PKV_CHECKED=1

HIP_SOURCES = ["api.hip", "reduce.hip", "prefix_mfma.hip", "cascade_fused.hip", "probe.hip", "paged_f32.hip",
               "paged_bf16.hip", "paged_fp8.hip"]
HOST_SOURCES = ["host.cpp"]

ARCH = "gfx950"
# Only the C ABI of include/pkv.h is exported (PKV_API); internal C++ symbols stay hidden.
COMMON = ["-std=c++17", "-fPIC", "-O3", "-fvisibility=hidden", "-DPKV_BUILDING_LIBRARY", f"-I{INCLUDE}",
          f"-I{CSRC}", "-Wall", "-Wno-unused-function"]
# Packed fp32 VALU instructions stay off on this target.
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-result"]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass of hipcc does not know the gfx950 feature flag; drop that line
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed: {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err)


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link libpkv.so and libpkv_checked.so; returns
    the path of libpkv.so."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    steps = []
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        steps.append(["g++", *COMMON, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        steps.append([hipcc, *COMMON, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    checked_obj = os.path.join(BUILD, CHECKED_SOURCE + ".checked.o")
    steps.append([hipcc, *COMMON, *HIP_FLAGS, "-DPKV_CHECKED=1", "-c", os.path.join(CSRC, CHECKED_SOURCE), "-o",
                  checked_obj])
    checked_objs = [checked_obj if o == os.path.join(BUILD, CHECKED_SOURCE + ".o") else o for o in objs]
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(steps)))) as ex:
        list(ex.map(lambda c: _run(c, verbose), steps))
    for lib, parts in ((LIB, objs), (CHECKED_LIB, checked_objs)):
        tmp = lib + ".tmp"
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *parts], verbose)
        os.replace(tmp, lib)
    return LIB


SANITIZE_EXE = os.path.join(BUILD, "host_sanitize")


def build_host_sanitize(verbose: bool = False) -> str:
    """The host half (host.cpp: lowering, validation, planners) linked into
    the seeded driver tests/host_sanitize.cpp with AddressSanitizer and
    UndefinedBehaviorSanitizer, as a CPU executable (g++ only, no device
    code); returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    _run(["g++", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-function",
          os.path.join(CSRC, "host.cpp"), os.path.join(ROOT, "tests", "host_sanitize.cpp"), "-o", SANITIZE_EXE],
         verbose)
    return SANITIZE_EXE


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_host_sanitize(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
