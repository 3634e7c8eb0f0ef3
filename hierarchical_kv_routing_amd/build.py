"""Build libhga.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

Usage: python -m hierarchical_kv_routing_amd.build [-v]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libhga.so")
SOURCES = ["summarize.hip", "route.hip", "attend.hip", "decode.hip", "backward.hip", "api.cpp",
           "host_tier.cpp"]
PEAK_LIB = os.path.join(HERE, "libhga_peak.so")   # roofline microbenchmarks (bench.py)
PEAK_SOURCES = ["peak.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libhga.so")


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950: libhga.so (the path) and
    libhga_peak.so (the peak microbenchmarks bench.py measures against)."""
    _build_lib(PEAK_LIB, PEAK_SOURCES, verbose)
    return _build_lib(LIB, SOURCES, verbose)


def _flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Wall", "-Wno-unused-function",
            # packed f32 VALU forms stay off (hipcc forms them by itself otherwise)
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(HERE, "..", "include")]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def _build_lib(lib: str, sources, verbose: bool) -> str:
    """Compile each source to an object (in parallel), then link."""
    from concurrent.futures import ThreadPoolExecutor
    tmpdir = tempfile.mkdtemp(prefix="hga_build_")
    tmp = lib + f".tmp{os.getpid()}"
    try:
        objs = [os.path.join(tmpdir, s + ".o") for s in sources]
        jobs = [[hipcc()] + _flags() + ["-c", os.path.join(CSRC, s), "-o", o]
                for s, o in zip(sources, objs)]
        with ThreadPoolExecutor(max_workers=min(len(jobs), 8)) as ex:
            for f in [ex.submit(_run, j, verbose) for j in jobs]:
                f.result()
        _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
        os.replace(tmp, lib)
    finally:
        if os.path.exists(tmp):
            os.remove(tmp)
        shutil.rmtree(tmpdir, ignore_errors=True)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
