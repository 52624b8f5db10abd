"""Build the HIP libraries for gfx950 in-tree.

    python -m hierarchical_speculative_attention_amd.build [--verbose]

libtfattn.so, the C-ABI library of the decode path, from every .hip file
under csrc/; libtfbench.so, a measurement aid the benchmark loads (a kernel
that only reads, for the HBM ceiling of the verification pass, and one that
only gathers the sparse pass's rows, for the ceiling of that call), from
bench_kernels/.  Each source is compiled to an object in parallel, then the
objects are linked.  Packed-fp32 instruction selection is disabled for the
device code (-Xclang -target-feature -Xclang -packed-fp32-ops); the host pass
warns that it does not know the feature, which is harmless.
"""

from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BENCH_SRC = os.path.join(PKG, "bench_kernels")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libtfattn.so")
BENCH_LIB = os.path.join(PKG, "libtfbench.so")
ARCH = "gfx950"
NOISE = "is not a recognized feature for this target"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libtfattn)")


def sources(src_dir=CSRC):
    return sorted(glob.glob(os.path.join(src_dir, "*.hip")))


def _flags(src_dir, extra):
    f = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall",
         "-Wno-unused-result", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", src_dir]
    return f + list(extra or [])


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if NOISE not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd[-3:])}\n{err}")
    if verbose and err.strip():
        print(err)


def build_one(src_dir: str, out: str, verbose: bool = False, extra=None) -> str:
    """Compile every .hip of src_dir (in parallel) and link them into out."""
    srcs = sources(src_dir)
    flags = _flags(src_dir, extra)
    with tempfile.TemporaryDirectory(prefix="tfbuild.") as tmp:
        objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in srcs]
        jobs = min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
        with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
            list(ex.map(lambda so: _run([hipcc()] + flags + ["-c", so[0], "-o", so[1]], verbose), zip(srcs, objs)))
        tmp_out = out + ".tmp"
        _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objs + ["-o", tmp_out], verbose)
        os.replace(tmp_out, out)
    return out


def build(verbose: bool = False, extra=None) -> str:
    """Compile libtfattn.so and libtfbench.so (always recompiles); returns
    the path of libtfattn.so."""
    build_one(CSRC, LIB, verbose, extra)
    build_one(BENCH_SRC, BENCH_LIB, verbose, extra)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
