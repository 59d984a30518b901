"""Build libsq.so in the package directory with hipcc for gfx950.

Usage: python -m compression_sq_compress_amd.build   (or call build()).

The HIP sources (one file per kernel family) and the host C++ sources are
compiled in parallel; the SHA-256 of every source under csrc/ is compiled into
the library (sq_build_digest) so that a library built from other sources is
refused at load time instead of being run.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsq.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = os.environ.get("SQ_OFFLOAD_ARCH", "gfx950")

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-result"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result"]
HOST_SOURCES = ("calib.cpp", "api.cpp")


def hip_sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))


def source_digest() -> str:
    """SHA-256 (first 16 hex digits) over the names and contents of every file
    under csrc/ and of the public header, in sorted order."""
    from .digest import source_digest as _d
    return _d()


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        # hipcc's host pass warns about the gfx-only target feature; show the rest
        lines = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l]
        if lines:
            print("\n".join(lines[-20:]), flush=True)


def build(verbose: bool = False, out: str = LIB, jobs: int = 0) -> str:
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    digest = source_digest()
    steps = []
    for src in HOST_SOURCES:
        o = os.path.join(bdir, src + ".o")
        steps.append(([shutil.which("g++") or "g++", *HOST_FLAGS, f"-I{ROCM}/include",
                       f'-DSQ_SOURCE_DIGEST="{digest}"', "-c", os.path.join(CSRC, src), "-o", o], o))
    for src in hip_sources():
        o = os.path.join(bdir, src + ".o")
        steps.append(([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", o], o))
    n = jobs or min(len(steps), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(max_workers=n) as ex:
        futs = [ex.submit(_run, cmd, verbose) for cmd, _ in steps]
        for f in futs:
            f.result()
    tmp = out + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *[o for _, o in steps], "-o", tmp,
          "-lpthread"], verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
