"""Build libsq.so in the package directory with hipcc for gfx950.

Usage: python -m compression_sq_compress_amd.build   (or call build()).
"""
from __future__ import annotations

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
            print("\n".join(lines), flush=True)


def build(verbose: bool = False, out: str = LIB) -> str:
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = []
    for src in ("calib.cpp", "api.cpp"):
        o = os.path.join(bdir, src + ".o")
        _run([shutil.which("g++") or "g++", *HOST_FLAGS, f"-I{ROCM}/include", "-c",
              os.path.join(CSRC, src), "-o", o], verbose)
        objs.append(o)
    o = os.path.join(bdir, "kernels.hip.o")
    _run([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, "kernels.hip"), "-o", o], verbose)
    objs.append(o)
    tmp = out + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp,
          "-lpthread"], verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
