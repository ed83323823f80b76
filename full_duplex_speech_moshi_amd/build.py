"""Build libpp.so (HIP kernels for gfx950 + the C-ABI engine) in-tree.

    python -m full_duplex_speech_moshi_amd.build

hipcc cross-compiles for gfx950 without a GPU present.  Every HIP source is
compiled with packed-fp32 instruction generation disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libpp.so")
ARCH = "gfx950"

HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include")]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include")]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")
    # the host pass does not know the GPU target feature: that warning is harmless
    noise = "is not a recognized feature for this target"
    rest = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if verbose and rest.strip():
        print(rest)


def build(verbose: bool = True) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    with tempfile.TemporaryDirectory() as tmp:
        units = (("kernels.hip", HIP_FLAGS), ("dep_loop.hip", HIP_FLAGS), ("codec.hip", HIP_FLAGS),
                 ("engine.cpp", HOST_FLAGS), ("codec.cpp", HOST_FLAGS))
        objs = [os.path.join(tmp, src + ".o") for src, _ in units]
        # the compilations are independent: run them side by side
        with ThreadPoolExecutor(len(units)) as ex:
            for f in [ex.submit(_run, [hipcc, *flags, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
                      for (src, flags), obj in zip(units, objs)]:
                f.result()
        tmp_lib = LIB + ".tmp"
        _run([hipcc, "-shared", f"--offload-arch={ARCH}", *objs, "-o", tmp_lib], verbose)
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
