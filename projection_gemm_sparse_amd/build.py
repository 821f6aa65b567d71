"""Build libfusedproj.so in-tree with hipcc for gfx950.

``python -m projection_gemm_sparse_amd.build`` compiles every HIP source of
the library into ``projection_gemm_sparse_amd/libfusedproj.so``.  Packed
fp32 instructions are disabled (the kernels use scalar fp32 and v_dot2 only);
no fast-math, no denormal flushing.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfusedproj.so")
SOURCES = [os.path.join(CSRC, "api.hip")]
HEADERS = [os.path.join(CSRC, f) for f in ("common.hpp", "skinny.hpp", "smfma.hpp", "tile.hpp",
                                           "tile_ring.hpp", "epilogue.hpp", "mxfp8.hpp",
                                           "stream.hpp")] + [
    os.path.join(ROOT, "include", "fusedproj.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # leading scalar kernel arguments arrive preloaded in SGPRs
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False) -> str:
    """Compile the library (always; the caller decides whether to rebuild)."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so;
    # that note is harmless, anything else is shown
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed (%d):\n%s" % (res.returncode, out))
    if out.strip() and verbose:
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
