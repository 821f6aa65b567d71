"""Build libfusedproj.so in-tree with hipcc for gfx950.

``python -m projection_gemm_sparse_amd.build`` compiles every HIP source of
the library into ``projection_gemm_sparse_amd/libfusedproj.so``.  The host
code (api.hip) and each kernel family (k_*.hip) are separate translation
units, compiled in parallel into ``_build/`` and linked into one shared
library.  Packed fp32 instructions are disabled (the kernels use scalar fp32
and v_dot2 only); no fast-math, no denormal flushing.

``build()`` recompiles every unit; ``build(incremental=True)`` (the
``--incremental`` flag) recompiles only units older than a source or header.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfusedproj.so")
OBJ_DIR = os.path.join(HERE, "_build")
SOURCES = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
HEADERS = sorted(glob.glob(os.path.join(CSRC, "*.hpp")) + glob.glob(os.path.join(CSRC, "*.h"))) + [
    os.path.join(ROOT, "include", "fusedproj.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # leading scalar kernel arguments arrive preloaded in SGPRs
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-I", os.path.join(ROOT, "include"),
]


def _filter(out: str) -> str:
    # hipcc's host pass does not know the packed-fp32 feature and says so;
    # that note is harmless, anything else is shown
    return "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)


def _compile(src: str, obj: str) -> tuple:
    tmp = obj + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-c", src, "-o", tmp]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode == 0:
        os.replace(tmp, obj)
    elif os.path.exists(tmp):
        os.remove(tmp)
    return res.returncode, " ".join(cmd), _filter(res.stdout)


def build(verbose: bool = False, incremental: bool = False, jobs: int = 0) -> str:
    """Compile the library (every unit, or only stale ones with
    ``incremental``) and link it."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    newest_header = max(os.path.getmtime(h) for h in HEADERS)
    todo = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(OBJ_DIR, os.path.basename(src)[:-4] + ".o")
        objs.append(obj)
        stale = (not incremental or not os.path.exists(obj) or
                 os.path.getmtime(obj) < max(newest_header, os.path.getmtime(src)))
        if stale:
            todo.append((src, obj))
    jobs = jobs or min(len(todo) or 1, max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda a: _compile(*a), todo))
    failed = [(cmd, out) for rc, cmd, out in results if rc != 0]
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n\n".join("%s\n%s" % f for f in failed))
    if verbose:
        for rc, cmd, out in results:
            print(cmd, flush=True)
            if out.strip():
                print(out)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", tmp]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("link failed (%d):\n%s" % (res.returncode, _filter(res.stdout)))
    if verbose:
        print(" ".join(cmd), flush=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, incremental="--incremental" in sys.argv))
