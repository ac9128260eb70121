"""Build the HIP library ``libfi.so`` (gfx950) in-tree with hipcc.

Every ``csrc/*.hip`` is one translation unit (the host code and one per
kernel family with many compile-time variants); they compile in parallel to
objects under ``_build/`` and link into ``libfi.so``."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfi.so")

HIPCC = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every translation unit and link libfi.so (always recompiles)."""
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    tag = "%d" % os.getpid()

    def compile_one(src):
        obj = os.path.join(OBJ, os.path.basename(src)[:-4] + "." + tag + ".o")
        cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
        if verbose:
            print(" ".join(cmd))
        return obj

    jobs = jobs or min(len(srcs), max(1, os.cpu_count() or 1), 16)
    objs = [os.path.join(OBJ, os.path.basename(s)[:-4] + "." + tag + ".o") for s in srcs]
    tmp = LIB + ".tmp" + tag
    try:
        with ThreadPoolExecutor(jobs) as ex:
            list(ex.map(compile_one, srcs))
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
        res = subprocess.run(cmd, capture_output=True, text=True)
    finally:
        # this build's objects go, whether it succeeded or not
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    if verbose:
        print(" ".join(cmd))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
