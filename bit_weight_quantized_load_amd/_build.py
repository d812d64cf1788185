"""Build of the HIP library libqwgemv.so (gfx950) from csrc/, in the package folder.

Each csrc/*.hip is compiled to an object file in parallel (the GEMV sources hold many
kernel instantiations), then the objects are linked into one shared library.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libqwgemv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fno-fast-math",
    "-ffp-contract=off",
    "-fno-gpu-flush-denormals-to-zero",
    # no packed fp32 arithmetic in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip into libqwgemv.so (always recompiles)."""
    tmpdir = tempfile.mkdtemp(prefix="qwbuild")
    try:
        def compile_one(src):
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            cmd = [HIPCC, *HIP_FLAGS, "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.check_call(cmd)
            return obj

        srcs = sources()
        workers = max(1, min(len(srcs), os.cpu_count() or 1, 16))
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            objs = list(ex.map(compile_one, srcs))
        tmp = LIB + ".tmp%d" % os.getpid()
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        os.replace(tmp, LIB)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
