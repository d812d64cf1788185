"""Build of the HIP library libqwgemv.so (gfx950) from csrc/, in the package folder.

Each csrc/*.hip is compiled to an object file in parallel (the GEMV sources hold many
kernel instantiations), then the objects are linked into one shared library.
"""
from __future__ import annotations

import concurrent.futures
import glob
import hashlib
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


def _inputs_hash(src: str) -> str:
    """Hash of a source, every header it may include and the flags."""
    h = hashlib.sha256(" ".join(HIP_FLAGS).encode())
    deps = [src] + sorted(glob.glob(os.path.join(HERE, "csrc", "*.hpp"))) + \
        sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))
    for f in deps:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:20]


def build(verbose: bool = False, incremental: bool = False) -> str:
    """Compile every csrc/*.hip into libqwgemv.so.  By default every source is compiled
    again; with incremental=True an object whose source, headers and flags are unchanged
    is taken from the _build/ cache at the repository root."""
    tmpdir = tempfile.mkdtemp(prefix="qwbuild")
    cache = os.path.join(ROOT, "_build", "obj")
    if incremental:
        os.makedirs(cache, exist_ok=True)
    try:
        def compile_one(src):
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            cached = os.path.join(cache, "%s.%s.o" % (os.path.basename(src), _inputs_hash(src)))
            if incremental and os.path.exists(cached):
                return cached
            cmd = [HIPCC, *HIP_FLAGS, "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.check_call(cmd)
            if incremental:
                shutil.copyfile(obj, cached)
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
    import sys

    print(build(verbose=True, incremental="--incremental" in sys.argv))
