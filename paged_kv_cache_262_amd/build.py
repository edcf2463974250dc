"""Build libpa.so in-tree: hand-written HIP kernels for gfx950 + the C ABI.

    python -m paged_kv_cache_262_amd.build

Each .hip source is compiled by hipcc for gfx950 only, and each .cpp source
(host-only code) by the host C++ compiler, in parallel; the objects are linked
into paged_kv_cache_262_amd/libpa.so.  Packed fp32 VALU
instructions are disabled for device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "libpa.so")
BUILD_DIR = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


HOST_CXX = os.environ.get("CXX_HOST", "g++")
HOST_FLAGS = ["-std=c++17", "-O2", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    if src.endswith(".cpp"):  # host-only code (the block manager)
        subprocess.run([HOST_CXX, *HOST_FLAGS, "-c", src, "-o", obj], check=True)
    else:
        subprocess.run([HIPCC, *CFLAGS, "-c", src, "-o", obj], check=True)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = OUT + ".tmp"
    subprocess.run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp],
                   check=True)
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build()
    sys.exit(0)
