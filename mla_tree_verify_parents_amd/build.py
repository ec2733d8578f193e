"""Build libddt.so (the HIP library behind include/ddt.h) for gfx950, in-tree.

    python -m mla_tree_verify_parents_amd.build

compiles every csrc/*.hip file with hipcc into one object each, in parallel,
and links them into mla_tree_verify_parents_amd/libddt.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import ctypes
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libddt.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops are kept out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs unless a kernel pins an accumulator to AGPRs
    # itself: the attention scores are read by VALU code right away
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", INCLUDE, "-I", CSRC,
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(extra=(), jobs: int = 8) -> str:
    """Compile and link libddt.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra)), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    # a library with unresolved symbols (e.g. a kernel whose host launch stub
    # the compiler dropped) links fine but cannot be loaded: refuse it here
    try:
        ctypes.CDLL(tmp)
    except OSError as e:
        os.remove(tmp)
        raise RuntimeError(f"built library does not load: {e}") from None
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    extra = sys.argv[1:]
    print(build(extra))
