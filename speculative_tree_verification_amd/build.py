"""Build libtree_ssd.so (HIP, gfx950) in-tree with hipcc.

    python -m speculative_tree_verification_amd.build [-v]

Every .hip file under csrc/ is compiled for gfx950 only and linked into
speculative_tree_verification_amd/libtree_ssd.so, whose exported symbols are
the extern "C" entry points declared in include/tree_ssd.h.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtree_ssd.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

# Packed fp32 VALU ops are disabled: hipcc would otherwise form v_pk_* fp32
# instructions from plain float code.
COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-variable", "-Wno-unused-function",
    "-I" + os.path.join(ROOT, "include"),
]


# Per-file additions: in verify_tiny.hip the first kernel arguments (up to 14
# dwords) are preloaded into scalar registers, so that its latency-bound
# one-wave work-groups issue their first loads without reading the kernel
# arguments first (the kernel orders its arguments for it). Measured against
# the same build without it, in one process: 3.82 -> 3.58 us per launch of the
# 15-node, 80-head layer; the commit kernel ran slower with it (69.3 -> 73.4 us
# for the 64-layer commit), so it is not preloaded.
FILE_FLAGS = {"verify_tiny.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=16"]}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
