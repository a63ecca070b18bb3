"""Compile libkvq.so (HIP kernels for gfx950 + host code) in-tree with hipcc."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libkvq.so")
BUILD = os.path.join(PKG, "_build")
# the bounds-checked debug build (KVQ_DEBUG): same sources, own objects
OUT_DEBUG = os.path.join(PKG, "libkvq_debug.so")
BUILD_DEBUG = os.path.join(PKG, "_build_debug")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in ordinary VGPRs: their results feed VALU code
    # directly, without a v_accvgpr_read per value
    "-mllvm", "--amdgpu-mfma-vgpr-form",
    "-Wno-unused-command-line-argument",
]


# Per-file additions.  kvq_nsn.hip: its arg max runs over finite scores (sums
# of finite products), and without NaN semantics a maximum of four is one
# v_max3 and one v_max with no canonicalising moves in between.
FILE_FLAGS = {"kvq_nsn.hip": ["-fno-honor-nans"]}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src: str, debug: bool = False) -> str:
    obj = os.path.join(BUILD_DEBUG if debug else BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *(["-DKVQ_DEBUG"] if debug else []), *FILE_FLAGS.get(os.path.basename(src), []),
           "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose: bool = False, debug: bool = False) -> str:
    """libkvq.so, or with debug=True the bounds-checked libkvq_debug.so."""
    out = OUT_DEBUG if debug else OUT
    os.makedirs(BUILD_DEBUG if debug else BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda f: _compile(f, debug), srcs))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    build(verbose=True, debug=True)
    sys.exit(0)
