"""Build libdsa.so (gfx950) in-tree with hipcc.

Each HIP source is compiled to an object with the common flags plus its own,
then everything is linked into ``long_context_sparse_02_amd/libdsa.so``.
Packed-fp32 instructions are disabled for all device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdsa.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-fno-strict-aliasing",
          f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include")]
# Per-source extra flags.  The indexer's ReLU is a plain max: with NaNs honoured
# the compiler would canonicalise every matrix-core result first, doubling the
# vector-ALU work of its inner loop.  Indexer inputs are finite FP8 values.
# The warm-up loss kernel's matrix-core results are read by vector code right away: with
# them in VGPRs (not AGPRs) no copy per score is needed.
# The decode indexer reserves candidate slots with one atomic per group of pages and reads the
# reply only after its page loop; the atomic optimizer would rewrite that atomic into a form
# whose reply is read (and waited for, with every page in flight) right where it is issued.
EXTRA = {"indexer.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-atomic-optimizer-strategy=None"],
         "warmup.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
SOURCES = ["indexer.hip", "topk.hip", "attention.hip", "cache.hip", "train.hip", "warmup.hip",
           "dedup.hip", "noalloc.hip", "dsa_api.cpp"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libdsa)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, src + ".o")
    cmd = [_hipcc(), *COMMON, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libdsa.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
