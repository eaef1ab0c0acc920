"""Build libgdr.so (the HIP kernels + C ABI) in-tree for gfx950.

    python -m linear_attention_sequence_03_amd.build

Each source compiles to an object in parallel, then one shared library is
linked next to this file.  All device code is built with packed-fp32 ops
disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgdr.so")
SOURCES = ["gdr_api.cpp", "gdr_decode.hip", "gdr_chunk.hip", "gdr_fused.hip", "gdr_fg2.hip", "gdr_gdn2.hip",
           "gdr_gdn2_chunk.hip", "gdr_scratch.hip", "gdr_tree.hip"]
# plain device copy used only to calibrate hardware byte counters (bench.py --traffic)
CALIB_LIB = os.path.join(PKG, "libgdr_calib.so")
CALIB_SOURCES = ["gdr_calib.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags() -> list:
    return ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # keep MFMA accumulators in VGPRs: the kernels post-process every
            # accumulator with VALU ops, and AGPR copies cost more than they save
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            "-Wno-unused-command-line-argument"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + flags() + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH] + objs + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every source and link libgdr.so and libgdr_calib.so (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + CALIB_SOURCES
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in CALIB_SOURCES], CALIB_LIB)
    if verbose:
        print("built", LIB, "and", CALIB_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
