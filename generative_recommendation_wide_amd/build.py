"""Build the HIP library libgrw.so in-tree for gfx950.

    python generative_recommendation_wide_amd/build.py

(run it by path: importing the package loads the library this script builds)

Every source is compiled with hipcc for gfx950 only, with packed-FP32 instruction
selection disabled, then linked into one shared library next to this file.  The benchmark's
MFMA ceiling probe (csrc/ceiling.hip) goes into a library of its own, libgrw_ceiling.so, so
that the decode library holds the decode path only.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgrw.so")
SOURCES = ["api.hip", "attn_shared.hip", "attn_unshared.hip", "select.hip", "selftest.hip"]
CEILING_LIB = os.path.join(HERE, "libgrw_ceiling.so")
CEILING_SOURCES = ["ceiling.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Wno-unused-function", "-Wno-unused-variable",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(HERE, "..", "include")]


# per-file extra flags: the attention kernels never see NaN (finite bf16 / fp8 / fp32 inputs),
# so max operations need no NaN quieting; infinities (used for masking) keep IEEE semantics
EXTRA = {"attn_shared.hip": ["-fno-honor-nans"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *flags(), *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is harmless
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(lib: str, objs) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + CEILING_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link(LIB, [objs[s] for s in SOURCES])
    _link(CEILING_LIB, [objs[s] for s in CEILING_SOURCES])
    if verbose:
        print("built", LIB, "and", CEILING_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
