"""Build the HIP library ``libmqa_decode.so`` for gfx950, in-tree.

hipcc cross-compiles for gfx950 without a GPU.  Every HIP source is compiled
with packed-fp32 instructions disabled; objects go to ``_build/`` and the
shared object next to this file, where :mod:`.binding` loads it.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
BUILD = ROOT / "_build"
LIB = PKG / "libmqa_decode.so"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["abi.cpp", "plan.cpp", "decode_mfma.hip", "decode_valu.hip", "combine.hip", "probe.hip"]
COMMON = ["-x", "hip", "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
          "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # matrix-core accumulators in ordinary VGPRs: the online-softmax
          # rescale touches them with vector ALU ops, and AGPR accumulators
          # cost a copy in and out around every product
          "-mllvm", "-amdgpu-mfma-vgpr-form",
          "-I", str(ROOT / "include")]


def _compile(src: str) -> Path:
    obj = BUILD / (src + ".o")
    cmd = [HIPCC] + COMMON + ["-c", str(CSRC / src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed on %s" % src)
    return obj


def build(verbose: bool = False) -> Path:
    BUILD.mkdir(exist_ok=True)
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8")))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB.with_suffix(".so.tmp%d" % os.getpid())
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", str(tmp)] + [str(o) for o in objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link of libmqa_decode.so failed")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
