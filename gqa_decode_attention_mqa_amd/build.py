"""Build the HIP library ``libmqa_decode.so`` for gfx950, in-tree.

hipcc cross-compiles for gfx950 without a GPU.  Every HIP source is compiled
with packed-fp32 instructions disabled; objects go to ``_build/`` and the
shared object next to this file, where :mod:`.binding` loads it.
``python -m gqa_decode_attention_mqa_amd.build --sanitize`` builds the host
sanitizer variant (see build_sanitized).
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

SOURCES = ["abi.cpp", "plan.cpp", "decode_mfma.hip", "decode_valu.hip", "combine.hip", "probe.hip", "prefill_mfma.hip"]
COMMON = ["-x", "hip", "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
          "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # matrix-core accumulators in ordinary VGPRs: the online-softmax
          # rescale touches them with vector ALU ops, and AGPR accumulators
          # cost a copy in and out around every product
          "-mllvm", "-amdgpu-mfma-vgpr-form",
          "-I", str(ROOT / "include")]


def _flags(src: str) -> list:
    return COMMON


def _compile(src: str) -> Path:
    obj = BUILD / (src + ".o")
    cmd = [HIPCC] + _flags(src) + ["-c", str(CSRC / src), "-o", str(obj)]
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


# Host-only sanitizer build: abi.cpp and plan.cpp (the argument checks,
# planner and workspace cache) are recompiled with AddressSanitizer and
# UndefinedBehaviorSanitizer on their host side only; the device objects are
# the regular ones.  The result, _build/libmqa_decode_asan.so, is loaded by a
# process that preloads the ASan runtime (asan_runtime()); the CPU test
# tests/test_host_sanitized.py runs the host ABI tests that way.
HOST_SOURCES = ["abi.cpp", "plan.cpp"]
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-g"]
ASAN_LIB = BUILD / "libmqa_decode_asan.so"


def asan_runtime() -> str:
    """Path of the shared ASan runtime of the HIP toolchain's clang."""
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "lib", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return r.stdout.strip()


def build_sanitized(verbose: bool = False) -> Path:
    BUILD.mkdir(exist_ok=True)
    objs = []
    for src in SOURCES:
        if src in HOST_SOURCES:
            obj = BUILD / (src + ".asan.o")
            cmd = [HIPCC] + _flags(src) + SAN_FLAGS + ["-c", str(CSRC / src), "-o", str(obj)]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                sys.stderr.write(r.stdout + r.stderr)
                raise RuntimeError("hipcc (sanitized host) failed on %s" % src)
        else:
            obj = BUILD / (src + ".o")
            if not obj.exists() or obj.stat().st_mtime < (CSRC / src).stat().st_mtime:
                obj = _compile(src)
        objs.append(obj)
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", str(ASAN_LIB)] + [str(o) for o in objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link of libmqa_decode_asan.so failed")
    if verbose:
        print("built", ASAN_LIB)
    return ASAN_LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        build_sanitized(verbose=True)
    else:
        build(verbose=True)
