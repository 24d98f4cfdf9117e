"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

abi.cpp and plan.cpp (argument checks, planning, the workspace cache's host
logic) are rebuilt with both sanitizers on their host side
(gqa_decode_attention_mqa_amd.build.build_sanitized) and the host ABI tests run
against that build in a child process that preloads the ASan runtime.  Any
sanitizer report fails the child (UBSan is built non-recoverable).  No GPU is
used: those tests make no HIP call that reaches a device.
"""
import os
import subprocess
import sys
from pathlib import Path

import pytest

from gqa_decode_attention_mqa_amd import build

ROOT = Path(__file__).resolve().parent.parent


def test_host_abi_tests_pass_under_asan_and_ubsan():
    rt = build.asan_runtime()
    if not rt or not os.path.exists(rt):
        pytest.skip("no ASan runtime in this toolchain")
    lib = build.build_sanitized()
    env = dict(os.environ, LD_PRELOAD=rt, MQA_DECODE_LIB=str(lib),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        str(ROOT / "tests" / "test_host_abi.py")], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
    assert " passed" in tail
