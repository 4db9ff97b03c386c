"""The C ABI's host side under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU).

A copy of libmxmoe.so is built with the host code instrumented
(-fsanitize=address,undefined on the host compilation only; the gfx950 code
is built as usual) and every ABI test (tests/test_abi.py: exports, capacity
and workspace arithmetic, every argument-rejection path of every entry point)
runs against it in a child process that preloads the sanitizer runtime.  Any
report is fatal.  These paths return before any HIP call, so no GPU is
needed."""

import glob
import os
import subprocess
import sys

import pytest

from combine_topk_ids_expert_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

DRIVER = """
import sys
import combine_topk_ids_expert_amd as mx
mx._LIB_PATH = sys.argv[1]
import pytest
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", "tests/test_abi.py"]))
"""


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def test_abi_checks_under_asan_and_ubsan(tmp_path):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("clang sanitizer runtime not installed")
    lib = build.build(out_path=str(tmp_path / "libmxmoe_san.so"),
                      extra_flags=["-O1", "-g", "-fno-omit-frame-pointer",
                                   "-Xarch_host", "-fsanitize=address,undefined",
                                   "-Xarch_host", "-fno-sanitize-recover=all", "-shared-libsan"])
    env = dict(os.environ, PYTHONPATH=ROOT, LD_PRELOAD=rt,
               LD_LIBRARY_PATH=os.path.dirname(rt) + ":" + os.environ.get("LD_LIBRARY_PATH", ""),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:alloc_dealloc_mismatch=0:"
                            "detect_odr_violation=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    proc = subprocess.run([sys.executable, "-c", DRIVER, lib], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=600)
    out = proc.stdout + proc.stderr
    assert proc.returncode == 0, out[-4000:]
    assert "Sanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
