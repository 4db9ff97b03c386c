"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

A copy of oracle/oracle.c is built with -fsanitize=address,undefined (any
report is fatal) and every pin runs against it in a child process that
preloads the sanitizer runtimes.  An out-of-bounds access, a use after free
or undefined integer behaviour anywhere the pins reach fails the test."""

import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    try:
        p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                           timeout=60).stdout.strip()
    except (OSError, subprocess.SubprocessError):
        return None
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_pins_pass_under_asan_and_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    lib = oracle.build(out_path=str(tmp_path / "liboracle_san.so"),
                       extra_flags=["-O1", "-g", "-fno-omit-frame-pointer",
                                    "-fsanitize=address,undefined",
                                    "-fno-sanitize-recover=all"])
    env = dict(os.environ, PYTHONPATH=ROOT, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    proc = subprocess.run([sys.executable, "-c",
                           f"import tests.oracle_pins as p; p.run_all({lib!r})"],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert proc.returncode == 0, proc.stderr[-3000:]
    assert "Sanitizer" not in proc.stderr, proc.stderr[-3000:]
