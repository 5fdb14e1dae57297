"""The oracle's pin tests against an AddressSanitizer + UndefinedBehaviorSanitizer
build of ddt_oracle.c: out-of-bounds accesses, use of freed memory and
undefined behaviour (signed overflow, bad shifts, misaligned loads) abort the
run.  The pin tests run in a child process with the sanitizer runtimes loaded
ahead of the (uninstrumented) interpreter."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_TESTS = ["test_oracle_tree_build.py", "test_oracle_attention.py", "test_oracle_accept.py",
             "test_oracle_commit.py", "test_oracle_topk.py", "test_oracle_sampling.py",
             "test_oracle_loop.py"]


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_asan_ubsan():
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    oracle.build_sanitized()
    env = dict(os.environ)
    env["DDT_ORACLE_LIB"] = oracle.SAN_PATH
    env["LD_PRELOAD"] = " ".join(p for p in (asan, ubsan, os.environ.get("LD_PRELOAD", "")) if p)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "4"
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"]
    cmd += [os.path.join(ROOT, "tests", t) for t in PIN_TESTS]
    r = subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr, tail
